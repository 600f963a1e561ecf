// C ABI of libkvp: argument validation, status codes and kernel launches.
// Declarations and the contract of every entry point are in include/kvp.h.
#include "kvp.h"

#include <cmath>
#include <cstdint>

#include "kvp_launch.h"

namespace {

constexpr int32_t kAbiVersion = 8;
// Limits that keep every index the kernels form in 32-bit ints, and the bytes
// of one head (S * d * 4 at most) within a 32-bit buffer range.
constexpr int64_t kMaxSeq = int64_t(1) << 22;
constexpr int64_t kMaxBlocks = (int64_t(1) << 31) - 1;
// Element-wise kernels index with 64-bit flat indices but launch 256-thread
// blocks in a 32-bit grid.
constexpr int64_t kMaxElems = kMaxBlocks * 256;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shared validation of the dims.  Returns KVP_OK and fills `sh`, or an error.
kvp_status_t check_dims(const kvp_dims_t& d, bool need_heads_ratio, kvp::Shape& sh) {
  if (d.batch < 0 || d.seq_len < 0 || d.n_q_heads < 1 || d.n_kv_heads < 1) return KVP_EINVAL;
  if (need_heads_ratio && d.n_q_heads % d.n_kv_heads != 0) return KVP_EINVAL;
  if (d.head_dim != 64 && d.head_dim != 128) return KVP_EUNSUPPORTED;
  if (d.seq_len > kMaxSeq) return KVP_EUNSUPPORTED;
  const int64_t units = int64_t(d.batch) * d.n_kv_heads;
  if (units * ((int64_t(d.seq_len) + 63) / 64) * (d.n_q_heads / d.n_kv_heads) > kMaxBlocks)
    return KVP_EUNSUPPORTED;
  sh.B = d.batch;
  sh.Hq = d.n_q_heads;
  sh.Hkv = d.n_kv_heads;
  sh.S = d.seq_len;
  sh.D = d.head_dim;
  sh.G = d.n_q_heads / d.n_kv_heads;
  return KVP_OK;
}

bool valid_dtype(kvp_dtype_t t) { return t == KVP_BF16 || t == KVP_F32; }

float resolve_scale(float scale, int head_dim) {
  return scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(head_dim));
}

kvp_status_t from_hip(hipError_t e) { return e == hipSuccess ? KVP_OK : KVP_EHIP; }

}  // namespace

extern "C" {

int32_t kvp_abi_version(void) { return kAbiVersion; }

const char* kvp_status_string(kvp_status_t s) {
  switch (s) {
    case KVP_OK: return "ok";
    case KVP_EINVAL: return "invalid argument";
    case KVP_EUNSUPPORTED: return "unsupported configuration";
    case KVP_EWORKSPACE: return "workspace too small";
    case KVP_EHIP: return "HIP launch error";
  }
  return "unknown status";
}

int64_t kvp_keep_count(int64_t S, int64_t w, int64_t s, int64_t k) {
  if (S < 0 || w < 0 || s < 0 || k < 0) return -1;
  const int64_t sinks = s < S ? s : S;
  const int64_t win_lo = (S - w > s) ? S - w : s;  // window part not already a sink
  const int64_t window = S > win_lo ? S - win_lo : 0;
  const int64_t elig = S - w - s > 0 ? S - w - s : 0;
  return sinks + window + (k < elig ? k : elig);
}

kvp_status_t kvp_lse_fwd(const void* q, const void* k, kvp_dtype_t dtype, kvp_dims_t dims,
                         float scale, float* lse, hipStream_t stream) {
  kvp::Shape sh;
  const kvp_status_t st = check_dims(dims, true, sh);
  if (st != KVP_OK) return st;
  if (!valid_dtype(dtype)) return KVP_EUNSUPPORTED;
  if (std::isnan(scale) || std::isinf(scale)) return KVP_EINVAL;
  if (sh.B == 0 || sh.S == 0) return KVP_OK;
  if (!q || !k || !lse || !aligned(q, 16) || !aligned(k, 16) || !aligned(lse, 4))
    return KVP_EINVAL;
  return from_hip(kvp::launch_lse(q, k, dtype == KVP_BF16 ? 0 : 1, sh,
                                  resolve_scale(scale, sh.D), lse, stream));
}

kvp_status_t kvp_lse_sparse(const void* q, const void* k, kvp_dtype_t dtype, kvp_dims_t dims,
                            float scale, const int32_t* rank, const int32_t* cutoff, int32_t window,
                            float* lse, hipStream_t stream) {
  kvp::Shape sh;
  const kvp_status_t st = check_dims(dims, true, sh);
  if (st != KVP_OK) return st;
  if (!valid_dtype(dtype)) return KVP_EUNSUPPORTED;
  if (std::isnan(scale) || std::isinf(scale) || window < 0) return KVP_EINVAL;
  if (sh.B == 0 || sh.S == 0) return KVP_OK;
  if (!q || !k || !lse || !rank || !cutoff || !aligned(q, 16) || !aligned(k, 16) ||
      !aligned(lse, 4) || !aligned(rank, 4) || !aligned(cutoff, 4))
    return KVP_EINVAL;
  const int w = window > sh.S ? sh.S : window;
  return from_hip(kvp::launch_lse_sparse(q, k, dtype == KVP_BF16 ? 0 : 1, sh,
                                         resolve_scale(scale, sh.D), rank, cutoff, w, lse, stream));
}

kvp_status_t kvp_future_mass(const void* q, const void* k, const float* lse, kvp_dtype_t dtype,
                             kvp_dims_t dims, float scale, int32_t window, float* mass,
                             hipStream_t stream) {
  kvp::Shape sh;
  const kvp_status_t st = check_dims(dims, true, sh);
  if (st != KVP_OK) return st;
  if (!valid_dtype(dtype)) return KVP_EUNSUPPORTED;
  if (std::isnan(scale) || std::isinf(scale) || window < 0) return KVP_EINVAL;
  if (sh.B == 0 || sh.S == 0) return KVP_OK;
  if (!q || !k || !lse || !mass || !aligned(q, 16) || !aligned(k, 16) || !aligned(lse, 4) ||
      !aligned(mass, 4))
    return KVP_EINVAL;
  // A window beyond the sequence leaves no future query for any key.
  const int w = window > sh.S ? sh.S : window;
  return from_hip(kvp::launch_mass(q, k, lse, dtype == KVP_BF16 ? 0 : 1, sh,
                                   resolve_scale(scale, sh.D), w, 0, mass, stream));
}

kvp_status_t kvp_future_mass_per_head(const void* q, const void* k, const float* lse,
                                      kvp_dtype_t dtype, kvp_dims_t dims, float scale,
                                      int32_t window, float* mass, hipStream_t stream) {
  kvp::Shape sh;
  const kvp_status_t st = check_dims(dims, true, sh);
  if (st != KVP_OK) return st;
  if (!valid_dtype(dtype)) return KVP_EUNSUPPORTED;
  if (std::isnan(scale) || std::isinf(scale) || window < 0) return KVP_EINVAL;
  if (sh.B == 0 || sh.S == 0) return KVP_OK;
  if (!q || !k || !lse || !mass || !aligned(q, 16) || !aligned(k, 16) || !aligned(lse, 4) ||
      !aligned(mass, 4))
    return KVP_EINVAL;
  const int w = window > sh.S ? sh.S : window;
  return from_hip(kvp::launch_mass(q, k, lse, dtype == KVP_BF16 ? 0 : 1, sh,
                                   resolve_scale(scale, sh.D), w, 1, mass, stream));
}

size_t kvp_future_mass_workspace_bytes(kvp_dims_t dims, kvp_dtype_t dtype, int32_t window,
                                       int32_t per_head) {
  kvp::Shape sh;
  if (check_dims(dims, true, sh) != KVP_OK || !valid_dtype(dtype) || window < 0) return 0;
  if (per_head != 0 && per_head != 1) return 0;
  if (sh.B == 0 || sh.S == 0) return 0;
  const int w = window > sh.S ? sh.S : window;
  return kvp::mass_workspace_bytes(dtype == KVP_BF16 ? 0 : 1, sh, w, per_head);
}

kvp_status_t kvp_future_mass_chunked(const void* q, const void* k, const float* lse,
                                     kvp_dtype_t dtype, kvp_dims_t dims, float scale,
                                     int32_t window, int32_t per_head, float* mass, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  kvp::Shape sh;
  const kvp_status_t st = check_dims(dims, true, sh);
  if (st != KVP_OK) return st;
  if (!valid_dtype(dtype)) return KVP_EUNSUPPORTED;
  if (std::isnan(scale) || std::isinf(scale) || window < 0) return KVP_EINVAL;
  if (per_head != 0 && per_head != 1) return KVP_EINVAL;
  if (sh.B == 0 || sh.S == 0) return KVP_OK;
  if (!q || !k || !lse || !mass || !aligned(q, 16) || !aligned(k, 16) || !aligned(lse, 4) ||
      !aligned(mass, 4))
    return KVP_EINVAL;
  const int w = window > sh.S ? sh.S : window;
  const int dt = dtype == KVP_BF16 ? 0 : 1;
  const size_t need = kvp::mass_workspace_bytes(dt, sh, w, per_head);
  if (workspace_bytes < need) return KVP_EWORKSPACE;
  if (need > 0 && (!workspace || !aligned(workspace, 256))) return KVP_EINVAL;
  return from_hip(kvp::launch_mass_ws(q, k, lse, dt, sh, resolve_scale(scale, sh.D), w, per_head,
                                      mass, need > 0 ? workspace : nullptr, stream));
}

kvp_status_t kvp_target_scores(const float* mass, int32_t per_head, kvp_dims_t dims, int32_t window,
                               int32_t normalize, kvp_agg_t agg, float eps, int32_t query,
                               int32_t decay_step, const float* log_gamma, float* score,
                               hipStream_t stream) {
  if (dims.batch < 0 || dims.seq_len < 0 || dims.n_q_heads < 1 || dims.n_kv_heads < 1 ||
      dims.n_q_heads % dims.n_kv_heads != 0)
    return KVP_EINVAL;
  if (dims.seq_len > kMaxSeq) return KVP_EUNSUPPORTED;
  if (window < 0 || (per_head != 0 && per_head != 1) || (normalize != 0 && normalize != 1))
    return KVP_EINVAL;
  if (agg != KVP_AGG_LOG_MEAN && agg != KVP_AGG_MEAN_LOG && agg != KVP_AGG_MAX_LOG)
    return KVP_EINVAL;
  if (!per_head && agg != KVP_AGG_LOG_MEAN) return KVP_EINVAL;  // needs per-head masses
  if (!(eps >= 0.f) || std::isinf(eps)) return KVP_EINVAL;
  if (query >= 0 && decay_step < 1) return KVP_EINVAL;
  if ((int64_t)dims.batch * dims.n_q_heads * dims.seq_len > kMaxElems) return KVP_EUNSUPPORTED;
  if (dims.batch == 0 || dims.seq_len == 0) return KVP_OK;
  if (!mass || !score || !aligned(mass, 4) || !aligned(score, 4)) return KVP_EINVAL;
  if (query >= 0 && (!log_gamma || !aligned(log_gamma, 4))) return KVP_EINVAL;
  kvp::Shape sh;
  sh.B = dims.batch;
  sh.Hq = dims.n_q_heads;
  sh.Hkv = dims.n_kv_heads;
  sh.S = dims.seq_len;
  sh.D = dims.head_dim;
  sh.G = dims.n_q_heads / dims.n_kv_heads;
  const int w = window > sh.S ? sh.S : window;
  return from_hip(kvp::launch_target(mass, per_head, sh, w, normalize, (int)agg, eps, query,
                                     query >= 0 ? decay_step : 1, log_gamma, score, stream));
}

kvp_status_t kvp_static_priority(const float* score, kvp_dims_t dims, int32_t decay_step,
                                 const float* log_gamma, float* priority, hipStream_t stream) {
  if (dims.batch < 0 || dims.seq_len < 0 || dims.n_kv_heads < 1 || decay_step < 1)
    return KVP_EINVAL;
  if (dims.seq_len > kMaxSeq) return KVP_EUNSUPPORTED;
  if ((int64_t)dims.batch * dims.n_kv_heads * dims.seq_len > kMaxElems) return KVP_EUNSUPPORTED;
  if (dims.batch == 0 || dims.seq_len == 0) return KVP_OK;
  if (!score || !log_gamma || !priority || !aligned(score, 4) || !aligned(log_gamma, 4) ||
      !aligned(priority, 4))
    return KVP_EINVAL;
  kvp::Shape sh;
  sh.B = dims.batch;
  sh.Hq = dims.n_kv_heads;
  sh.Hkv = dims.n_kv_heads;
  sh.S = dims.seq_len;
  sh.D = dims.head_dim;
  sh.G = 1;
  return from_hip(kvp::launch_priority(score, sh, decay_step, log_gamma, priority, stream));
}

size_t kvp_select_workspace_bytes(kvp_dims_t dims, int32_t top_k) {
  if (dims.batch < 0 || dims.seq_len < 0 || dims.n_kv_heads < 1 || top_k < 0) return 0;
  if (dims.seq_len > kMaxSeq) return 0;
  return kvp::select_workspace_bytes(int64_t(dims.batch) * dims.n_kv_heads, dims.seq_len);
}

kvp_status_t kvp_select_topk(const float* mass, kvp_dims_t dims, int32_t window, int32_t n_sink,
                             int32_t top_k, int32_t* keep, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  if (dims.batch < 0 || dims.seq_len < 0 || dims.n_kv_heads < 1) return KVP_EINVAL;
  if (window < 0 || n_sink < 0 || top_k < 0) return KVP_EINVAL;
  if (dims.seq_len > kMaxSeq) return KVP_EUNSUPPORTED;
  const int64_t rows = int64_t(dims.batch) * dims.n_kv_heads;
  if (rows > kMaxBlocks || kvp::select_split_blocks(rows, dims.seq_len) > kMaxBlocks)
    return KVP_EUNSUPPORTED;
  const int64_t n_keep = kvp_keep_count(dims.seq_len, window, n_sink, top_k);
  if (rows == 0 || dims.seq_len == 0) return KVP_OK;
  if (!mass || !keep || !aligned(mass, 4) || !aligned(keep, 4)) return KVP_EINVAL;
  const size_t need = kvp::select_workspace_bytes(rows, dims.seq_len);
  if (workspace_bytes < need) return KVP_EWORKSPACE;
  if (need > 0 && (!workspace || !aligned(workspace, 256))) return KVP_EINVAL;
  const int S = dims.seq_len;
  const int w = window > S ? S : window;
  const int s = n_sink > S ? S : n_sink;
  return from_hip(kvp::launch_select(mass, rows, S, w, s, top_k, n_keep, keep, workspace, stream));
}

kvp_status_t kvp_select_topk_noalloc(const float* mass, kvp_dims_t dims, int32_t window,
                                     int32_t n_sink, int32_t top_k, int32_t* keep,
                                     hipStream_t stream) {
  if (dims.batch < 0 || dims.seq_len < 0 || dims.n_kv_heads < 1) return KVP_EINVAL;
  if (window < 0 || n_sink < 0 || top_k < 0) return KVP_EINVAL;
  if (dims.seq_len > kMaxSeq) return KVP_EUNSUPPORTED;
  const int64_t rows = int64_t(dims.batch) * dims.n_kv_heads;
  if (rows > kMaxBlocks || kvp::select_split_blocks(rows, dims.seq_len) > kMaxBlocks)
    return KVP_EUNSUPPORTED;
  const int64_t n_keep = kvp_keep_count(dims.seq_len, window, n_sink, top_k);
  if (rows == 0 || dims.seq_len == 0) return KVP_OK;
  if (!mass || !keep || !aligned(mass, 4) || !aligned(keep, 4)) return KVP_EINVAL;
  const size_t need = kvp::select_workspace_bytes(rows, dims.seq_len);
  static_assert(kvp::kSelectScratchBytes == KVP_SELECT_NOALLOC_MAX_WORKSPACE,
                "the header states the size of the library's own workspace");
  if (need > kvp::kSelectScratchBytes) return KVP_EWORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = kvp::select_scratch(&ws);
    if (e != hipSuccess) return KVP_EHIP;
  }
  const int S = dims.seq_len;
  const int w = window > S ? S : window;
  const int s = n_sink > S ? S : n_sink;
  return from_hip(kvp::launch_select(mass, rows, S, w, s, top_k, n_keep, keep, ws, stream));
}

int64_t kvp_block_count(int64_t seq_len, int64_t block_start, int64_t block_len) {
  if (seq_len < 0 || block_start < 0 || block_len < 1) return -1;
  return seq_len > block_start ? (seq_len - block_start + block_len - 1) / block_len : 0;
}

kvp_status_t kvp_block_future_scores(const void* q, const void* k, const float* lse,
                                     kvp_dtype_t dtype, kvp_dims_t dims, float scale,
                                     int32_t window, int32_t per_head, int32_t block_start,
                                     int32_t block_len, float* block_scores, float* future_scores,
                                     hipStream_t stream) {
  kvp::Shape sh;
  const kvp_status_t st = check_dims(dims, true, sh);
  if (st != KVP_OK) return st;
  if (!valid_dtype(dtype)) return KVP_EUNSUPPORTED;
  if (std::isnan(scale) || std::isinf(scale) || window < 0) return KVP_EINVAL;
  if ((per_head != 0 && per_head != 1) || block_start < 0 || block_len < 1) return KVP_EINVAL;
  if (block_start % 32 != 0 || block_len % 32 != 0) return KVP_EUNSUPPORTED;
  const int64_t n_blocks = kvp_block_count(sh.S, block_start, block_len);
  if (sh.B == 0 || n_blocks == 0) return KVP_OK;
  if (!q || !k || !lse || !future_scores || !aligned(q, 16) || !aligned(k, 16) ||
      !aligned(lse, 4) || !aligned(future_scores, 4) || (block_scores && !aligned(block_scores, 4)))
    return KVP_EINVAL;
  const int w = window > sh.S ? sh.S : window;
  const kvp::SegOut seg{block_start, block_len, static_cast<int>(n_blocks), block_scores,
                        future_scores};
  return from_hip(kvp::launch_block_scores(q, k, lse, dtype == KVP_BF16 ? 0 : 1, sh,
                                           resolve_scale(scale, sh.D), w, per_head, seg, stream));
}

kvp_status_t kvp_soft_topk_fwd(const float* x, int64_t rows, int32_t n, const float* k, float tau,
                               float* y, float* lam, hipStream_t stream) {
  if (rows < 0 || n < 0 || !(tau > 0.f) || std::isinf(tau)) return KVP_EINVAL;
  if (rows > kMaxBlocks || n > (1 << 30)) return KVP_EUNSUPPORTED;
  if (rows == 0 || n == 0) return KVP_OK;
  if (!x || !k || !y || !aligned(x, 4) || !aligned(k, 4) || !aligned(y, 4) ||
      (lam && !aligned(lam, 4)))
    return KVP_EINVAL;
  return from_hip(kvp::launch_soft_topk_fwd(x, k, rows, n, tau, y, lam, stream));
}

kvp_status_t kvp_soft_topk_bwd(const float* x, const float* lam, const float* dy, int64_t rows,
                               int32_t n, float tau, float* dx, float* dk, hipStream_t stream) {
  if (rows < 0 || n < 0 || !(tau > 0.f) || std::isinf(tau)) return KVP_EINVAL;
  if (rows > kMaxBlocks || n > (1 << 30)) return KVP_EUNSUPPORTED;
  if (rows == 0 || n == 0) return KVP_OK;
  if (!x || !lam || !dy || !dx || !aligned(x, 4) || !aligned(lam, 4) || !aligned(dy, 4) ||
      !aligned(dx, 4) || (dk && !aligned(dk, 4)))
    return KVP_EINVAL;
  return from_hip(kvp::launch_soft_topk_bwd(x, lam, dy, rows, n, tau, dx, dk, stream));
}

size_t kvp_running_cutoff_workspace_bytes(kvp_dims_t dims, int32_t n_sink) {
  if (dims.batch < 0 || dims.seq_len < 0 || dims.n_kv_heads < 1 || n_sink < 0) return 0;
  const int64_t rows = int64_t(dims.batch) * dims.n_kv_heads;
  const int S = dims.seq_len;
  return kvp::cutoff_workspace_bytes(rows, S, n_sink > S ? S : n_sink);
}

kvp_status_t kvp_running_cutoff(const float* score, kvp_dims_t dims, int32_t window, int32_t n_sink,
                                int32_t top_k, int32_t* rank, int32_t* cutoff, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (dims.batch < 0 || dims.seq_len < 0 || dims.n_kv_heads < 1) return KVP_EINVAL;
  if (window < 0 || n_sink < 0 || top_k < 0) return KVP_EINVAL;
  if (dims.seq_len > kMaxSeq) return KVP_EUNSUPPORTED;
  const int64_t rows = int64_t(dims.batch) * dims.n_kv_heads;
  if (rows > kMaxBlocks) return KVP_EUNSUPPORTED;
  if (rows == 0 || dims.seq_len == 0) return KVP_OK;
  if (!score || !rank || !cutoff || !aligned(score, 4) || !aligned(rank, 4) ||
      !aligned(cutoff, 4))
    return KVP_EINVAL;
  const int S = dims.seq_len;
  // one wave per (row, 1024 queries), four waves per workgroup
  if (rows * ((S + 1023) / 1024) > 4 * kMaxBlocks) return KVP_EUNSUPPORTED;
  const int w = window > S ? S : window;
  const int s = n_sink > S ? S : n_sink;
  const size_t need = kvp::cutoff_workspace_bytes(rows, S, s);
  if (workspace_bytes < need) return KVP_EWORKSPACE;
  if (need > 0 && (!workspace || !aligned(workspace, 4))) return KVP_EINVAL;
  return from_hip(kvp::launch_cutoff(score, rows, S, w, s, top_k, rank, cutoff, workspace,
                                     stream));
}

}  // extern "C"
