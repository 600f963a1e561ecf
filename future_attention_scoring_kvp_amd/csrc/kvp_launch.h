// Internal launcher interface between the C ABI (kvp_api.cpp) and the kernel
// translation units.  Arguments are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvp {

struct Shape {
  int B, Hq, Hkv, S, D;
  int G;  // Hq / Hkv
};

// dtype: 0 = bf16 (matrix cores), 1 = fp32 (exact fp32 path, launch_*_f32).
hipError_t launch_lse(const void* q, const void* k, int dtype, const Shape& sh, float scale,
                      float* lse, hipStream_t stream);
// LSE over the running top-k pattern: j counts for i iff j <= i and
// (i - j < window or rank[j] <= cutoff[i]); rank, cutoff [B, Hkv, S].
hipError_t launch_lse_sparse(const void* q, const void* k, int dtype, const Shape& sh, float scale,
                             const int32_t* rank, const int32_t* cutoff, int window, float* lse,
                             hipStream_t stream);
// per_head = 0: mass [B, Hkv, S] summed over each group; 1: mass [B, Hq, S].
hipError_t launch_mass(const void* q, const void* k, const float* lse, int dtype, const Shape& sh,
                       float scale, int window, int per_head, float* mass, hipStream_t stream);
// The same pass with a workspace: short sequences cut each key tile's query
// sweep into chunks whose partial masses go to the workspace and are added in
// chunk order by a second kernel.  mass_workspace_bytes is 0 where no launch
// is cut; launch_mass_ws then (or with a null workspace) runs launch_mass.
size_t mass_workspace_bytes(int dtype, const Shape& sh, int window, int per_head);
hipError_t launch_mass_ws(const void* q, const void* k, const float* lse, int dtype,
                          const Shape& sh, float scale, int window, int per_head, float* mass,
                          void* workspace, hipStream_t stream);
// Query-block mode of the mass pass (Golden-Eviction scores): blocks
// [start + t len, start + (t+1) len) clipped to S, start and len multiples of
// 32, n blocks; block (may be null) and future are [B, U, n, S] with U = Hkv
// (group mean) or Hq (per_head).
struct SegOut {
  int start, len, n;
  float* block;
  float* future;
};
hipError_t launch_block_scores(const void* q, const void* k, const float* lse, int dtype,
                               const Shape& sh, float scale, int window, int per_head,
                               const SegOut& seg, hipStream_t stream);
// fp32 inputs: the LSE (sparse when rank is not null) and the mass / block
// scores computed in fp32 on the vector ALUs, with no rounding of the inputs.
hipError_t launch_lse_f32(const void* q, const void* k, const Shape& sh, float scale,
                          const int32_t* rank, const int32_t* cutoff, int window, float* lse,
                          hipStream_t stream);
hipError_t launch_mass_f32(const void* q, const void* k, const float* lse, const Shape& sh,
                           float scale, int window, int per_head, float* mass, const SegOut& seg,
                           hipStream_t stream);
// Target scores [B, Hkv, S] from masses ([B, Hq, S] per head or [B, Hkv, S]
// group sums); agg: 0 log of the mean, 1 mean of the logs, 2 max of the logs;
// query < 0: no decay.
hipError_t launch_target(const float* mass, int per_head, const Shape& sh, int window,
                         int normalize, int agg, float eps, int query, int decay_step,
                         const float* log_gamma, float* score, hipStream_t stream);
// Keep-set of `rows` rows of S scores.  Rows longer than 32768 are split
// over several workgroups with their state in `workspace`, of
// select_workspace_bytes(rows, S) bytes (0: no workspace is read); its
// blocks number select_split_blocks(rows, S) per launch.
size_t select_workspace_bytes(int64_t rows, int S);
int64_t select_split_blocks(int64_t rows, int S);
// Static priorities [B, Hkv, S] of the running top-k from undecayed scores.
hipError_t launch_priority(const float* score, const Shape& sh, int decay_step,
                           const float* log_gamma, float* priority, hipStream_t stream);
hipError_t launch_select(const float* mass, int64_t rows, int S, int window, int n_sink,
                         int top_k, int64_t n_keep, int32_t* keep, void* workspace,
                         hipStream_t stream);
// The library's own fixed workspace for the selection (a device array of
// kSelectScratchBytes per GPU): its device address on the current device,
// looked up once per device.  Calls that use it on one GPU share it.
constexpr size_t kSelectScratchBytes = size_t(32) << 20;
hipError_t select_scratch(void** ptr);

// Running top-k cutoff: rank [rows, S] and cutoff [rows, S] (int32) from
// scores [rows, S]; workspace of cutoff_workspace_bytes(rows, S, n_sink).
size_t cutoff_workspace_bytes(int64_t rows, int S, int n_sink);
hipError_t launch_cutoff(const float* score, int64_t rows, int S, int window, int n_sink,
                         int top_k, int32_t* rank, int32_t* cutoff, void* workspace,
                         hipStream_t stream);

// LKV Soft-TopK per row of n scores: forward (y, lam) and backward (dx, dk).
hipError_t launch_soft_topk_fwd(const float* x, const float* k, int64_t rows, int n, float tau,
                                float* y, float* lam, hipStream_t stream);
hipError_t launch_soft_topk_bwd(const float* x, const float* lam, const float* dy, int64_t rows,
                                int n, float tau, float* dx, float* dk, hipStream_t stream);

}  // namespace kvp
