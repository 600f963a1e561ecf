// fp32 inputs: the same quantities as the bf16 matrix-core passes, computed in
// fp32 on the vector ALUs, so that fp32 queries and keys are used as given
// (no rounding to bf16 before the products).
//
//   lse[b, g, i]  = ln sum_{j in K(i)} exp(scale <q_i, k_j>)          (LKV §3 Eq. 1;
//                   K(i) = { j <= i }, or in sparse mode the running top-k
//                   pattern { j <= i : i - j < w or rank[j] <= cutoff[i] },
//                   KVpop §3.2)
//   mass[b, u, j] = sum over the unit's query heads g and rows i >= j + w of
//                   exp(scale <q_i, k_j> - lse[b, g, i])               (KVpop §3.1 Eq. 2,
//                   App. B.1; u = KV head with its G query heads, or one
//                   query head)
//   block mode:     the same sums per query block of the Golden-Eviction
//                   scores, their means and suffix maxima (ForesightKV §3.2).
//
// One thread per query row (LSE) or per key (mass); tiles of 32 keys or
// query rows are staged in LDS and shared by the 256 rows / keys of a
// workgroup.  Dot products are fp32 fused multiply-adds in index order; the
// LSE uses a running maximum, so no row overflows; the mass sums in fp64.
// These passes are O(S^2 d) on the VALU: the exact path for fp32 callers,
// not the fast one (bf16 inputs run on the matrix cores).
#include "kvp_device.h"
#include "kvp_launch.h"

namespace kvp {
namespace {

constexpr int kF32Threads = 256;
constexpr int kF32Tile = 32;

struct F32LseArgs {
  const float* q;
  const float* k;
  float* lse;
  int B, Hq, Hkv, S, G;
  float scale;
  const int32_t* rank;    // sparse mode: [B, Hkv, S]
  const int32_t* cutoff;  // sparse mode: [B, Hkv, S]
  int window;
};

template <int D, bool kSp>
__global__ __launch_bounds__(kF32Threads) void f32_lse_kernel(F32LseArgs a) {
  __shared__ float kt[kF32Tile][D];
  __shared__ int rt[kF32Tile];
  const int S = a.S;
  const int per_head = (S + kF32Threads - 1) / kF32Threads;
  const int bg = blockIdx.x / per_head;  // b * Hq + g
  const int i0 = (blockIdx.x - bg * per_head) * kF32Threads;
  const int b = bg / a.Hq, g = bg - b * a.Hq, h = g / a.G;
  const int i = i0 + (int)threadIdx.x;
  const bool valid = i < S;
  const float* __restrict__ kb = a.k + (size_t)(b * a.Hkv + h) * S * D;
  float qv[D];
  {
    const float* __restrict__ qr = a.q + ((size_t)bg * S + (valid ? i : 0)) * D;
#pragma unroll
    for (int e = 0; e < D; ++e) qv[e] = qr[e];
  }
  int cut = 0;
  if (kSp && valid) cut = a.cutoff[(size_t)(b * a.Hkv + h) * S + i];
  float m = -__builtin_inff(), s = 0.f;
  const int j_end = min(S, i0 + kF32Threads);  // keys any row of the block reaches
  for (int j0 = 0; j0 < j_end; j0 += kF32Tile) {
    __syncthreads();
    for (int e = threadIdx.x; e < kF32Tile * D; e += kF32Threads) {
      const int jj = j0 + e / D;
      kt[e / D][e % D] = jj < S ? kb[(size_t)jj * D + e % D] : 0.f;
    }
    if (kSp && threadIdx.x < kF32Tile) {
      const int jj = j0 + (int)threadIdx.x;
      rt[threadIdx.x] = jj < S ? a.rank[(size_t)(b * a.Hkv + h) * S + jj] : 0;
    }
    __syncthreads();
    if (!valid) continue;
    const int jn = min(kF32Tile, i - j0 + 1);  // keys j0 .. min(i, j0 + 31)
    for (int jj = 0; jj < jn; ++jj) {
      if (kSp && !(i - (j0 + jj) < a.window || rt[jj] <= cut)) continue;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = __builtin_fmaf(qv[e], kt[jj][e], dot);
      const float x = dot * a.scale;
      if (x > m) {
        s = s * expf(m - x) + 1.f;
        m = x;
      } else {
        s += expf(x - m);
      }
    }
  }
  if (valid) a.lse[(size_t)bg * S + i] = s > 0.f ? m + logf(s) : -__builtin_inff();
}

struct F32MassArgs {
  const float* q;
  const float* k;
  const float* lse;
  float* mass;
  int B, Hq, Hkv, S, G, window, per_head;
  float scale;
  // block mode: blocks [seg_start + t len, ...) clipped to S (start, len
  // multiples of 32), n_seg blocks; seg_block may be null
  int seg_start, seg_len, n_seg;
  float* seg_block;
  float* seg_future;
};

template <int D, bool kSeg>
__global__ __launch_bounds__(kF32Threads) void f32_mass_kernel(F32MassArgs a) {
  __shared__ float qt[kF32Tile][D];
  __shared__ float lt[kF32Tile];
  const int S = a.S, w = a.window;
  const int U = a.per_head ? a.Hq : a.Hkv;
  const int per_unit = (S + kF32Threads - 1) / kF32Threads;
  const int bu = blockIdx.x / per_unit;  // b * U + u
  const int j0 = (blockIdx.x - bu * per_unit) * kF32Threads;
  const int b = bu / U, u = bu - b * U;
  const int h = a.per_head ? u / a.G : u;
  const int g_lo = a.per_head ? u : u * a.G;
  const int ng = a.per_head ? 1 : a.G;
  const int j = j0 + (int)threadIdx.x;
  const bool valid = j < S;
  float kv[D];
  {
    const float* __restrict__ kr = a.k + ((size_t)(b * a.Hkv + h) * S + (valid ? j : 0)) * D;
#pragma unroll
    for (int e = 0; e < D; ++e) kv[e] = kr[e];
  }
  // first query row any key of the block counts (and, in block mode, that
  // belongs to a block)
  int i_lo = j0 + w;
  if (kSeg) i_lo = max(i_lo, a.seg_start);
  double acc = 0.0;
  const size_t seg_row0 = (size_t)bu * a.n_seg;
  int t_first = a.n_seg;  // first block this sweep reaches
  for (int i0 = i_lo / kF32Tile * kF32Tile; i0 < S; i0 += kF32Tile) {
    for (int gg = 0; gg < ng; ++gg) {
      const int g = g_lo + gg;
      const float* __restrict__ qb = a.q + (size_t)(b * a.Hq + g) * S * D;
      __syncthreads();
      for (int e = threadIdx.x; e < kF32Tile * D; e += kF32Threads) {
        const int ii = i0 + e / D;
        qt[e / D][e % D] = ii < S ? qb[(size_t)ii * D + e % D] : 0.f;
      }
      if (threadIdx.x < kF32Tile) {
        const int ii = i0 + (int)threadIdx.x;
        lt[threadIdx.x] = ii < S ? a.lse[(size_t)(b * a.Hq + g) * S + ii] : 0.f;
      }
      __syncthreads();
      if (!valid) continue;
      for (int ii = 0; ii < kF32Tile; ++ii) {
        const int i = i0 + ii;
        if (i >= S || i < j + w) continue;
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) dot = __builtin_fmaf(qt[ii][e], kv[e], dot);
        acc += (double)expf(dot * a.scale - lt[ii]);
      }
    }
    if constexpr (kSeg) {
      // the tile lies in one block; flush after the block's last tile
      const int t = (i0 - a.seg_start) / a.seg_len;
      const int end = min(S, a.seg_start + (t + 1) * a.seg_len);
      if (i0 + kF32Tile >= end) {
        if (valid) {
          const int rows = end - (a.seg_start + t * a.seg_len);
          const float mean = (float)(acc / ((double)rows * ng));
          if (a.seg_block) a.seg_block[(seg_row0 + t) * S + j] = mean;
          a.seg_future[(seg_row0 + t) * S + j] = mean;  // turned into the suffix maximum below
        }
        if (t < t_first) t_first = t;
        acc = 0.0;
      }
    }
  }
  if (!valid) return;
  if constexpr (kSeg) {
    // blocks before the first one swept: no query sees the key there; then
    // the suffix maximum from the last block down
    for (int t = 0; t < t_first; ++t) {
      if (a.seg_block) a.seg_block[(seg_row0 + t) * S + j] = 0.f;
      a.seg_future[(seg_row0 + t) * S + j] = 0.f;
    }
    float run = 0.f;
    for (int t = a.n_seg - 1; t >= 0; --t) {
      float* f = a.seg_future + (seg_row0 + t) * S + j;
      run = fmaxf(run, *f);
      *f = run;
    }
  } else {
    a.mass[(size_t)bu * S + j] = (float)acc;
  }
}

template <int D>
hipError_t lse_f32_d(const void* q, const void* k, const Shape& sh, float scale, const int32_t* rank,
                     const int32_t* cutoff, int window, float* lse, hipStream_t stream) {
  F32LseArgs a;
  a.q = static_cast<const float*>(q);
  a.k = static_cast<const float*>(k);
  a.lse = lse;
  a.B = sh.B;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.S = sh.S;
  a.G = sh.G;
  a.scale = scale;
  a.rank = rank;
  a.cutoff = cutoff;
  a.window = window;
  const int64_t blocks = (int64_t)sh.B * sh.Hq * ((sh.S + kF32Threads - 1) / kF32Threads);
  if (rank)
    hipLaunchKernelGGL((f32_lse_kernel<D, true>), dim3((unsigned)blocks), dim3(kF32Threads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((f32_lse_kernel<D, false>), dim3((unsigned)blocks), dim3(kF32Threads), 0,
                       stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t mass_f32_d(const void* q, const void* k, const float* lse, const Shape& sh, float scale,
                      int window, int per_head, float* mass, const SegOut& seg,
                      hipStream_t stream) {
  F32MassArgs a;
  a.q = static_cast<const float*>(q);
  a.k = static_cast<const float*>(k);
  a.lse = lse;
  a.mass = mass;
  a.B = sh.B;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.S = sh.S;
  a.G = sh.G;
  a.window = window;
  a.per_head = per_head;
  a.scale = scale;
  a.seg_start = seg.start;
  a.seg_len = seg.len;
  a.n_seg = seg.n;
  a.seg_block = seg.block;
  a.seg_future = seg.future;
  const int64_t units = (int64_t)sh.B * (per_head ? sh.Hq : sh.Hkv);
  const int64_t blocks = units * ((sh.S + kF32Threads - 1) / kF32Threads);
  if (seg.n > 0)
    hipLaunchKernelGGL((f32_mass_kernel<D, true>), dim3((unsigned)blocks), dim3(kF32Threads), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((f32_mass_kernel<D, false>), dim3((unsigned)blocks), dim3(kF32Threads), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_f32(const void* q, const void* k, const Shape& sh, float scale,
                          const int32_t* rank, const int32_t* cutoff, int window, float* lse,
                          hipStream_t stream) {
  return sh.D == 128 ? lse_f32_d<128>(q, k, sh, scale, rank, cutoff, window, lse, stream)
                     : lse_f32_d<64>(q, k, sh, scale, rank, cutoff, window, lse, stream);
}

hipError_t launch_mass_f32(const void* q, const void* k, const float* lse, const Shape& sh,
                           float scale, int window, int per_head, float* mass, const SegOut& seg,
                           hipStream_t stream) {
  return sh.D == 128
             ? mass_f32_d<128>(q, k, lse, sh, scale, window, per_head, mass, seg, stream)
             : mass_f32_d<64>(q, k, lse, sh, scale, window, per_head, mass, seg, stream);
}

}  // namespace kvp
