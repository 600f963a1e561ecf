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
// R consecutive lanes per query row (LSE) or per key (mass), R = 1 for large
// problems and up to 16 for small ones; tiles of 32 KiB of key or query rows
// are staged in LDS and shared by the workgroup.  Dot products are fp32 fused
// multiply-adds (four partial sums); the LSE uses a running maximum, so no
// row overflows; the mass sums in fp64; the lanes of a group merge their
// partial results in a fixed order.
// These passes are O(S^2 d) on the VALU: the exact path for fp32 callers,
// not the fast one (bf16 inputs run on the matrix cores).
#include "kvp_device.h"
#include "kvp_launch.h"

namespace kvp {
namespace {

constexpr int kF32Threads = 256;
// rows per LDS tile: 32 KiB of fp32 rows (128 at d = 64, 64 at d = 128)
template <int D>
constexpr int f32_tile() {
  return 32768 / (4 * D);
}

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

// Dot product of a register row and an LDS row, with four partial sums for
// instruction-level parallelism.
template <int D>
__device__ __forceinline__ float dot_f32(const float (&x)[D], const float* y) {
  float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < D; ++e) p[e & 3] = __builtin_fmaf(x[e], y[e], p[e & 3]);
  return (p[0] + p[1]) + (p[2] + p[3]);
}

// Online log-sum-exp state (running maximum m, sum s relative to it).  The
// sum is kept in fp64: with one dominant term (s near 1) a row's thousands of
// terms below half an fp32 ulp of s would each be rounded away in an fp32 sum,
// a relative loss of up to their total (1e-4 seen on a 7.5K-key row).
__device__ __forceinline__ void lse_add(float& m, double& s, float x) {
  if (x > m) {
    s = s * (double)expf(m - x) + 1.0;
    m = x;
  } else {
    s += (double)expf(x - m);
  }
}
__device__ __forceinline__ void lse_merge(float& m, double& s, float m2, double s2) {
  if (m2 > m) {
    s = s * (double)expf(m - m2) + s2;
    m = m2;
  } else if (s2 > 0.0) {
    s += s2 * (double)expf(m2 - m);
  }
}

// R consecutive lanes share a query row (R = 1 for large problems, more for
// small ones so that the grid fills the GPU); lane r of a group takes the keys
// j = r (mod R), and the group merges its partial states in a fixed order.
template <int D, bool kSp, int R>
__global__ __launch_bounds__(kF32Threads) void f32_lse_kernel(F32LseArgs a) {
  constexpr int kRows = kF32Threads / R;  // query rows per workgroup
  constexpr int kF32Tile = f32_tile<D>();
  __shared__ float kt[kF32Tile][D];
  __shared__ int rt[kF32Tile];
  const int S = a.S;
  const int per_head = (S + kRows - 1) / kRows;
  const int bg = blockIdx.x / per_head;  // b * Hq + g
  const int i0 = (blockIdx.x - bg * per_head) * kRows;
  const int b = bg / a.Hq, g = bg - b * a.Hq, h = g / a.G;
  const int r = (int)threadIdx.x % R;
  const int i = i0 + (int)threadIdx.x / R;
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
  float m = -__builtin_inff();
  double s = 0.0;
  const int j_end = min(S, i0 + kRows);  // keys any row of the block reaches
  for (int j0 = 0; j0 < j_end; j0 += kF32Tile) {
    __syncthreads();
    for (int e = threadIdx.x; e < kF32Tile * D; e += kF32Threads) {
      const int jj = j0 + e / D;
      kt[e / D][e % D] = jj < S ? kb[(size_t)jj * D + e % D] : 0.f;
    }
    if (kSp)
      for (int t = threadIdx.x; t < kF32Tile; t += kF32Threads) {
        const int jj = j0 + t;
        rt[t] = jj < S ? a.rank[(size_t)(b * a.Hkv + h) * S + jj] : 0;
      }
    __syncthreads();
    if (!valid) continue;
    const int jn = min(kF32Tile, i - j0 + 1);  // keys j0 .. min(i, j0 + kF32Tile - 1)
    for (int jj = r; jj < jn; jj += R) {
      if (kSp && !(i - (j0 + jj) < a.window || rt[jj] <= cut)) continue;
      lse_add(m, s, dot_f32<D>(qv, kt[jj]) * a.scale);
    }
  }
#pragma unroll
  for (int off = 1; off < R; off <<= 1) {
    const float m2 = __shfl_xor(m, off);
    const double s2 = __shfl_xor(s, off);
    // lanes merge in the same order on both sides of each exchange
    if ((r & off) == 0)
      lse_merge(m, s, m2, s2);
    else {
      float mm = m2;
      double ss = s2;
      lse_merge(mm, ss, m, s);
      m = mm;
      s = ss;
    }
  }
  if (valid && r == 0) a.lse[(size_t)bg * S + i] = s > 0.0 ? (float)((double)m + log(s)) : -__builtin_inff();
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

// Sum of a double over the R lanes of a group, in a fixed order.
template <int R>
__device__ __forceinline__ double group_sum(double v) {
#pragma unroll
  for (int off = 1; off < R; off <<= 1) {
    const double o = __shfl_xor(v, off);
    v = ((threadIdx.x & off) == 0) ? v + o : o + v;
  }
  return v;
}

// R consecutive lanes share a key; lane r of a group takes the query rows
// i = r (mod R) of every staged tile.
template <int D, bool kSeg, int R>
__global__ __launch_bounds__(kF32Threads) void f32_mass_kernel(F32MassArgs a) {
  constexpr int kKeys = kF32Threads / R;  // keys per workgroup
  // block mode: tiles of 32 rows, so that none straddles a block edge
  constexpr int kF32Tile = kSeg ? 32 : f32_tile<D>();
  __shared__ float qt[kF32Tile][D];
  __shared__ float lt[kF32Tile];
  const int S = a.S, w = a.window;
  const int U = a.per_head ? a.Hq : a.Hkv;
  const int per_unit = (S + kKeys - 1) / kKeys;
  const int bu = blockIdx.x / per_unit;  // b * U + u
  const int j0 = (blockIdx.x - bu * per_unit) * kKeys;
  const int b = bu / U, u = bu - b * U;
  const int h = a.per_head ? u / a.G : u;
  const int g_lo = a.per_head ? u : u * a.G;
  const int ng = a.per_head ? 1 : a.G;
  const int r = (int)threadIdx.x % R;
  const int j = j0 + (int)threadIdx.x / R;
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
      for (int t = threadIdx.x; t < kF32Tile; t += kF32Threads) {
        const int ii = i0 + t;
        lt[t] = ii < S ? a.lse[(size_t)(b * a.Hq + g) * S + ii] : 0.f;
      }
      __syncthreads();
      if (!valid) continue;
      for (int ii = r; ii < kF32Tile; ii += R) {
        const int i = i0 + ii;
        if (i >= S || i < j + w) continue;
        acc += (double)expf(dot_f32<D>(kv, qt[ii]) * a.scale - lt[ii]);
      }
    }
    if constexpr (kSeg) {
      // the tile lies in one block; flush after the block's last tile
      const int t = (i0 - a.seg_start) / a.seg_len;
      const int end = min(S, a.seg_start + (t + 1) * a.seg_len);
      if (i0 + kF32Tile >= end) {
        const double tot = group_sum<R>(acc);
        if (valid && r == 0) {
          const int rows = end - (a.seg_start + t * a.seg_len);
          const float mean = (float)(tot / ((double)rows * ng));
          if (a.seg_block) a.seg_block[(seg_row0 + t) * S + j] = mean;
          a.seg_future[(seg_row0 + t) * S + j] = mean;  // turned into the suffix maximum below
        }
        if (t < t_first) t_first = t;
        acc = 0.0;
      }
    }
  }
  if constexpr (kSeg) {
    if (!valid || r != 0) return;
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
    const double tot = group_sum<R>(acc);
    if (valid && r == 0) a.mass[(size_t)bu * S + j] = (float)tot;
  }
}

// Lanes per row / key: 1 when the problem already gives every CU several
// workgroups, up to 16 for small ones.
int lanes_for(int64_t rows) {
  int R = 1;
  while (R < 16 && rows * R < (int64_t)kNumCUs * kF32Threads * 2) R *= 2;
  return R;
}

template <int D, bool kSp, int R>
void lse_f32_launch(const F32LseArgs& a, hipStream_t stream) {
  constexpr int kRows = kF32Threads / R;
  const int64_t blocks = (int64_t)a.B * a.Hq * ((a.S + kRows - 1) / kRows);
  hipLaunchKernelGGL((f32_lse_kernel<D, kSp, R>), dim3((unsigned)blocks), dim3(kF32Threads), 0,
                     stream, a);
}

template <int D, bool kSp>
void lse_f32_r(const F32LseArgs& a, int R, hipStream_t stream) {
  switch (R) {
    case 1: lse_f32_launch<D, kSp, 1>(a, stream); break;
    case 2: lse_f32_launch<D, kSp, 2>(a, stream); break;
    case 4: lse_f32_launch<D, kSp, 4>(a, stream); break;
    case 8: lse_f32_launch<D, kSp, 8>(a, stream); break;
    default: lse_f32_launch<D, kSp, 16>(a, stream); break;
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
  const int R = lanes_for((int64_t)sh.B * sh.Hq * sh.S);
  if (rank)
    lse_f32_r<D, true>(a, R, stream);
  else
    lse_f32_r<D, false>(a, R, stream);
  return hipGetLastError();
}

template <int D, bool kSeg, int R>
void mass_f32_launch(const F32MassArgs& a, int64_t units, hipStream_t stream) {
  constexpr int kKeys = kF32Threads / R;
  const int64_t blocks = units * ((a.S + kKeys - 1) / kKeys);
  hipLaunchKernelGGL((f32_mass_kernel<D, kSeg, R>), dim3((unsigned)blocks), dim3(kF32Threads), 0,
                     stream, a);
}

template <int D, bool kSeg>
void mass_f32_r(const F32MassArgs& a, int64_t units, int R, hipStream_t stream) {
  switch (R) {
    case 1: mass_f32_launch<D, kSeg, 1>(a, units, stream); break;
    case 2: mass_f32_launch<D, kSeg, 2>(a, units, stream); break;
    case 4: mass_f32_launch<D, kSeg, 4>(a, units, stream); break;
    case 8: mass_f32_launch<D, kSeg, 8>(a, units, stream); break;
    default: mass_f32_launch<D, kSeg, 16>(a, units, stream); break;
  }
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
  const int R = lanes_for(units * sh.S);
  if (seg.n > 0)
    mass_f32_r<D, true>(a, units, R, stream);
  else
    mass_f32_r<D, false>(a, units, R, stream);
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
