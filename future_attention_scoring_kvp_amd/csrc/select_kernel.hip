// Per-KV-head keep-set for gfx950.
//
//   keep = ascending( sinks [0, min(s, S))  U  window [max(0, S - w), S)
//                     U  top-k of score over the eligible range [s, S - w) )
// KVpop Fig. 1 / §3 Eq. 1 (budget s + w + k per KV head) and Eq. 4 (eligible
// set at the last query).  The scores are future masses or any fp32 score
// (e.g. the log targets, which are negative).  Ranking: score descending,
// equal scores by ascending index.
//
// One workgroup (256 threads) per (batch, KV head) row:
//   1. radix select, most significant byte first, on an order-preserving
//      32-bit key of each fp32 score (any sign; see score_key): four passes of a
//      256-bin LDS histogram over the candidates that match the bytes fixed
//      so far give the k-th largest value T exactly and the number r of
//      copies of T that belong to the top-k (the r lowest-indexed ones);
//   2. one ordered sweep over the row in chunks of 256 positions: per chunk,
//      wave ballots plus a 4-wave LDS scan give every kept position its
//      output slot and every copy of T its tie rank, so the output is written
//      ascending with no sort.
#include "kvp_device.h"
#include "kvp_launch.h"

namespace kvp {
namespace {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;

struct SelArgs {
  const float* mass;
  int32_t* keep;
  int S, window, n_sink, top_k;
  int64_t n_keep;
};

// Order-preserving key of a float: unsigned key order equals numeric order
// for every non-NaN value (negative values have all bits flipped, positive
// ones the sign bit set); -0 is first mapped to +0 so that the two zeros tie.
__device__ __forceinline__ uint32_t score_key(float m) {
  uint32_t u = __builtin_bit_cast(uint32_t, m);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix (over the workgroup, in thread order) of a 0/1 flag, and
// the chunk total.  Uses wave ballots and a 4-entry LDS table.
__device__ __forceinline__ int block_prefix(bool flag, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint64_t bal = __ballot(flag);
  const int in_wave = __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
  if (lane == 0) wave_tot[wave] = __popcll(bal);
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int t = wave_tot[w];
    if (w < wave) before += t;
    total += t;
  }
  __syncthreads();
  return before + in_wave;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelArgs a) {
  __shared__ int hist[256];
  __shared__ int wave_tot[kSelWaves];
  __shared__ uint32_t sel_digit;
  __shared__ int sel_above;

  const int tid = threadIdx.x;
  const int S = a.S;
  const float* __restrict__ m = a.mass + (size_t)blockIdx.x * S;
  int32_t* __restrict__ out = a.keep + (size_t)blockIdx.x * a.n_keep;

  const int e_lo = a.n_sink;                 // eligible range [e_lo, e_hi)
  const int e_hi = S - a.window;             // may be <= e_lo (empty)
  const int n_elig = e_hi > e_lo ? e_hi - e_lo : 0;
  const int kk = a.top_k < n_elig ? a.top_k : n_elig;
  const bool take_all = kk == n_elig;

  // --- 1. threshold T and tie count r (only when 0 < kk < n_elig)
  uint32_t prefix = 0, pmask = 0;
  int r = kk;
  if (!take_all && kk > 0) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      for (int j = e_lo + tid; j < e_hi; j += kSelThreads) {
        const uint32_t u = score_key(m[j]);
        if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid == 0) {
        int above = 0;
        int d = 255;
        for (; d > 0; --d) {
          if (above + hist[d] >= r) break;
          above += hist[d];
        }
        sel_digit = (uint32_t)d;
        sel_above = above;
      }
      __syncthreads();
      prefix |= sel_digit << shift;
      pmask |= 255u << shift;
      r -= sel_above;
      __syncthreads();
    }
  }
  const uint32_t T = prefix;

  // --- 2. ordered emission
  int written = 0;
  int ties_seen = 0;
  for (int base = 0; base < S; base += kSelThreads) {
    const int j = base + tid;
    bool kept = false, is_tie = false;
    if (j < S) {
      if (j < a.n_sink || j >= e_hi) {
        kept = true;  // sink or protected window
      } else if (kk > 0) {
        if (take_all) {
          kept = true;
        } else {
          const uint32_t u = score_key(m[j]);
          kept = u > T;
          is_tie = u == T;
        }
      }
    }
    int n_ties = 0;
    const int tie_rank = ties_seen + block_prefix(is_tie, wave_tot, n_ties);
    if (is_tie && tie_rank < r) kept = true;
    ties_seen += n_ties;
    int n_kept = 0;
    const int slot = written + block_prefix(kept, wave_tot, n_kept);
    if (kept && slot < a.n_keep) out[slot] = j;
    written += n_kept;
  }
}

}  // namespace

hipError_t launch_select(const float* mass, int64_t rows, int S, int window, int n_sink,
                         int top_k, int64_t n_keep, int32_t* keep, hipStream_t stream) {
  SelArgs a;
  a.mass = mass;
  a.keep = keep;
  a.S = S;
  a.window = window;
  a.n_sink = n_sink;
  a.top_k = top_k;
  a.n_keep = n_keep;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)rows), dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvp
