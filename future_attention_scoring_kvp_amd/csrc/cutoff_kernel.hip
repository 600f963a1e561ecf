// Running top-k cutoff of KVpop for gfx950 (§3.2 "Efficient Target
// Implementation", the paragraphs on running top-k sparse attention and its
// kernel; Appendix I).
//
// Per (batch, KV head) row of static priorities score[0..S):
//   rank[t]   position of token t >= s in the order (priority descending,
//             equal priorities by ascending index), 0 = best; -1 for sinks;
//   cutoff[q] rank of the k-th best token of E(q) = {s <= t <= q - w}
//             (Eq. 4), S while fewer than k tokens are eligible, -1 if k = 0.
// At query q an eligible token t is retained iff rank[t] <= cutoff[q].
//
// The page inserts each newly eligible rank into a Fenwick tree and finds the
// k-th best by binary lifting.  Here the two passes exploit that the cutoff
// never rises once k tokens are eligible (adding a token can only push the
// k-th best to a better rank):
//   rank_kernel    one workgroup per row: stable LSD radix sort of the
//                  order-preserving keys, one bit per pass (a block-wide
//                  stable partition with wave ballots), passes whose bit is
//                  the same for every key are skipped; then rank[pos[r]] = r;
//   cutoff_kernel  one wave per row sweeps q in order.  While at most k
//                  tokens are eligible the cutoff is the largest eligible
//                  rank; afterwards a new token ranked below the cutoff moves
//                  it down to the next rank whose token is already eligible
//                  (pos[r] <= q - w).  The cutoff only moves down, so the
//                  sweep is O(S) per row; ranks and positions are read 64 at
//                  a time into lanes and consumed with uniform control flow.
#include "kvp_device.h"
#include "kvp_launch.h"

namespace kvp {
namespace {

constexpr int kRankThreads = 256;
constexpr int kRankWaves = kRankThreads / kWave;

__device__ __forceinline__ uint32_t order_key(float m) {
  uint32_t u = __builtin_bit_cast(uint32_t, m);
  if (u == 0x80000000u) u = 0u;  // -0 ties +0
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;  // ascending key order = descending priority
}

// Exclusive prefix over the workgroup (thread order) of a 0/1 flag, and the
// total; wave ballots and one LDS slot per wave.
__device__ __forceinline__ int rank_block_prefix(bool flag, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint64_t bal = __ballot(flag);
  const int in_wave = __popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
  if (lane == 0) wave_tot[wave] = __popcll(bal);
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kRankWaves; ++w) {
    const int t = wave_tot[w];
    if (w < wave) before += t;
    total += t;
  }
  __syncthreads();
  return before + in_wave;
}

struct CutoffArgs {
  const float* score;
  int32_t* rank;
  int32_t* cutoff;
  uint32_t* ws;  // per row: pos, keysA, idxA, keysB, idxB (n words each)
  int S, s, window, top_k;
};

__global__ __launch_bounds__(kRankThreads) void rank_kernel(CutoffArgs a) {
  __shared__ int wave_tot[kRankWaves];
  __shared__ int zero_count;
  const int S = a.S, s = a.s, n = S - s;
  const int tid = threadIdx.x;
  const float* __restrict__ m = a.score + (size_t)blockIdx.x * S;
  int32_t* __restrict__ rk = a.rank + (size_t)blockIdx.x * S;
  uint32_t* pos = a.ws + (size_t)blockIdx.x * 5 * n;
  uint32_t* ka = pos + n;
  uint32_t* ia = ka + n;
  uint32_t* kb = ia + n;
  uint32_t* ib = kb + n;

  for (int t = tid; t < s; t += kRankThreads) rk[t] = -1;
  for (int i = tid; i < n; i += kRankThreads) {
    ka[i] = order_key(m[s + i]);
    ia[i] = (uint32_t)(s + i);
  }
  __syncthreads();

  for (int bit = 0; bit < 32; ++bit) {
    // zeros of this bit
    if (tid == 0) zero_count = 0;
    __syncthreads();
    int local = 0;
    for (int i = tid; i < n; i += kRankThreads) local += ((ka[i] >> bit) & 1u) ? 0 : 1;
    atomicAdd(&zero_count, local);
    __syncthreads();
    const int zeros = zero_count;
    __syncthreads();
    if (zeros == 0 || zeros == n) continue;  // every key has the same bit: order unchanged
    // stable partition: zeros first, then ones, each in their current order
    int zeros_before = 0;
    for (int base = 0; base < n; base += kRankThreads) {
      const int i = base + tid;
      const bool valid = i < n;
      const uint32_t key = valid ? ka[i] : 0u;
      const uint32_t idx = valid ? ia[i] : 0u;
      const bool zero = valid && !((key >> bit) & 1u);
      int chunk_zeros = 0;
      const int zpre = rank_block_prefix(zero, wave_tot, chunk_zeros);
      if (valid) {
        const int dst = zero ? zeros_before + zpre
                             : zeros + (base - zeros_before) + (tid - zpre);
        kb[dst] = key;
        ib[dst] = idx;
      }
      zeros_before += chunk_zeros;
    }
    __syncthreads();
    uint32_t* tk = ka; ka = kb; kb = tk;
    uint32_t* ti = ia; ia = ib; ib = ti;
  }
  for (int r = tid; r < n; r += kRankThreads) {
    const uint32_t t = ia[r];
    pos[r] = t;
    rk[t] = r;
  }
}

// One wave per row (4 rows per 256-thread block).
__global__ __launch_bounds__(256) void cutoff_kernel(CutoffArgs a, int rows) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int S = a.S, s = a.s, w = a.window, k = a.top_k, n = S - s;
  const int32_t* __restrict__ rk = a.rank + (size_t)row * S;
  const uint32_t* __restrict__ pos = a.ws + (size_t)row * 5 * n;
  int32_t* __restrict__ out = a.cutoff + (size_t)row * S;

  int eligible = 0;  // uniform state
  int tau = -1;
  int pchunk = 1 << 30;  // start of the positions held in lanes (none yet)
  uint32_t plane = 0;
  for (int q0 = 0; q0 < S; q0 += 64) {
    // ranks of the tokens that enter at q0 .. q0 + 63 (t = q - w), -2 if none
    const int t_l = q0 + lane - w;
    const int r_l = (t_l >= s && t_l < S && q0 + lane < S) ? rk[t_l] : -2;
    int my_out = 0;
    const int nq = min(64, S - q0);
    for (int j = 0; j < nq; ++j) {
      const int q = q0 + j;
      const int r_new = __builtin_amdgcn_readlane(r_l, j);
      if (r_new >= 0) {
        ++eligible;
        if (eligible <= k) {
          tau = max(tau, r_new);
        } else if (r_new < tau) {
          // next lower rank whose token is already eligible (pos <= q - w);
          // the new token itself qualifies, so the walk ends at r_new at the
          // latest (also the loop bound)
          for (;;) {
            --tau;
            if (tau <= r_new) break;
            if (tau < pchunk) {
              pchunk = max(0, tau - 63);
              plane = (pchunk + lane < n) ? pos[pchunk + lane] : 0u;
            }
            const int p = (int)__builtin_amdgcn_readlane((int)plane, tau - pchunk);
            if (p <= q - w) break;
          }
        }
      }
      const int c = (k == 0) ? -1 : (eligible < k ? S : tau);
      if (lane == j) my_out = c;
    }
    if (lane < nq) out[q0 + lane] = my_out;
  }
}

}  // namespace

size_t cutoff_workspace_bytes(int64_t rows, int S, int n_sink) {
  const int64_t n = S > n_sink ? (int64_t)S - n_sink : 0;
  return (size_t)(rows * n * 5 * sizeof(uint32_t));
}

hipError_t launch_cutoff(const float* score, int64_t rows, int S, int window, int n_sink,
                         int top_k, int32_t* rank, int32_t* cutoff, void* workspace,
                         hipStream_t stream) {
  CutoffArgs a;
  a.score = score;
  a.rank = rank;
  a.cutoff = cutoff;
  a.ws = static_cast<uint32_t*>(workspace);
  a.S = S;
  a.s = n_sink;
  a.window = window;
  a.top_k = top_k;
  hipLaunchKernelGGL(rank_kernel, dim3((unsigned)rows), dim3(kRankThreads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(cutoff_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a,
                     (int)rows);
  return hipGetLastError();
}

}  // namespace kvp
