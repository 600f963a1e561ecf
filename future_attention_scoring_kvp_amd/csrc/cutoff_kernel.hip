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
// k-th best by binary lifting.  Here, two kernels:
//   rank_kernel    one workgroup per row: stable LSD radix sort of the
//                  order-preserving keys in 4-bit digits (see below); then
//                  rank[pos[r]] = r;
//   cutoff_kernel  one wave per chunk of 1024 queries of a row.  Its first
//                  state is counted directly from the ranks; then, since the
//                  cutoff never rises once k tokens are eligible (a new token
//                  can only push the k-th best to a better rank), a new token
//                  ranked below the cutoff moves it down to the next rank
//                  whose token is already eligible (pos[r] <= q - w).  Ranks
//                  and positions are read 64 at a time into lanes and consumed
//                  with uniform control flow; when k << n the walks are long
//                  and test 64 ranks per ballot.
#include "kvp_device.h"
#include "kvp_launch.h"

namespace kvp {
namespace {

constexpr int kRankThreads = 1024;
constexpr int kRankWaves = kRankThreads / kWave;

__device__ __forceinline__ uint32_t order_key(float m) {
  uint32_t u = __builtin_bit_cast(uint32_t, m);
  if (u == 0x80000000u) u = 0u;  // -0 ties +0
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;  // ascending key order = descending priority
}

struct CutoffArgs {
  const float* score;
  int32_t* rank;
  int32_t* cutoff;
  uint32_t* ws;  // per row: pos, keysA, idxA, keysB, idxB (n words each)
  int S, s, window, top_k;
};

constexpr int kDigitBits = 4;
constexpr int kDigits = 1 << kDigitBits;
constexpr int kPasses = 32 / kDigitBits;

// Stable LSD radix sort of one row, 4-bit digits.  One counting pass builds
// the digit histograms of all eight passes; each pass then scatters the keys
// chunk by chunk (one element per thread, in order): an element's slot is its digit's
// running base + the count of equal digits in earlier waves of the chunk +
// its rank among equal digits in its wave (four ballots give the lanes with
// the same digit).  Passes whose digit is the same for every key are skipped.
__global__ __launch_bounds__(kRankThreads) void rank_kernel(CutoffArgs a) {
  __shared__ int hist[kPasses][kDigits];
  __shared__ int whist[kRankWaves][kPasses][kDigits];  // per-wave copies: fewer atomic collisions
  __shared__ int wave_cnt[kRankWaves][kDigits];
  __shared__ int base[kDigits];
  const int S = a.S, s = a.s, n = S - s;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const float* __restrict__ m = a.score + (size_t)blockIdx.x * S;
  int32_t* __restrict__ rk = a.rank + (size_t)blockIdx.x * S;
  uint32_t* pos = a.ws + (size_t)blockIdx.x * 5 * n;
  uint32_t* ka = pos + n;
  uint32_t* ia = ka + n;
  uint32_t* kb = ia + n;
  uint32_t* ib = kb + n;

  for (int i = tid; i < kRankWaves * kPasses * kDigits; i += kRankThreads) (&whist[0][0][0])[i] = 0;
  for (int t = tid; t < s; t += kRankThreads) rk[t] = -1;
  __syncthreads();
  for (int i = tid; i < n; i += kRankThreads) {
    const uint32_t key = order_key(m[s + i]);
    ka[i] = key;
    ia[i] = (uint32_t)(s + i);
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
      atomicAdd(&whist[wave][p][(key >> (kDigitBits * p)) & (kDigits - 1)], 1);
  }
  __syncthreads();
  if (tid < kPasses * kDigits) {
    int tot = 0;
    for (int w2 = 0; w2 < kRankWaves; ++w2) tot += (&whist[w2][0][0])[tid];
    (&hist[0][0])[tid] = tot;
  }
  __syncthreads();

  for (int i = tid; i < kRankWaves * kDigits; i += kRankThreads) (&wave_cnt[0][0])[i] = 0;
  for (int p = 0; p < kPasses; ++p) {
    const int shift = kDigitBits * p;
    bool trivial = false;
#pragma unroll
    for (int d = 0; d < kDigits; ++d) trivial |= hist[p][d] == n;
    if (trivial || n == 0) continue;  // uniform: the order does not change
    if (tid < kDigits) {
      int acc = 0;
      for (int d = 0; d < tid; ++d) acc += hist[p][d];
      base[tid] = acc;
    }
    // the next chunk's key and index are loaded while this one is scattered
    uint32_t nkey = tid < n ? ka[tid] : 0u;
    uint32_t nidx = tid < n ? ia[tid] : 0u;
    for (int c = 0; c < n; c += kRankThreads) {
      const int i = c + tid;
      const bool valid = i < n;
      const uint32_t key = nkey;
      const uint32_t idx = nidx;
      if (i + kRankThreads < n) {
        nkey = ka[i + kRankThreads];
        nidx = ia[i + kRankThreads];
      }
      const int d = (int)((key >> shift) & (kDigits - 1));
      uint64_t same = __ballot(valid);
#pragma unroll
      for (int bbit = 0; bbit < kDigitBits; ++bbit) {
        const uint64_t bal = __ballot(valid && ((d >> bbit) & 1));
        same &= ((d >> bbit) & 1) ? bal : ~bal;
      }
      const int in_rank = __popcll(same & lt_mask);
      // bases of this chunk final and the counts cleared (by wave 0, below)
      __syncthreads();
      if (valid && in_rank == 0) wave_cnt[wave][d] = __popcll(same);
      __syncthreads();
      if (valid) {
        int before = base[d];
        for (int w2 = 0; w2 < wave; ++w2) before += wave_cnt[w2][d];
        kb[before + in_rank] = key;
        ib[before + in_rank] = idx;
      }
      __syncthreads();
      // wave 0 alone advances the bases and then clears the counts: both in
      // its own program order, before the next chunk's first barrier
      if (wave == 0) {
        if (lane < kDigits) {
          int tot = 0;
#pragma unroll
          for (int w2 = 0; w2 < kRankWaves; ++w2) tot += wave_cnt[w2][lane];
          base[lane] += tot;
        }
        for (int e = lane; e < kRankWaves * kDigits; e += kWave) (&wave_cnt[0][0])[e] = 0;
      }
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

constexpr int kChunk = 1024;  // queries swept by one wave

// One wave per (row, chunk of kChunk queries).  The state before the chunk's
// first query q0 is found directly: with c = |E(q0 - 1)| eligible tokens,
// the cutoff is the largest eligible rank while c <= k (needed once c reaches
// k), else the rank of the k-th best eligible token: the k-th rank r in
// order whose token pos[r] <= q0 - 1 - w, counted 64 ranks at a time with
// ballots.  The chunk then runs the sequential update: a new token ranked
// below the cutoff moves it down to the next rank whose token is eligible.
template <bool kWindowWalk>
__global__ __launch_bounds__(256) void cutoff_kernel(CutoffArgs a, int rows, int n_chunks) {
  // wave-uniform state lives in scalar registers (readfirstlane tells the
  // compiler so), and the sweep's branches are scalar
  const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int row = gw / n_chunks;
  if (row >= rows) return;
  const int chunk = gw - row * n_chunks;
  const int lane = threadIdx.x & 63;
  const int S = a.S, s = a.s, w = a.window, k = a.top_k, n = S - s;
  const int32_t* __restrict__ rk = a.rank + (size_t)row * S;
  const uint32_t* __restrict__ pos = a.ws + (size_t)row * 5 * n;
  int32_t* __restrict__ out = a.cutoff + (size_t)row * S;
  const int q_begin = chunk * kChunk;
  const int q_end = min(S, q_begin + kChunk);
  if (k == 0) {
    for (int q = q_begin + lane; q < q_end; q += 64) out[q] = -1;
    return;
  }

  // state after the queries before q_begin
  int eligible = max(0, min(n, q_begin - w - s));  // tokens s .. q_begin - 1 - w
  int tau = -1;
  if (eligible > 0 && eligible <= k) {
    int mx = -1;
    for (int t = s + lane; t < s + eligible; t += 64) mx = max(mx, rk[t]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off));
    tau = __builtin_amdgcn_readfirstlane(mx);
  } else if (eligible > k) {
    const int last = q_begin - 1 - w;  // eligible tokens are s .. last
    int seen = 0;
    tau = n - 1;  // not reached: more than k ranks qualify
    constexpr int kAhead = 8;  // 64-rank groups whose positions are loaded together
    bool found = false;
    for (int r0 = 0; r0 < n && !found; r0 += 64 * kAhead) {
      uint32_t pv[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) {
        const int r = r0 + 64 * u + lane;
        pv[u] = r < n ? pos[r] : 0xFFFFFFFFu;
      }
#pragma unroll
      for (int u = 0; u < kAhead; ++u) {
        if (found) break;
        const bool ok = (int)pv[u] <= last && pv[u] != 0xFFFFFFFFu;
        const uint64_t bal = __ballot(ok);
        const int cnt = __popcll(bal);
        if (seen + cnt >= k) {
          const int need = k - seen;  // 1-based position among this group's hits
          const int upto = __popcll(bal & (~0ull >> (63 - lane)));
          const uint64_t hit = __ballot(ok && upto == need);
          tau = __builtin_amdgcn_readfirstlane(r0 + 64 * u + (int)__builtin_ctzll(hit));
          found = true;
        }
        seen += cnt;
      }
    }
  }

  // Positions of the ranks [pchunk, pchunk + 64) are held in lanes; the
  // window walk also loads the window below ahead of use.  Ranks outside
  // [0, n) hold 0 and are never tested.
  auto load_win = [&](int base) __attribute__((always_inline)) {
    const int r = base + lane;
    return (r >= 0 && r < n) ? pos[r] : 0u;
  };
  int pchunk = 1 << 30, pnext_base = -(1 << 30);  // no window yet
  uint32_t plane = 0, pnext = 0;
  for (int q0 = q_begin; q0 < q_end; q0 += 64) {
    // ranks of the tokens that enter at q0 .. q0 + 63 (t = q - w), -2 if none
    const int t_l = q0 + lane - w;
    const int r_l = (t_l >= s && t_l < S && q0 + lane < q_end) ? rk[t_l] : -2;
    int my_out = 0;
    const int nq = min(64, q_end - q0);
    for (int j = 0; j < nq; ++j) {
      const int q = q0 + j;
      const int r_new = __builtin_amdgcn_readlane(r_l, j);
      if (r_new >= 0) {
        ++eligible;
        if (eligible <= k) {
          tau = max(tau, r_new);
        } else if (r_new < tau) {
          // The new cutoff: the largest rank in (r_new, tau) whose token is
          // already eligible (pos <= q - w), else r_new itself (the new token
          // qualifies).
          if constexpr (kWindowWalk) {
            // long walks (k << n): 64 ranks per ballot, from the top window
            // down
            int hi_r = tau, result = r_new;
            for (;;) {
              const int want = hi_r - 1;  // highest untested rank
              if (want <= r_new) break;
              if (want < pchunk || want >= pchunk + 64) {
                if (want >= pnext_base && want < pnext_base + 64) {  // the window loaded ahead
                  pchunk = pnext_base;
                  plane = pnext;
                } else {  // place the window to end at want
                  pchunk = max(0, want - 63);
                  plane = load_win(pchunk);
                }
                pnext_base = pchunk - 64;
                pnext = load_win(pnext_base);
              }
              const int r = pchunk + lane;
              const uint64_t hit = __ballot(r > r_new && r < hi_r && r < n && (int)plane <= q - w);
              if (hit) {
                result = pchunk + 63 - (int)__builtin_clzll(hit);
                break;
              }
              hi_r = pchunk;  // nothing in [pchunk, hi_r)
              if (pchunk <= 0) break;
            }
            tau = result;
          } else {
            // short walks: rank by rank; the walk ends at r_new at the latest
            // (also the loop bound)
            for (;;) {
              --tau;
              if (tau <= r_new) break;
              if (tau < pchunk) {
                pchunk = max(0, tau - 63);
                plane = load_win(pchunk);
              }
              const int p = (int)__builtin_amdgcn_readlane((int)plane, tau - pchunk);
              if (p <= q - w) break;
            }
          }
        }
      }
      const int c = eligible < k ? S : tau;
      my_out = lane == j ? c : my_out;
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
  const int n_chunks = (S + kChunk - 1) / kChunk;
  const int64_t waves = rows * n_chunks;
  // The walk from one cutoff to the next crosses about n / k ranks per step
  // once k tokens are eligible: long walks test 64 ranks per ballot, short
  // ones go rank by rank.
  const int64_t n = S > n_sink ? (int64_t)S - n_sink : 0;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  if ((int64_t)top_k * 8 <= n)
    hipLaunchKernelGGL(cutoff_kernel<true>, grid, block, 0, stream, a, (int)rows, n_chunks);
  else
    hipLaunchKernelGGL(cutoff_kernel<false>, grid, block, 0, stream, a, (int)rows, n_chunks);
  return hipGetLastError();
}

}  // namespace kvp
