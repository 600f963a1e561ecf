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
//   cutoff_kernel  one wave per chunk of 1024 queries of a row, in groups
//                  of 64.  Its first state is counted directly from the
//                  ranks.  Groups with fewer than k eligible tokens keep all.
//                  Past k, the cutoff never rises (a new token can only push
//                  the k-th best to a better rank): each lane (query) counts
//                  down from the group's first cutoff to its own k-th best
//                  over a window of ranks (see the group step below), or,
//                  where the window is too shallow, a new token ranked below
//                  the cutoff moves it down to the next rank whose token is
//                  already eligible (pos[r] <= q - w), token by token with
//                  uniform control flow; when k << n those walks are long
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
// the digit histograms of all eight passes; each pass then reorders the keys
// chunk by chunk, kRows elements per thread (element c + 1024 e + thread of
// chunk c).  An element's place among the chunk's equal digits is the count
// of equal digits earlier in the chunk (earlier rows, and earlier waves of
// its row: one exclusive scan per digit over the chunk's (row, wave) counts,
// wave d scanning digit d) + its rank among equal digits in its wave (four
// ballots give the lanes with the same digit).  The chunk is first ordered by
// digit in LDS and then written out in that order, so each digit's run is
// one contiguous, coalesced store.  Passes whose digit is the same for every
// key are skipped.  The inverse permutation rank[pos[r]] = r is assembled in
// LDS, a window of tokens at a time, and stored contiguously.
constexpr int kRows = 4;
constexpr int kChunkElems = kRows * kRankThreads;
constexpr int kBatch = 8;        // global loads per thread in flight in the copy loops
constexpr int kHistCopies = 4;   // histogram copies per wave (lane % 4): fewer same-address atomics
constexpr int kRankWindow = 8192;       // tokens per LDS window of the inverse permutation
constexpr int kRankWindowsMax = 4;      // longer rows scatter the ranks directly
// one LDS buffer: the histogram copies, then a chunk's keys and indices, then
// a window of ranks
constexpr int kBigWords = kRankWindow > 2 * kChunkElems ? kRankWindow : 2 * kChunkElems;
static_assert(kBigWords >= kRankWaves * kHistCopies * kPasses * kDigits, "histogram copies fit");
static_assert(kRows * kRankWaves == kWave && kDigits == kRankWaves,
              "one wave per digit scans the chunk's (row, wave) counts across its lanes");
// Barrier for LDS traffic only: the global loads and stores in flight (the
// next chunk's keys, the last chunk's stores) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__global__ __launch_bounds__(kRankThreads, 8) void rank_kernel(CutoffArgs a) {
  __shared__ uint32_t big[kBigWords];
  __shared__ int hist[kPasses][kDigits];
  __shared__ int cnt[kDigits][kRows * kRankWaves];  // per digit: count of each (row, wave)
  __shared__ int loc[kDigits][kRows * kRankWaves];  // per digit: equal digits before each (row, wave)
  __shared__ int tot[kDigits];                      // per digit: count in the chunk
  __shared__ int base[2][kDigits];                  // per digit: first output slot (by chunk parity)
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

  // ---- digit histograms of all passes
  int* whist = reinterpret_cast<int*>(big);  // [wave][copy][pass][digit]
  for (int i = tid; i < kRankWaves * kHistCopies * kPasses * kDigits; i += kRankThreads) whist[i] = 0;
  for (int t = tid; t < s; t += kRankThreads) rk[t] = -1;
  __syncthreads();
  int* my_hist = whist + (wave * kHistCopies + (lane & (kHistCopies - 1))) * kPasses * kDigits;
  for (int i0 = tid; i0 < n; i0 += kBatch * kRankThreads) {
    float mv[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u * kRankThreads;
      mv[u] = i < n ? m[s + i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u * kRankThreads;
      if (i < n) {
        const uint32_t key = order_key(mv[u]);
        ka[i] = key;
        ia[i] = (uint32_t)(s + i);
#pragma unroll
        for (int p = 0; p < kPasses; ++p)
          atomicAdd(&my_hist[p * kDigits + ((key >> (kDigitBits * p)) & (kDigits - 1))], 1);
      }
    }
  }
  __syncthreads();
  if (tid < kPasses * kDigits) {
    int t = 0;
    for (int c = 0; c < kRankWaves * kHistCopies; ++c) t += whist[c * kPasses * kDigits + tid];
    (&hist[0][0])[tid] = t;
  }
  __syncthreads();

  // ---- the passes
  uint32_t* lk = big;                // a chunk's keys, ordered by digit
  uint32_t* li = big + kChunkElems;  // and their token indices
  for (int i = tid; i < kDigits * kRows * kRankWaves; i += kRankThreads) (&cnt[0][0])[i] = 0;
  for (int p = 0; p < kPasses; ++p) {
    const int shift = kDigitBits * p;
    bool trivial = false;
#pragma unroll
    for (int d = 0; d < kDigits; ++d) trivial |= hist[p][d] == n;
    if (trivial || n == 0) continue;  // uniform: the order does not change
    if (tid < kDigits) {
      int acc = 0;
      for (int d = 0; d < tid; ++d) acc += hist[p][d];
      base[0][tid] = acc;
    }
    // the next chunk's keys and indices are loaded while this one is reordered
    uint32_t nkey[kRows], nidx[kRows];
#pragma unroll
    for (int e = 0; e < kRows; ++e) {
      const int i = e * kRankThreads + tid;
      nkey[e] = i < n ? ka[i] : 0u;
      nidx[e] = i < n ? ia[i] : 0u;
    }
    int par = 0;
    for (int c = 0; c < n; c += kChunkElems, par ^= 1) {
      uint32_t key[kRows], idx[kRows];
      int dig[kRows], in_rank[kRows];
      uint64_t same[kRows];
#pragma unroll
      for (int e = 0; e < kRows; ++e) {
        const int i = c + e * kRankThreads + tid;
        key[e] = nkey[e];
        idx[e] = nidx[e];
        if (i + kChunkElems < n) {
          nkey[e] = ka[i + kChunkElems];
          nidx[e] = ia[i + kChunkElems];
        }
        const bool valid = i < n;
        dig[e] = (int)((key[e] >> shift) & (kDigits - 1));
        same[e] = __ballot(valid);
#pragma unroll
        for (int bbit = 0; bbit < kDigitBits; ++bbit) {
          const uint64_t bal = __ballot(valid && ((dig[e] >> bbit) & 1));
          same[e] &= ((dig[e] >> bbit) & 1) ? bal : ~bal;
        }
        in_rank[e] = __popcll(same[e] & lt_mask);
      }
      // the previous chunk has read its counts (cleared them), its places and
      // its LDS keys
      lds_barrier();
#pragma unroll
      for (int e = 0; e < kRows; ++e)
        if (c + e * kRankThreads + tid < n && in_rank[e] == 0)
          cnt[dig[e]][e * kRankWaves + wave] = __popcll(same[e]);
      lds_barrier();
      {
        // wave d: exclusive scan of digit d's counts over the chunk's
        // (row, wave) pairs in element order
        const int d = wave;
        const int v = cnt[d][lane];
        cnt[d][lane] = 0;
        int incl = v;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const int u = __shfl_up(incl, off);
          if (lane >= off) incl += u;
        }
        loc[d][lane] = incl - v;
        if (lane == kWave - 1) tot[d] = incl;
      }
      lds_barrier();
      // every wave: the chunk's digit runs start at lstart[d] in LDS and go to
      // base[d] + (place - lstart[d]) in the output (lanes d < 16 hold digit d)
      int lstart = 0, delta = 0;
      {
        const int t = lane < kDigits ? tot[lane] : 0;
        int incl = t;
#pragma unroll
        for (int off = 1; off < kDigits; off <<= 1) {
          const int u = __shfl_up(incl, off);
          if (lane >= off) incl += u;
        }
        lstart = incl - t;
        const int b = lane < kDigits ? base[par][lane] : 0;
        delta = b - lstart;
        if (wave == 0 && lane < kDigits) base[par ^ 1][lane] = b + t;
      }
#pragma unroll
      for (int e = 0; e < kRows; ++e) {
        // (the shuffle runs on every lane: a lane past the row still holds
        // a digit's start for the others)
        const int ls = __shfl(lstart, dig[e]);
        if (c + e * kRankThreads + tid < n) {
          const int place = ls + loc[dig[e]][e * kRankWaves + wave] + in_rank[e];
          lk[place] = key[e];
          li[place] = idx[e];
        }
      }
      lds_barrier();
      const int len = min(kChunkElems, n - c);
#pragma unroll
      for (int e = 0; e < kRows; ++e) {
        const int place = e * kRankThreads + tid;
        const uint32_t k2 = place < len ? lk[place] : 0u;
        const int d = (int)((k2 >> shift) & (kDigits - 1));
        const int slot = __shfl(delta, d) + place;
        if (place < len) {
          kb[slot] = k2;
          ib[slot] = li[place];
        }
      }
    }
    __syncthreads();
    uint32_t* tk = ka; ka = kb; kb = tk;
    uint32_t* ti = ia; ia = ib; ib = ti;
  }

  // ---- pos[r] = token of rank r; rank[token] = r
  const int n_windows = (n + kRankWindow - 1) / kRankWindow;
  if (n_windows > kRankWindowsMax) {
    for (int r0 = tid; r0 < n; r0 += kBatch * kRankThreads) {
      uint32_t tv[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int r = r0 + u * kRankThreads;
        tv[u] = r < n ? ia[r] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int r = r0 + u * kRankThreads;
        if (r < n) {
          pos[r] = tv[u];
          rk[tv[u]] = r;
        }
      }
    }
    return;
  }
  int* wrank = reinterpret_cast<int*>(big);
  for (int wdw = 0; wdw < n_windows; ++wdw) {
    const int t_lo = s + wdw * kRankWindow;  // tokens [t_lo, t_lo + kRankWindow)
    for (int r0 = tid; r0 < n; r0 += kBatch * kRankThreads) {
      uint32_t tv[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int r = r0 + u * kRankThreads;
        tv[u] = r < n ? ia[r] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int r = r0 + u * kRankThreads;
        if (r < n) {
          if (wdw == 0) pos[r] = tv[u];
          const int o = (int)tv[u] - t_lo;
          if (o >= 0 && o < kRankWindow) wrank[o] = r;
        }
      }
    }
    __syncthreads();
    const int w_len = min(kRankWindow, S - t_lo);
    for (int o = tid; o < w_len; o += kRankThreads) rk[t_lo + o] = wrank[o];
    __syncthreads();
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
constexpr int kDepth = 256;      // ranks below the cutoff a group step examines at most
constexpr int kBackoffMax = 64;  // most groups swept token by token after too-deep ones
template <bool kWindowWalk>
__global__ __launch_bounds__(256) void cutoff_kernel(CutoffArgs a, int rows, int n_chunks) {
  // per wave: the query within the current group at which each of the
  // kDepth ranks below the cutoff becomes eligible
  __shared__ int t_enter[4][kDepth];
  // wave-uniform state lives in scalar registers (readfirstlane tells the
  // compiler so), and the sweep's branches are scalar
  const int gw = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  const int row = gw / n_chunks;
  if (row >= rows) return;
  const int chunk = gw - row * n_chunks;
  const int lane = threadIdx.x & 63;
  const int wave_in_wg = threadIdx.x >> 6;
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
  int vec_skip = 0, backoff = 4;  // groups left to sweep token by token, and the next such run
  uint32_t plane = 0, pnext = 0;
  // The cutoff after a new token ranked r_new < tau enters at query q (more
  // than k eligible): the largest rank in (r_new, tau) whose token is
  // already eligible (pos <= q - w), else r_new itself (the new token
  // qualifies).
  auto walk = [&](int r_new, int q) __attribute__((always_inline)) {
    if constexpr (kWindowWalk) {
      // long walks (k << n): 64 ranks per ballot, from the top window down
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
  };
  for (int q0 = q_begin; q0 < q_end; q0 += 64) {
    // ranks of the tokens that enter at q0 .. q0 + 63 (t = q - w), -2 if none
    const int t_l = q0 + lane - w;
    const int r_l = (t_l >= s && t_l < S && q0 + lane < q_end) ? rk[t_l] : -2;
    const int nq = min(64, q_end - q0);
    const int n_new = __popcll(__ballot(r_l >= 0));
    if (eligible + n_new < k) {
      // fewer than k eligible through the whole group: every query keeps
      // all (cutoff S), and tau is the largest eligible rank so far
      int mx = r_l;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off));
      tau = max(tau, __builtin_amdgcn_readfirstlane(mx));
      eligible += n_new;
      if (lane < nq) out[q0 + lane] = S;
      continue;
    }
    int my_out = 0;
    if (eligible >= k) {
      // More than k eligible at every new token.  The cutoff c0 at the
      // group's start is the k-th best eligible rank; at query j the k-th
      // best is then the one with m_j eligible ranks between it and c0, m_j
      // the new tokens ranked below c0 up to query j (each pushes the k-th
      // place down by one).  Each lane (query) counts the eligible ranks
      // down from c0 over a window of kDepth ranks, with the query at which
      // each enters; if some query's answer lies deeper, the group is swept
      // token by token instead, and so are the next few groups (4, doubling
      // while the windows stay too shallow, at most kBackoffMax).
      const uint64_t below = __ballot(r_l >= 0 && r_l < tau);
      bool done = below == 0;  // no new token moves the cutoff
      if (done) {
        my_out = tau;
      } else if (vec_skip > 0) {
        --vec_skip;
      } else {
        const int c0 = tau;
        const int m = __popcll(below & ((2ull << lane) - 1));  // through this lane's query
        int hits_last = 0;  // ranks of the window eligible at the group's last query
#pragma unroll
        for (int u = 0; u < kDepth / 64; ++u) {
          const int r = c0 - 64 * u - lane;
          int t = 1 << 20;  // not eligible within the group
          if (r >= 0) {
            const int j = (int)pos[r] + w - q0;  // the query at which its token enters
            t = j < 0 ? -1 : (j < nq ? j : 1 << 20);
          }
          t_enter[wave_in_wg][64 * u + lane] = t;
          hits_last += __popcll(__ballot(t <= nq - 1));
        }
        // the last query needs m + 1 eligible ranks in the window
        const int m_last = __popcll(below);
        int cnt = 0, res = -1;  // eligible ranks passed; the answer's depth
        for (int i0 = 0; i0 < kDepth && hits_last > m_last; i0 += 16) {
#pragma unroll
          for (int ii = 0; ii < 16; ++ii) {
            const bool hit = t_enter[wave_in_wg][i0 + ii] <= lane;
            res = (hit && cnt == m && res < 0) ? i0 + ii : res;
            cnt += hit ? 1 : 0;
          }
          if (!__any(res < 0 && lane < nq)) break;
        }
        if (hits_last > m_last && !__any(res < 0 && lane < nq)) {
          my_out = c0 - res;
          tau = __builtin_amdgcn_readlane(c0 - res, nq - 1);
          done = true;
          backoff = 4;
        } else {
          vec_skip = backoff;
          backoff = min(2 * backoff, kBackoffMax);
        }
      }
      // otherwise only a token ranked below the current cutoff moves it: the
      // sweep jumps from one such token to the next (a ballot against the
      // cutoff of the moment), the queries in between keeping it
      int j = 0;
      while (!done) {
        const uint64_t upd = __ballot(lane >= j && r_l >= 0 && r_l < tau);
        const int jj = upd ? (int)__builtin_ctzll(upd) : nq;
        my_out = (lane >= j && lane < jj) ? tau : my_out;
        if (jj >= nq) break;
        walk(__builtin_amdgcn_readlane(r_l, jj), q0 + jj);
        my_out = lane == jj ? tau : my_out;
        j = jj + 1;
      }
      eligible += n_new;
    } else {
      for (int j = 0; j < nq; ++j) {
        const int r_new = __builtin_amdgcn_readlane(r_l, j);
        if (r_new >= 0) {
          ++eligible;
          if (eligible <= k)
            tau = max(tau, r_new);
          else if (r_new < tau)
            walk(r_new, q0 + j);
        }
        const int c = eligible < k ? S : tau;
        my_out = lane == j ? c : my_out;
      }
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
