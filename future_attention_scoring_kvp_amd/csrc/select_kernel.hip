// Per-KV-head keep-set for gfx950.
//
//   keep = ascending( sinks [0, min(s, S))  U  window [max(0, S - w), S)
//                     U  top-k of score over the eligible range [s, S - w) )
// KVpop Fig. 1 / §3 Eq. 1 (budget s + w + k per KV head) and Eq. 4 (eligible
// set at the last query).  The scores are future masses or any fp32 score
// (e.g. the log targets, which are negative).  Ranking: score descending,
// equal scores by ascending index.
//
// Both paths work in two steps:
//   1. radix select, most significant digit first, on an order-preserving
//      32-bit key of each fp32 score (any sign; see score_key): histograms of
//      the candidates that match the digits fixed so far give the k-th
//      largest value T exactly and the number r of copies of T that belong to
//      the top-k (the r lowest-indexed ones);
//   2. ordered emission: position j is kept iff it is a sink or in the
//      window, or its key is above T, or it is among the first r copies of T;
//      its output slot is the number of kept positions before it, so the
//      output is ascending with no sort.
// Rows of up to 32768 scores (select_reg_kernel, one 1024-thread workgroup
// per row): each thread holds KPT consecutive keys in registers, so the row
// is read from memory once; four 8-bit passes histogram from registers into
// per-wave LDS copies, and one block-wide scan of (kept, tie) counts places
// every kept position.
// Longer rows are split into chunks of 4096 or more positions, one 256-thread
// workgroup per (row, chunk), with the per-chunk integer state in a caller
// workspace (deterministic: integer counts, fixed reduction order):
//   sel_hist_kernel     per chunk, a 2048-bin histogram of key bits 31..21,
//                       stored as suffix counts (keys in that bin or above);
//   sel_bin_kernel      per row, the bin b1 of the k-th largest key (from the
//                       summed chunk suffix counts), the count of keys above
//                       b1 per chunk and each chunk's offset into the
//                       candidate list (the keys in bin b1);
//   sel_compact_kernel  per chunk, its keys in bin b1 into its segment of the
//                       candidate list;
//   sel_finish_kernel   per row, two more radix passes (bits 20..10, 9..0)
//                       over the candidates give T and r; per chunk, the kept
//                       and tie counts before it;
//   sel_emit_kernel     per chunk, flags, a block scan and the stores.
#include <mutex>

#include "kvp_device.h"
#include "kvp_launch.h"

namespace kvp {
namespace {

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

// ---- rows of up to kRegThreads * KPT scores: keys held in registers

constexpr int kRegThreads = 1024;
constexpr int kRegWaves = kRegThreads / kWave;

template <int KPT>
__global__ __launch_bounds__(kRegThreads) void select_reg_kernel(SelArgs a, bool vec4) {
  static_assert(KPT % 4 == 0 && KPT <= 32 && kRegThreads * KPT <= 32768,
                "packed 16-bit counts need rows of at most 32768 scores");
  constexpr int kChunks = KPT / 4;               // chunks of 4 * kRegThreads positions
  constexpr int kChunkLen = 4 * kRegThreads;
  // Histogram copies per (wave, lane group): lanes of a wave whose keys share
  // a digit add to kSub different words (different banks), which cuts the
  // serialised collisions of skewed rows.  They live in the keep-list buffer,
  // which is free until the emission.
  constexpr int kSub = KPT / 4;  // 2, 4 or 8 lane groups: exactly the buffer
  static_assert(kRegWaves * 256 * kSub == kRegThreads * KPT, "histogram copies fill the keep-list buffer");
  __shared__ __attribute__((aligned(16))) int hist[4][256];  // merged partial counts
  __shared__ uint32_t wave_sum[kChunks][kRegWaves];
  __shared__ uint32_t sel_digit;
  __shared__ int sel_above;
  __shared__ __attribute__((aligned(16))) int32_t out_lds[kRegThreads * KPT];  // the row's keep list, written out coalesced

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int S = a.S;
  const float* __restrict__ m = a.mass + (size_t)blockIdx.x * S;
  int32_t* __restrict__ out = a.keep + (size_t)blockIdx.x * a.n_keep;

  const int e_lo = a.n_sink;                 // eligible range [e_lo, e_hi)
  const int e_hi = S - a.window;             // may be <= e_lo (empty)
  const int n_elig = e_hi > e_lo ? e_hi - e_lo : 0;
  const int kk = a.top_k < n_elig ? a.top_k : n_elig;
  const bool take_all = kk == n_elig;

  // Element e of this thread is position pos(e): chunk e / 4, four
  // consecutive positions per thread within a chunk, so every load
  // instruction of a wave reads 1 KB of consecutive scores.  Positions >= S
  // hold key 0 and take part in nothing.
  auto pos = [&](int e) __attribute__((always_inline)) {
    return (e >> 2) * kChunkLen + 4 * tid + (e & 3);
  };
  uint32_t key[KPT];
  if (vec4) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int j = c * kChunkLen + 4 * tid;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < S) v = *reinterpret_cast<const float4*>(m + j);  // S % 4 == 0
      key[4 * c] = score_key(v.x);
      key[4 * c + 1] = score_key(v.y);
      key[4 * c + 2] = score_key(v.z);
      key[4 * c + 3] = score_key(v.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < KPT; ++e) key[e] = pos(e) < S ? score_key(m[pos(e)]) : 0u;
  }

  // --- 1. threshold T and tie count r (only when 0 < kk < n_elig)
  uint32_t prefix = 0, pmask = 0;
  int r = kk;
  if (!take_all && kk > 0) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      int* const sh = out_lds;  // [wave][bin][lane group]
      for (int i = 4 * tid; i < kRegWaves * 256 * kSub; i += 4 * kRegThreads)
        *reinterpret_cast<int4*>(sh + i) = make_int4(0, 0, 0, 0);
      __syncthreads();
      const int sub = lane & (kSub - 1);
#pragma unroll
      for (int e = 0; e < KPT; ++e) {
        const int j = pos(e);
        if (j >= e_lo && j < e_hi && (key[e] & pmask) == prefix)
          atomicAdd(&sh[(wave * 256 + (int)((key[e] >> shift) & 255u)) * kSub + sub], 1);
      }
      __syncthreads();
      {  // merge: thread t adds the copies of bin t % 256 from a quarter of the waves
        const int bin = tid & 255, part = tid >> 8;
        int t = 0;
#pragma unroll
        for (int w = 4 * part; w < 4 * part + 4; ++w)
#pragma unroll
          for (int u = 0; u < kSub; ++u) t += sh[(w * 256 + bin) * kSub + u];
        hist[part][bin] = t;
      }
      __syncthreads();
      if (tid < 256) hist[0][tid] += hist[1][tid] + hist[2][tid] + hist[3][tid];  // its own column
      __syncthreads();
      if (wave == 0) {
        // lane l owns bins 4l .. 4l + 3; counts from the top bin down
        const int4 c4 = *reinterpret_cast<const int4*>(&hist[0][4 * lane]);
        const int c[4] = {c4.x, c4.y, c4.z, c4.w};
        const int own = c[0] + c[1] + c[2] + c[3];
        int suf = own;  // candidates in bins >= 4 lane
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const int o = __shfl_down(suf, off);
          if (lane + off < kWave) suf += o;
        }
        const int above = suf - own;  // candidates in bins > 4 lane + 3
        // the digit d is the largest with (count in bins > d) < r <= (count
        // in bins >= d); exactly one lane holds it (r >= 1, total >= r)
        if (above < r && r <= suf) {
          int acc = above, d = 4 * lane + 3;
#pragma unroll
          for (int i = 3; i > 0; --i) {
            if (acc + c[i] >= r) break;
            acc += c[i];
            --d;
          }
          sel_digit = (uint32_t)d;
          sel_above = acc;
        }
      }
      __syncthreads();
      prefix |= sel_digit << shift;
      pmask |= 255u << shift;
      r -= sel_above;
    }
  }
  const uint32_t T = prefix;

  // --- 2. ordered emission.  Per position: forced-or-above (sink, window,
  // key > T, or every eligible one when all are taken) or a tie (key == T),
  // as one bit each.  Kept before position j = (forced-or-above before j) +
  // min(ties before j, r).
  uint32_t fa_bits = 0, tie_bits = 0;
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    const int j = pos(e);
    bool fa = false, tie = false;
    if (j < S) {
      if (j < a.n_sink || j >= e_hi) {
        fa = true;
      } else if (kk > 0) {
        fa = take_all || key[e] > T;
        tie = !take_all && key[e] == T;
      }
    }
    fa_bits |= (uint32_t)fa << e;
    tie_bits |= (uint32_t)tie << e;
  }
  // Counts before each (chunk, thread) in position order: per chunk, an
  // in-wave inclusive scan of (forced-or-above << 16 | ties), unsigned (row
  // totals of either count are at most 32768, so the tie half never
  // carries); then one wave turns the (chunk, wave) totals into exclusive
  // offsets.
  uint32_t packed[kChunks], incl[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const uint32_t nib = 0xFu << (4 * c);
    packed[c] = ((uint32_t)__popc(fa_bits & nib) << 16) | (uint32_t)__popc(tie_bits & nib);
    uint32_t x = packed[c];
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const uint32_t o = __shfl_up(x, off);
      if (lane >= off) x += o;
    }
    incl[c] = x;
    if (lane == kWave - 1) wave_sum[c][wave] = x;
  }
  __syncthreads();
  constexpr int kTot = kChunks * kRegWaves;  // <= 128 (chunk, wave) totals
  static_assert(kTot <= 2 * kWave, "one wave scans the totals, two per lane");
  uint32_t total = 0;
  if (wave == 0) {
    uint32_t* flat = &wave_sum[0][0];
    const uint32_t v0 = 2 * lane < kTot ? flat[2 * lane] : 0u;
    const uint32_t v1 = 2 * lane + 1 < kTot ? flat[2 * lane + 1] : 0u;
    uint32_t x = v0 + v1;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const uint32_t o = __shfl_up(x, off);
      if (lane >= off) x += o;
    }
    const uint32_t ex = x - v0 - v1;
    if (2 * lane < kTot) flat[2 * lane] = ex;
    if (2 * lane + 1 < kTot) flat[2 * lane + 1] = ex + v0;
  }
  __syncthreads();
  // kept positions in the row: forced-or-above + min(ties, r), from the last
  // (chunk, wave) offset plus that wave's totals
  {
    const uint32_t last = wave_sum[kChunks - 1][kRegWaves - 1];
    const uint32_t t = __shfl(incl[kChunks - 1], kWave - 1);
    total = wave == kRegWaves - 1 ? last + t : 0u;
  }
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const uint32_t base = wave_sum[c][wave] + incl[c] - packed[c];
    int fa_before = (int)(base >> 16);
    int tie_before = (int)(base & 0xFFFFu);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * c + q;
      const bool fa = (fa_bits >> e) & 1u;
      const bool tie = (tie_bits >> e) & 1u;
      if (fa || (tie && tie_before < r)) {
        const int slot = fa_before + min(tie_before, r);
        if (slot < a.n_keep) out_lds[slot] = pos(e);
      }
      fa_before += fa;
      tie_before += tie;
    }
  }
  // the last wave knows the row's kept count; publish it through sel_above
  if (wave == kRegWaves - 1 && lane == 0) {
    const int n_fa = (int)(total >> 16), n_tie = (int)(total & 0xFFFFu);
    sel_above = n_fa + min(n_tie, r);
  }
  __syncthreads();
  const int n_out = min((int64_t)sel_above, a.n_keep);
  for (int i = tid; i < n_out; i += kRegThreads) out[i] = out_lds[i];
}


// ---- rows split over several workgroups (state in the caller's workspace)

constexpr int kMbThreads = 256;
constexpr int kMbWaves = kMbThreads / kWave;
constexpr int kSubLen = 4 * kMbThreads;     // positions per sub-chunk (one float4 per thread)
constexpr int kBins1 = 2048;                // digit 1: key bits 31..21
constexpr int kBins2 = 2048;                // digit 2: key bits 20..10
constexpr int kBins3 = 1024;                // digit 3: key bits 9..0
constexpr int kFinThreads = 1024;
constexpr int kFinWaves = kFinThreads / kWave;
constexpr int kCandLds = 32768;             // candidates held in LDS by sel_finish_kernel
constexpr int kStateInts = 8;               // per row: b1, k1, n_cand, T, r
constexpr int kMaxChunks = 256;             // chunks per row: one thread each in sel_bin_kernel
constexpr int kMinChunk = 4 * kSubLen;
static_assert(kMaxChunks <= kMbThreads, "sel_bin_kernel gives every chunk a thread");

// Selection of a row: 0 = no eligible token is taken (k = 0 or none
// eligible), 1 = every eligible token is taken, 2 = a real top-k.
enum { kTakeNone = 0, kTakeAll = 1, kSelect = 2 };

struct MbArgs {
  const float* mass;
  int32_t* keep;
  int S, window, n_sink, kk, mode;
  int nc, C;            // chunks per row, chunk length (a multiple of kSubLen)
  int64_t n_keep;
  bool vec4;            // rows are 16-byte aligned (S % 4 == 0)
  int32_t* hist;        // [rows][nc][kBins1]
  int32_t* chunk;       // [rows][nc][4]: keys above bin b1, candidate offset, kept base, tie base
  int32_t* state;       // [rows][kStateInts]
  uint32_t* cand;       // [rows][S] candidate keys, chunk segments in chunk order
};

// Four consecutive scores at position p of a row (p % 4 == 0); positions at
// or past S read 0 and are never eligible.
__device__ __forceinline__ void load4(const float* __restrict__ m, int p, int S, bool vec4,
                                      float v[4]) {
  if (vec4 && p + 3 < S) {
    const float4 x = *reinterpret_cast<const float4*>(m + p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = p + q < S ? m[p + q] : 0.f;
  }
}

// Positions kept whatever the scores (sinks and window) in [0, p), p <= S.
__device__ __forceinline__ int forced_before(int p, int S, int w, int s) {
  const int sp = min(s, S);
  const int wl = max(sp, S - w);  // first window position that is not a sink
  return min(p, sp) + max(0, p - wl);
}

// Sub-chunks whose loads are issued together before their keys are used.
constexpr int kBatch = 4;

// Exclusive prefix sum over the threads of a block and the block total;
// `tot` is LDS scratch of one int per wave.
template <int kWaves>
__device__ __forceinline__ int block_prefix_excl(int v, int* tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(x, off);
    if (lane >= off) x += o;
  }
  if (lane == kWave - 1) tot[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = tot[w];
    if (w < wave) before += t;
    total += t;
  }
  __syncthreads();
  return before + x - v;
}

// Per chunk: the count of its eligible keys in each bin of key bits 31..21
// and above, i.e. suf[b] = #{keys with bin >= b}, so that the per-row kernel
// reads any bin's count and the count above it with two loads.
__global__ __launch_bounds__(kMbThreads) void sel_hist_kernel(MbArgs a) {
  constexpr int kPer = kBins1 / kMbThreads;  // 8 bins per thread
  __shared__ int h[kMbWaves][kBins1];
  __shared__ int tot[kMbWaves];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int row = blockIdx.x / a.nc, c = blockIdx.x - row * a.nc;
  for (int i = tid; i < kMbWaves * kBins1; i += kMbThreads) (&h[0][0])[i] = 0;
  __syncthreads();
  const float* __restrict__ m = a.mass + (size_t)row * a.S;
  const int e_lo = a.n_sink, e_hi = a.S - a.window;
  const int p_end = min(a.S, (c + 1) * a.C);
  for (int p0 = c * a.C + 4 * tid; p0 < p_end; p0 += kBatch * kSubLen) {
    float v[kBatch][4];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) load4(m, p0 + u * kSubLen, a.S, a.vec4, v[u]);
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int p = p0 + u * kSubLen + q;
        if (p < p_end && p >= e_lo && p < e_hi) atomicAdd(&h[wave][score_key(v[u][q]) >> 21], 1);
      }
  }
  __syncthreads();
  int cnt[kPer], own = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = kPer * tid + i;
    cnt[i] = h[0][b] + h[1][b] + h[2][b] + h[3][b];
    own += cnt[i];
  }
  int total;
  const int excl = block_prefix_excl<kMbWaves>(own, tot, total);
  int suf = total - excl;  // keys in bins >= kPer * tid
  int out8[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    out8[i] = suf;
    suf -= cnt[i];
  }
  int4* out = reinterpret_cast<int4*>(a.hist + ((size_t)row * a.nc + c) * kBins1 + kPer * tid);
  out[0] = make_int4(out8[0], out8[1], out8[2], out8[3]);
  out[1] = make_int4(out8[4], out8[5], out8[6], out8[7]);
}

// Inclusive suffix sum over the threads of a block (thread t gets the sum of
// `v` over threads >= t); `tot` is LDS scratch of one int per wave.
template <int kWaves>
__device__ __forceinline__ int block_suffix(int v, int* tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_down(x, off);
    if (lane + off < kWave) x += o;
  }
  if (lane == 0) tot[wave] = x;
  __syncthreads();
  int later = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
    if (w > wave) later += tot[w];
  __syncthreads();
  return x + later;
}

// Digit search over per-thread bin counts: thread t owns bins [kPer t,
// kPer t + kPer).  Finds the digit d with (count above d) < r <= (count at or
// above d) and writes d and the count above it to *dig / *above.  r >= 1 and
// the total is >= r, so exactly one thread finds it.
template <int kWaves, int kPer>
__device__ __forceinline__ void find_digit(const int (&c)[kPer], int r, int* tot, int* dig,
                                           int* above) {
  int own = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) own += c[i];
  const int suf = block_suffix<kWaves>(own, tot);
  const int ab = suf - own;  // in bins above this thread's
  if (ab < r && r <= suf) {
    int acc = ab, d = kPer * (int)threadIdx.x + kPer - 1;
#pragma unroll
    for (int i = kPer - 1; i > 0; --i) {
      if (acc + c[i] >= r) break;
      acc += c[i];
      --d;
    }
    *dig = d;
    *above = acc;
  }
}

// Per row: the bin b1 of the k-th largest key (the largest bin with at least
// k keys at or above it), the keys above b1 in each chunk and each chunk's
// offset into the candidate list.  One 256-thread workgroup per row.
__global__ __launch_bounds__(kMbThreads) void sel_bin_kernel(MbArgs a) {
  constexpr int kPer = kBins1 / kMbThreads;  // 8 bins per thread
  __shared__ int tot[kMbWaves];
  __shared__ int first[kMbThreads];
  __shared__ int s_b1, s_above;
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int32_t* hist = a.hist + (size_t)row * a.nc * kBins1;
  if (tid == 0) {  // found by exactly one thread below; set for safety
    s_b1 = 0;
    s_above = 0;
  }
  // suffix counts of the row: the sum of the chunks' suffix counts
  int g[kPer] = {};
#pragma unroll 8
  for (int c = 0; c < a.nc; ++c) {
    const int4* p = reinterpret_cast<const int4*>(hist + (size_t)c * kBins1 + kPer * tid);
    const int4 x = p[0], y = p[1];
    g[0] += x.x; g[1] += x.y; g[2] += x.z; g[3] += x.w;
    g[4] += y.x; g[5] += y.y; g[6] += y.z; g[7] += y.w;
  }
  first[tid] = g[0];
  __syncthreads();
  const int next = tid + 1 < kMbThreads ? first[tid + 1] : 0;  // suffix count of bin kPer (tid + 1)
  // bin b is b1 iff suf[b] >= k > suf[b + 1]: exactly one bin, since suf is
  // non-increasing, suf[0] = eligible keys >= k and suf[2048] = 0 < k
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int nb = i + 1 < kPer ? g[i + 1] : next;
    if (g[i] >= a.kk && nb < a.kk) {
      s_b1 = kPer * tid + i;
      s_above = nb;
    }
  }
  __syncthreads();
  const int b1 = s_b1 & (kBins1 - 1);
  int32_t* st = a.state + (size_t)row * kStateInts;
  int32_t* ch = a.chunk + (size_t)row * a.nc * 4;
  // per chunk (one thread each, at most kMbThreads chunks): keys above b1 and
  // the candidates in b1, then the candidate offsets
  int cand = 0;
  if (tid < a.nc) {
    const int32_t* hc = hist + (size_t)tid * kBins1;
    const int above_c = b1 + 1 < kBins1 ? hc[b1 + 1] : 0;
    cand = hc[b1] - above_c;
    ch[4 * tid] = above_c;
  }
  int n_cand;
  const int off = block_prefix_excl<kMbWaves>(cand, tot, n_cand);
  if (tid < a.nc) ch[4 * tid + 1] = off;
  if (tid == 0) {
    st[0] = b1;
    st[1] = a.kk - s_above;  // rank of T among the candidates (1-based)
    st[2] = n_cand;          // candidates
  }
}

// Per chunk: its keys in bin b1 go to its segment of the candidate list (in
// any order inside the segment).
__global__ __launch_bounds__(kMbThreads) void sel_compact_kernel(MbArgs a) {
  __shared__ int n;
  const int tid = threadIdx.x, lane = tid & 63;
  const int row = blockIdx.x / a.nc, c = blockIdx.x - row * a.nc;
  if (tid == 0) n = 0;
  __syncthreads();
  const uint32_t b1 = (uint32_t)a.state[(size_t)row * kStateInts] & (kBins1 - 1);
  uint32_t* out = a.cand + (size_t)row * a.S + a.chunk[((size_t)row * a.nc + c) * 4 + 1];
  const float* __restrict__ m = a.mass + (size_t)row * a.S;
  const int e_lo = a.n_sink, e_hi = a.S - a.window;
  const int p_end = min(a.S, (c + 1) * a.C);
  // every lane of the block runs the same trip count (ballots below)
  for (int p0 = c * a.C; p0 < p_end; p0 += kBatch * kSubLen) {
    float v[kBatch][4];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) load4(m, p0 + u * kSubLen + 4 * tid, a.S, a.vec4, v[u]);
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int p = p0 + u * kSubLen + 4 * tid + q;
        const uint32_t key = score_key(v[u][q]);
        const bool is_c = p < p_end && p >= e_lo && p < e_hi && (key >> 21) == b1;
        const uint64_t bal = __ballot(is_c);
        if (bal == 0) continue;
        int base = 0;
        if (lane == 0) base = atomicAdd(&n, __popcll(bal));
        base = __shfl(base, 0);
        if (is_c) out[base + __popcll(bal & ((1ull << lane) - 1ull))] = key;
      }
  }
}

// Per row: T and r from the candidates, then the kept / tie bases of every
// chunk.  One 1024-thread workgroup per row.
__global__ __launch_bounds__(kFinThreads) void sel_finish_kernel(MbArgs a) {
  __shared__ uint32_t keys[kCandLds];
  __shared__ int h[kBins2];
  __shared__ int tot[kFinWaves];
  __shared__ int s_d, s_above;
  __shared__ int s_gt[kWave], s_eq[kWave];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  int32_t* st = a.state + (size_t)row * kStateInts;
  const uint32_t b1 = (uint32_t)st[0] & (kBins1 - 1);
  int r = st[1];
  const int n = min(st[2], a.S);
  const uint32_t* gk = a.cand + (size_t)row * a.S;
  const bool in_lds = n <= kCandLds;
  if (in_lds)
    for (int i = tid; i < n; i += kFinThreads) keys[i] = gk[i];
  const uint32_t* src = in_lds ? keys : gk;

  // digit 2 (bits 20..10) over all candidates, then digit 3 (bits 9..0) over
  // those that match it
  uint32_t prefix = b1 << 21;
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    const uint32_t pmask = pass == 0 ? 0xFFE00000u : 0xFFFFFC00u;
    const int nb = pass == 0 ? kBins2 : kBins3;
    for (int i = tid; i < kBins2; i += kFinThreads) h[i] = 0;
    if (tid == 0) {  // found by exactly one thread below; set for safety
      s_d = 0;
      s_above = 0;
    }
    __syncthreads();
    for (int i = tid; i < n; i += kFinThreads) {
      const uint32_t u = src[i];
      if ((u & pmask) == prefix) atomicAdd(&h[(u >> shift) & (uint32_t)(nb - 1)], 1);
    }
    __syncthreads();
    if (pass == 0) {
      int c2[2] = {h[2 * tid], h[2 * tid + 1]};
      find_digit<kFinWaves, 2>(c2, r, tot, &s_d, &s_above);
    } else {
      int c1[1] = {h[tid]};
      find_digit<kFinWaves, 1>(c1, r, tot, &s_d, &s_above);
    }
    __syncthreads();
    prefix |= (uint32_t)s_d << shift;
    r -= s_above;
    __syncthreads();
  }
  const uint32_t T = prefix;

  // per chunk: candidates above T and equal to T, one wave per chunk over its
  // segment; then the exclusive prefixes over chunks
  int32_t* ch = a.chunk + (size_t)row * a.nc * 4;
  const int S = a.S, w = a.window, s = a.n_sink;
  int fa_base = 0, tie_base = 0;
  for (int c0 = 0; c0 < a.nc; c0 += kWave) {
    const int nch = min(kWave, a.nc - c0);
    for (int cc = wave; cc < nch; cc += kFinWaves) {
      const int c = c0 + cc;
      const int lo = max(0, min(ch[4 * c + 1], n));
      const int hi = c + 1 < a.nc ? max(lo, min(ch[4 * c + 5], n)) : n;
      int gt = 0, eq = 0;
      for (int i = lo + lane; i < hi; i += kWave) {
        const uint32_t u = src[i];
        gt += u > T;
        eq += u == T;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        gt += __shfl_xor(gt, off);
        eq += __shfl_xor(eq, off);
      }
      if (lane == 0) {
        s_gt[cc] = gt;
        s_eq[cc] = eq;
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int c = c0 + lane;
      int fa = 0, eq = 0;
      if (lane < nch) {
        const int p_lo = c * a.C, p_hi = min(S, (c + 1) * a.C);
        fa = forced_before(p_hi, S, w, s) - forced_before(p_lo, S, w, s) + ch[4 * c] + s_gt[lane];
        eq = s_eq[lane];
      }
      int xf = fa, xe = eq;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int of = __shfl_up(xf, off), oe = __shfl_up(xe, off);
        if (lane >= off) {
          xf += of;
          xe += oe;
        }
      }
      if (lane < nch) {
        ch[4 * c + 2] = fa_base + xf - fa;
        ch[4 * c + 3] = tie_base + xe - eq;
      }
      fa_base += __shfl(xf, kWave - 1);
      tie_base += __shfl(xe, kWave - 1);
    }
    __syncthreads();
  }
  if (tid == 0) {
    st[3] = (int32_t)T;
    st[4] = r;
  }
}

// Per chunk: keep flags, a block scan in position order and the stores.
__global__ __launch_bounds__(kMbThreads) void sel_emit_kernel(MbArgs a) {
  __shared__ uint32_t tot[kMbWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x / a.nc, c = blockIdx.x - row * a.nc;
  const int S = a.S;
  const int e_lo = a.n_sink, e_hi = S - a.window;
  const float* __restrict__ m = a.mass + (size_t)row * S;
  int32_t* __restrict__ out = a.keep + (size_t)row * a.n_keep;
  uint32_t T = 0;
  int r = 0, fa_before, tie_before = 0;
  if (a.mode == kSelect) {
    const int32_t* st = a.state + (size_t)row * kStateInts;
    const int32_t* ch = a.chunk + ((size_t)row * a.nc + c) * 4;
    T = (uint32_t)st[3];
    r = st[4];
    fa_before = ch[2];
    tie_before = ch[3];
  } else if (a.mode == kTakeAll) {
    fa_before = c * a.C;
  } else {
    fa_before = forced_before(c * a.C, S, a.window, a.n_sink);
  }
  const int p_end = min(S, (c + 1) * a.C);
  float vb[kBatch][4];
  for (int p0 = c * a.C; p0 < p_end; p0 += kSubLen) {
    const int p = p0 + 4 * tid;
    // keys of the next kBatch sub-chunks, loaded together
    const int u = ((p0 - c * a.C) / kSubLen) % kBatch;
    if (a.mode == kSelect && u == 0) {
#pragma unroll
      for (int uu = 0; uu < kBatch; ++uu) load4(m, p + uu * kSubLen, S, a.vec4, vb[uu]);
    }
    bool fa[4], tie[4];
    if (a.mode == kSelect) {
      float v[4];
#pragma unroll
      for (int uu = 0; uu < kBatch; ++uu)  // v = vb[u] with a constant index
        if (uu == u) {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = vb[uu][q];
        }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = p + q;
        const bool elig = j >= e_lo && j < e_hi;
        const uint32_t key = score_key(v[q]);
        fa[q] = j < S && (!elig || key > T);
        tie[q] = elig && key == T;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = p + q;
        fa[q] = j < S && (a.mode == kTakeAll || j < e_lo || j >= e_hi);
        tie[q] = false;
      }
    }
    // (forced-or-above << 16 | ties) of this thread's four positions; the
    // sub-chunk totals are at most 1024, so the tie half never carries
    const uint32_t mine = ((uint32_t)(fa[0] + fa[1] + fa[2] + fa[3]) << 16) |
                          (uint32_t)(tie[0] + tie[1] + tie[2] + tie[3]);
    uint32_t x = mine;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const uint32_t o = __shfl_up(x, off);
      if (lane >= off) x += o;
    }
    if (lane == kWave - 1) tot[wave] = x;
    __syncthreads();
    uint32_t before = x - mine, all = 0;
#pragma unroll
    for (int wv = 0; wv < kMbWaves; ++wv) {
      const uint32_t t = tot[wv];
      if (wv < wave) before += t;
      all += t;
    }
    __syncthreads();
    int fb = fa_before + (int)(before >> 16);
    int tb = tie_before + (int)(before & 0xFFFFu);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (fa[q] || (tie[q] && tb < r)) {
        const int slot = fb + min(tb, r);
        if (slot < a.n_keep) out[slot] = p + q;
      }
      fb += fa[q];
      tb += tie[q];
    }
    fa_before += (int)(all >> 16);
    tie_before += (int)(all & 0xFFFFu);
  }
}

// Chunking of the split path: chunk length a multiple of kSubLen, at least
// 4096, aiming at about 1024 workgroups per launch and at most kMaxChunks
// chunks per row (the per-row kernels then read at most 2 MB of histograms).

void mb_plan(int64_t rows, int S, int& nc, int& C) {
  int64_t want = (1024 + rows - 1) / rows;
  const int64_t most = (S + kMinChunk - 1) / kMinChunk;
  if (want > most) want = most;
  if (want > kMaxChunks) want = kMaxChunks;
  if (want < 1) want = 1;
  int64_t len = (S + want - 1) / want;
  len = (len + kMinChunk - 1) / kMinChunk * kMinChunk;
  C = (int)len;
  nc = (int)((S + len - 1) / len);
  if (nc < 1) nc = 1;
}

// Rows longer than the register kernel holds take the split path.
bool use_split(int64_t, int S) { return S > 32768; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

int64_t select_split_blocks(int64_t rows, int S) {
  if (rows <= 0 || S <= 0 || !use_split(rows, S)) return 0;
  int nc, C;
  mb_plan(rows, S, nc, C);
  return rows * nc;
}

size_t select_workspace_bytes(int64_t rows, int S) {
  if (rows <= 0 || S <= 0 || !use_split(rows, S)) return 0;
  int nc, C;
  mb_plan(rows, S, nc, C);
  return align256((size_t)rows * nc * kBins1 * 4) + align256((size_t)rows * nc * 16) +
         align256((size_t)rows * kStateInts * 4) + align256((size_t)rows * S * 4);
}

hipError_t launch_select(const float* mass, int64_t rows, int S, int window, int n_sink,
                         int top_k, int64_t n_keep, int32_t* keep, void* workspace,
                         hipStream_t stream) {
  // 16-byte loads when every row starts 16-byte aligned
  const bool vec4 = S % 4 == 0 && reinterpret_cast<uintptr_t>(mass) % 16 == 0;
  if (!use_split(rows, S)) {
    SelArgs a;
    a.mass = mass;
    a.keep = keep;
    a.S = S;
    a.window = window;
    a.n_sink = n_sink;
    a.top_k = top_k;
    a.n_keep = n_keep;
    const dim3 grid((unsigned)rows), reg_block(kRegThreads);
    if (S <= kRegThreads * 8)
      hipLaunchKernelGGL(select_reg_kernel<8>, grid, reg_block, 0, stream, a, vec4);
    else if (S <= kRegThreads * 16)
      hipLaunchKernelGGL(select_reg_kernel<16>, grid, reg_block, 0, stream, a, vec4);
    else
      hipLaunchKernelGGL(select_reg_kernel<32>, grid, reg_block, 0, stream, a, vec4);
    return hipGetLastError();
  }
  MbArgs a;
  a.mass = mass;
  a.keep = keep;
  a.S = S;
  a.window = window;
  a.n_sink = n_sink;
  const int e_hi = S - window;
  const int n_elig = e_hi > n_sink ? e_hi - n_sink : 0;
  a.kk = top_k < n_elig ? top_k : n_elig;
  a.mode = a.kk == 0 ? kTakeNone : (a.kk == n_elig ? kTakeAll : kSelect);
  mb_plan(rows, S, a.nc, a.C);
  a.n_keep = n_keep;
  a.vec4 = vec4;
  char* ws = static_cast<char*>(workspace);
  a.hist = reinterpret_cast<int32_t*>(ws);
  ws += align256((size_t)rows * a.nc * kBins1 * 4);
  a.chunk = reinterpret_cast<int32_t*>(ws);
  ws += align256((size_t)rows * a.nc * 16);
  a.state = reinterpret_cast<int32_t*>(ws);
  ws += align256((size_t)rows * kStateInts * 4);
  a.cand = reinterpret_cast<uint32_t*>(ws);
  const dim3 chunks((unsigned)(rows * a.nc)), per_row((unsigned)rows);
  if (a.mode == kSelect) {
    hipLaunchKernelGGL(sel_hist_kernel, chunks, dim3(kMbThreads), 0, stream, a);
    hipLaunchKernelGGL(sel_bin_kernel, per_row, dim3(kMbThreads), 0, stream, a);
    hipLaunchKernelGGL(sel_compact_kernel, chunks, dim3(kMbThreads), 0, stream, a);
    hipLaunchKernelGGL(sel_finish_kernel, per_row, dim3(kFinThreads), 0, stream, a);
  }
  hipLaunchKernelGGL(sel_emit_kernel, chunks, dim3(kMbThreads), 0, stream, a);
  return hipGetLastError();
}

// ---- the same selection for callers that cannot allocate: the split path's
// state in a fixed device array of this library (one copy per GPU)

namespace {

__device__ __align__(256) unsigned char scratch[kSelectScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t select_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    // the device address of this GPU's copy of the array; the name itself is
    // only a host-side stand-in and must never reach a kernel
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace kvp
