// Per-KV-head keep-set for gfx950.
//
//   keep = ascending( sinks [0, min(s, S))  U  window [max(0, S - w), S)
//                     U  top-k of score over the eligible range [s, S - w) )
// KVpop Fig. 1 / §3 Eq. 1 (budget s + w + k per KV head) and Eq. 4 (eligible
// set at the last query).  The scores are future masses or any fp32 score
// (e.g. the log targets, which are negative).  Ranking: score descending,
// equal scores by ascending index.
//
// One workgroup per (batch, KV head) row, in two steps:
//   1. radix select, most significant byte first, on an order-preserving
//      32-bit key of each fp32 score (any sign; see score_key): four passes of a
//      256-bin LDS histogram over the candidates that match the bytes fixed
//      so far give the k-th largest value T exactly and the number r of
//      copies of T that belong to the top-k (the r lowest-indexed ones);
//   2. ordered emission: position j is kept iff it is a sink or in the
//      window, or its key is above T, or it is among the first r copies of T;
//      its output slot is the number of kept positions before it, so the
//      output is ascending with no sort.
// Rows of up to 32768 scores (select_reg_kernel, 1024 threads): each thread
// holds KPT consecutive keys in registers, so the row is read from memory
// once; the passes histogram from registers into per-wave LDS copies, and
// one block-wide scan of (kept, tie) counts places every kept position.
// Longer rows (select_kernel, 256 threads) re-read the row from memory per
// pass and emit in chunks of 256 positions with a ballot scan per chunk.
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
  // 16-byte loads when every row starts 16-byte aligned
  const bool vec4 = S % 4 == 0 && reinterpret_cast<uintptr_t>(mass) % 16 == 0;
  const dim3 grid((unsigned)rows), reg_block(kRegThreads);
  if (S <= kRegThreads * 8)
    hipLaunchKernelGGL(select_reg_kernel<8>, grid, reg_block, 0, stream, a, vec4);
  else if (S <= kRegThreads * 16)
    hipLaunchKernelGGL(select_reg_kernel<16>, grid, reg_block, 0, stream, a, vec4);
  else if (S <= kRegThreads * 32)
    hipLaunchKernelGGL(select_reg_kernel<32>, grid, reg_block, 0, stream, a, vec4);
  else
    hipLaunchKernelGGL(select_kernel, grid, dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvp
