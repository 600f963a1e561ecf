// Causal log-sum-exp pass for gfx950.
//
//   lse[b, g, i] = ln sum_{j <= i} exp(scale * <q_i, k_j>)
// the dense causal normaliser of every query row (LKV §3 Eq. 1), i.e. the
// per-query log-normaliser that KVpop §3.2 (Eq. 8) reuses for the future mass.
//
// Work decomposition (queries stationary, keys streamed):
//   * one workgroup = 8 waves (one per CU; 4 waves, two per CU, for grids
//     too small to give every CU two); each wave owns 96 consecutive query
//     positions of one query head (three 32-column MFMA blocks kept as bf16 B
//     operands in registers; two blocks, 64 positions, in the sparse pass and
//     for grids too small for three; one block, 32 positions, in paired
//     8-wave grids of short sequences); the waves cover (position block, head) pairs
//     of one GQA group, heads fastest, so the group's shared keys are staged
//     once for all of them;
//   * keys are streamed in blocks of 32 from position 0 upwards, one block
//     per wave per LDS stage, double buffered; wave w stages block w of
//     every stage.
//     In LDS a key block is stored as the MFMA A operands themselves (per
//     16-wide slice of d, 1 KB with lane l's 16 bytes at 16 l), copied from
//     HBM through VGPRs in two halves, so every operand read is one
//     contiguous ds_read_b128;
//   * per key block and wave: 24 MFMA 32x32x16 give a 32-key x 96-query
//     tile (16 MFMA and 64 queries for fp32 input, the sparse pass and
//     grids too short to fill the CUs); each lane (one query column per
//     32-query block) adds
//     exp2(c*s - u) of its 16 values into one running sum per block;
//   * software pipeline inside each wave: the MFMAs of block p+1 are issued
//     between the VALU operations of block p;
//   * every workgroup of a (batch, KV head) walks the same key sequence
//     (shared L2), and workgroups run longest first; in grids of one
//     workgroup per CU whose tile pairs fill whole rounds of the CUs, each
//     workgroup takes the tile of the longest rows and then the tile of the
//     shortest, so every workgroup has the same work.
// Sparse mode (the running top-k pattern of KVpop §3.2, whose per-query
// log-normalisers the student returns): key j counts for query i iff j <= i
// and (i - j < w or rank[j] <= cutoff[i]).  Each staged key block carries its
// 32 ranks in LDS, read into registers with the block's operands; each lane
// holds the cutoffs of its two query columns.  Leading key blocks outside
// every query's window need only the rank test (pipelined like the dense
// path); the window band and the diagonal take the general test.
// The shift u of a row is the largest logit of its first key block (which
// always holds key 0, valid for every row), so the running sum is >= 1 and
// cannot underflow; it could only overflow if a later logit exceeded that by
// more than ~88 (natural units).  Such rows are flagged and recomputed
// exactly, after the sweep, by the wave that swept them: a max-then-sum pass
// over the row's keys.
#include <type_traits>

#include "kvp_device.h"
#include "kvp_launch.h"

namespace kvp {
namespace {

template <int D, int W, int NB>
struct LseCfg {
  static constexpr int kWaves = W;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kQueryBlocks = NB;        // 32-column query blocks per wave
  static constexpr int kQueriesPerWave = 32 * NB;
  static constexpr int kKSteps = D / 16;          // 16-wide slices of d
  static constexpr int kFragBytes = kWave * 16;   // one A operand (1 KB)
  static constexpr int kSlotBytes = kKSteps * kFragBytes;
  static constexpr int kSlots = kWaves;           // wave w stages slot w
  static constexpr int kStageBytes = kSlots * kSlotBytes;
  static constexpr int kMfmaPerBlock = NB * kKSteps;
};

// Most 32-query blocks per wave: three for the dense pass (every staged key
// block then feeds 24 MFMAs per wave), two for the sparse pass, whose rank
// registers would otherwise spill.  Grids too small for two 8-wave workgroups
// per CU at three blocks run two blocks per wave instead, so that short
// sequences still spread over every CU.
template <typename T, bool kSp>
constexpr int lse_query_blocks() {
  return kSp ? 2 : 3;
}

struct LseArgs {
  const void* q;
  const void* k;
  float* lse;
  int B, Hq, Hkv, S, G;
  int n_wg;  // tiles of 8 (or 4) waves per (batch, KV head); paired mode:
             // block x takes tiles x' and n_wg - 1 - x' of its unit (x' the
             // tile index the block mapping gives)
  float c;   // scale * log2(e)
  float scale;  // the logit scale itself (the exact recomputation of flagged rows)
  // sparse mode (running top-k pattern): key j counts for query i iff
  // j <= i and (i - j < window or rank[j] <= cutoff[i]); [B, Hkv, S] each
  const int32_t* rank;
  const int32_t* cutoff;
  int window;
};

template <bool kSp>
struct LTile {
  f32x16_t s0, s1, s2;  // logits: 32 keys (rows) x query block 0 / 1 / 2 (columns)
};
template <>
struct LTile<true> {
  f32x16_t s0, s1, s2;  // (s2 unused: the sparse pass keeps two query blocks)
  // ranks of this lane's 16 key rows (sparse mode), as fp32 bit patterns
  // (exact: ranks lie in [-1, S) and S <= 2^22)
  u32x4_t rk0, rk1, rk2, rk3;
  __device__ __forceinline__ float rank_of(int v) const {
    const u32x4_t& q = v < 4 ? rk0 : v < 8 ? rk1 : v < 12 ? rk2 : rk3;
    return __uint_as_float(q[v & 3]);
  }
};

// Exact LSE of row i of query head gq (batch bb, KV head hh), by the 64
// lanes of one wave: a max pass then a sum pass over the row's counted keys
// (all of j <= i, or the sparse pattern), one key per lane at a time, in
// fp32; an empty pattern gives -inf.  Lane 0 writes the result.
template <int D, typename T, bool kSp>
__device__ __forceinline__ void exact_row(const LseArgs& a, int bb, int hh, int gq, int i,
                                          int lane) {
  const int S = a.S;
  const size_t row = (size_t)(bb * a.Hq + gq) * S + i;
  const T* qi = static_cast<const T*>(a.q) + row * D;
  const T* kh = static_cast<const T*>(a.k) + (size_t)(bb * a.Hkv + hh) * S * D;
  u32x4_t q8[D / 8];  // the query row, bf16
#pragma unroll
  for (int c8 = 0; c8 < D / 8; ++c8) q8[c8] = load8(qi + c8 * 8);
  auto logit = [&](int j) {
    const T* kj = kh + (size_t)j * D;
    float dot = 0.f;
#pragma unroll
    for (int c8 = 0; c8 < D / 8; ++c8) {
      const bf16x8_t qe = __builtin_bit_cast(bf16x8_t, q8[c8]);
      const bf16x8_t ke = __builtin_bit_cast(bf16x8_t, load8(kj + c8 * 8));
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) dot = __builtin_fmaf((float)qe[e8], (float)ke[e8], dot);
    }
    return dot * a.scale;
  };
  const size_t kv_row = (size_t)(bb * a.Hkv + hh) * S;
  const int cut = kSp ? a.cutoff[kv_row + i] : 0;
  auto counts = [&](int j) {
    if constexpr (kSp) return (i - j < a.window) || (a.rank[kv_row + j] <= cut);
    return true;
  };
  float m = -__builtin_inff();
  for (int j = lane; j <= i; j += 64)
    if (counts(j)) m = fmaxf(m, logit(j));
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  float s = 0.f;
  for (int j = lane; j <= i; j += 64)
    if (counts(j)) s += __expf(logit(j) - m);
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) a.lse[row] = s > 0.f ? m + __logf(s) : -__builtin_inff();
}

template <int D, typename T, int W, bool kSp, bool kPair, int NB>
__global__ __launch_bounds__(kWave * W, 8 / W) void lse_kernel(LseArgs a) {
  static_assert(NB >= 1 && NB <= lse_query_blocks<T, kSp>(), "query blocks per wave");
  static_assert(NB >= 2 || !kSp, "one query block per wave: dense pass only");
  using C = LseCfg<D, W, NB>;
  using Tile = LTile<kSp>;
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds0[C::kStageBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds1[C::kStageBytes];
  // sparse mode: ranks of the staged key blocks, one int per key
  __shared__ __attribute__((aligned(16))) int r_lds0[kSp ? C::kSlots * kBlk : 4];
  __shared__ __attribute__((aligned(16))) int r_lds1[kSp ? C::kSlots * kBlk : 4];

  const int S = a.S, G = a.G;
  int unit, tile;
  // paired grids carry equal work per block: whole units per round of an
  // XCD; otherwise longest tiles first
  if constexpr (kPair)
    xcd_map_units(blockIdx.x, a.B * a.Hkv, (a.n_wg + 1) / 2, unit, tile);
  else
    xcd_map(blockIdx.x, a.B * a.Hkv, unit, tile);
  const int b = unit / a.Hkv;
  const int h = unit - b * a.Hkv;
  // Paired mode: the workgroup takes tile `tile` and then tile n_wg - 1 -
  // tile of the same unit, the longest rows with the shortest, so every
  // workgroup of the grid has the same work.
  const int tile_last = kPair ? a.n_wg - 1 - tile : tile;
  const int n_rep = tile_last != tile ? 2 : 1;
  for (int rep = 0; rep < n_rep; ++rep) {
  // the previous tile's last stage has read the stage buffers
  if (rep) __syncthreads();
  // lane indices are re-derived per tile from an opaque copy of the thread
  // id, so that nothing computed from them stays live across both tiles
  int tid = threadIdx.x;
  if constexpr (kPair) asm volatile("" : "+v"(tid));
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h32 = lane >> 5;

  // (position block, head) pairs, heads fastest; tile 0 takes the last pairs
  // (the longest rows).
  const int n_pb = (S + C::kQueriesPerWave - 1) / C::kQueriesPerWave;
  const int n_pairs = n_pb * G;
  const int pair0 = (a.n_wg - 1 - (rep ? tile_last : tile)) * C::kWaves;
  const int my_pair = pair0 + wave;
  const bool active = my_pair < n_pairs;
  const int pb = my_pair / G;
  const int g = my_pair - pb * G;
  const int p0 = pb * C::kQueriesPerWave;

  // Keys needed by the workgroup: [0, key_end).
  const int last_pair = min(pair0 + C::kWaves, n_pairs) - 1;
  const int key_end = min(S, (last_pair / G + 1) * C::kQueriesPerWave);
  const int n_kb = (key_end + kBlk - 1) / kBlk;
  const int n_stages = (n_kb + C::kSlots - 1) / C::kSlots;
  // For this wave: key blocks [0, kb_full) are entirely at or below every
  // query of the wave and inside the sequence (no mask); blocks [kb_full,
  // kb_end) need the mask; blocks >= kb_end hold no key for these queries.
  const int kb_end = active ? min(n_kb, (min(p0 + C::kQueriesPerWave, S) + kBlk - 1) / kBlk) : 0;
  const int kb_full = active ? min(kb_end, min(p0 + 1, S) / kBlk) : 0;

  const T* __restrict__ kbase = static_cast<const T*>(a.k) + (size_t)(b * a.Hkv + h) * S * D;
  const T* __restrict__ qrow = static_cast<const T*>(a.q) + (size_t)(b * a.Hq + h * G + g) * S * D;
  const uint32_t head_bytes = (uint32_t)S * D * sizeof(T);

  // Stationary queries: B operands of the NB 32-column blocks.
  u32x4_t qf[NB][C::kKSteps];
  {
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(qrow, active ? head_bytes : 0u);
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int ks = 0; ks < C::kKSteps; ++ks)  // rows >= S (or no pair) read 0
        qf[cb][ks] = buf_load8(qr, (uint32_t)(p0 + 32 * cb + l32) * D + 16 * ks + 8 * h32,
                               static_cast<const T*>(nullptr));
    // wait here once, so that no use of the queries inside the sweep waits on
    // the loads of the stage copies in flight
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  }

  const float c = a.c;
  float u0 = 0.f, u1 = 0.f, u2 = 0.f;        // per-row shifts (log2 units)
  float sum0 = 0.f, sum1 = 0.f, sum2 = 0.f;  // running sums of exp2(c*s - u)
  // Partial sums of the current eight key blocks, added into the running sums
  // every eighth block: a row with one dominant key has thousands of terms
  // below half an ulp of its sum, and a block's partial of 16 such terms is
  // rounded once per addition; eight blocks per addition keep that loss about
  // eight times smaller (at 131072 keys: from about 1e-4 to about 1e-5 of the
  // LSE in the worst rows).  The grouping follows the key-block index, so it
  // is the same for every launch configuration.
  float stg0 = 0.f, stg1 = 0.f, stg2 = 0.f;
  const int iq0 = p0 + l32;
  const int iq1 = iq0 + 32;
  const int iq2 = iq0 + 64;

  // sparse mode: the cutoffs of this lane's two query columns, and the
  // leading key blocks that lie outside every query's window (the rank test
  // alone decides there)
  const size_t kv_row = (size_t)(b * a.Hkv + h) * S;
  // The cutoffs are held as cut + 1 in fp32, clamped to [-1, S] first (no
  // rank lies outside [-1, S), so the test rank <= cut is unchanged and exact).
  float cut0 = 0.f, cut1 = 0.f;
  int kb_rank_end = 0;
  if constexpr (kSp) {
    cut0 = (float)(iq0 < S ? min(max(a.cutoff[kv_row + iq0], -1), S) : -1) + 1.f;
    cut1 = (float)(iq1 < S ? min(max(a.cutoff[kv_row + iq1], -1), S) : -1) + 1.f;
    const int lim = p0 - a.window + 1;  // keys j <= p0 - w are outside all windows
    kb_rank_end = active && lim > 0 ? min(kb_full, lim / kBlk) : 0;
  }
  int rank_pref = 0;

  // ---- staging: wave w copies key block kSlots * st + w of stage st, in halves
  constexpr int kHalf = C::kKSteps / 2;
  u32x4_t stage_regs[kHalf];
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase, head_bytes);
  auto issue_loads = [&](int st, int half) __attribute__((always_inline)) {
    const int kb = st * C::kSlots + wave;
    if (kb >= n_kb) return;
    if constexpr (kSp) {
      if (half == 0 && lane < kBlk) {
        const int j = kb * kBlk + lane;
        rank_pref = j < S ? a.rank[kv_row + j] : 0x7FFFFFFF;
      }
    }
    const uint32_t e0 = (uint32_t)(kb * kBlk + l32) * D + 8 * h32;
#pragma unroll
    for (int t = 0; t < kHalf; ++t)  // keys >= S read 0
      stage_regs[t] = buf_load8(kr, e0 + 16 * (half * kHalf + t), static_cast<const T*>(nullptr));
  };
  auto store_half = [&](int st, int half, unsigned char* kdst, int* rdst)
                        __attribute__((always_inline)) {
    if (st * C::kSlots + wave >= n_kb) return;
    if constexpr (kSp) {
      if (half == 1 && lane < kBlk) rdst[wave * kBlk + lane] = __float_as_int((float)rank_pref);
    }
    unsigned char* slot = kdst + wave * C::kSlotBytes + lane * 16;
#pragma unroll
    for (int t = 0; t < kHalf; ++t)
      *reinterpret_cast<u32x4_t*>(slot + (half * kHalf + t) * C::kFragBytes) = stage_regs[t];
  };

  // ---- compute
  auto mfma_block = [&](Tile& t, const unsigned char* ksrc, const int* rsrc, int slot)
                        __attribute__((always_inline)) {
    const unsigned char* src = ksrc + slot * C::kSlotBytes + lane * 16;
#pragma unroll
    for (int ks = 0; ks < C::kKSteps; ++ks) {
      const u32x4_t ak = *reinterpret_cast<const u32x4_t*>(src + ks * C::kFragBytes);
      t.s0 = mfma_32x32x16(ak, qf[0][ks], ks ? t.s0 : f32x16_t{});
      if constexpr (NB >= 2) t.s1 = mfma_32x32x16(ak, qf[NB >= 2 ? 1 : 0][ks], ks ? t.s1 : f32x16_t{});
      if constexpr (NB == 3) t.s2 = mfma_32x32x16(ak, qf[2][ks], ks ? t.s2 : f32x16_t{});
    }
    if constexpr (kSp) {
      // ranks of rows 8 g + 4 h32 + (0..3): the rows of values 4 g .. 4 g + 3
      // (read after the operands, so the operand reads keep their place in
      // the issue order)
      const int* rp = rsrc + slot * kBlk + 4 * h32;
      t.rk0 = *reinterpret_cast<const u32x4_t*>(rp);
      t.rk1 = *reinterpret_cast<const u32x4_t*>(rp + 8);
      t.rk2 = *reinterpret_cast<const u32x4_t*>(rp + 16);
      t.rk3 = *reinterpret_cast<const u32x4_t*>(rp + 24);
    }
  };
  auto exp_full = [&](const Tile& t) __attribute__((always_inline)) {
    float t0 = 0.f, t1 = 0.f, t2 = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      t0 += fast_exp2(__builtin_fmaf(t.s0[v], c, -u0));
      if constexpr (NB >= 2) t1 += fast_exp2(__builtin_fmaf(t.s1[v], c, -u1));
      if constexpr (NB == 3) t2 += fast_exp2(__builtin_fmaf(t.s2[v], c, -u2));
    }
    stg0 += t0;
    if constexpr (NB >= 2) stg1 += t1;
    if constexpr (NB == 3) stg2 += t2;
  };
  // sparse mode, blocks outside every window: a key counts iff its rank is
  // at most the query's cutoff.  The 0/1 weight is one clamped subtract,
  // clamp((cut + 1) - rank, 0, 1), applied in the accumulating fma: no
  // compare masks in scalar registers.  (A dropped term whose exponential
  // overflowed gives inf * 0 = NaN, which is flagged for the exact pass like
  // any overflow.)
  auto exp_rank = [&](const Tile& t) __attribute__((always_inline)) {
    if constexpr (kSp) {
      float t0 = 0.f, t1 = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float rk = t.rank_of(v);
        const float w0 = __builtin_amdgcn_fmed3f(cut0 - rk, 0.f, 1.f);
        const float w1 = __builtin_amdgcn_fmed3f(cut1 - rk, 0.f, 1.f);
        const float x0 = __builtin_fmaf(t.s0[v], c, -u0);
        const float x1 = __builtin_fmaf(t.s1[v], c, -u1);
        t0 = __builtin_fmaf(fast_exp2(x0), w0, t0);
        t1 = __builtin_fmaf(fast_exp2(x1), w1, t1);
      }
      stg0 += t0;
      stg1 += t1;
    }
  };
  // sparse mode, other blocks: causal, and window or rank
  auto exp_sparse = [&](const Tile& t, int kb) __attribute__((always_inline)) {
    if constexpr (kSp) {
      const int lim0 = min(iq0, S - 1) - kb * kBlk - 4 * h32;  // causal: r <= lim
      const int lim1 = min(iq1, S - 1) - kb * kBlk - 4 * h32;
      const int win0 = iq0 - a.window - kb * kBlk - 4 * h32;   // window: r > win
      const int win1 = iq1 - a.window - kb * kBlk - 4 * h32;
      float t0 = 0.f, t1 = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + (v & 3);
        const float rk = t.rank_of(v);
        const bool k0 = r <= lim0 && (r > win0 || rk < cut0);
        const bool k1 = r <= lim1 && (r > win1 || rk < cut1);
        const float x0 = __builtin_fmaf(t.s0[v], c, -u0);
        const float x1 = __builtin_fmaf(t.s1[v], c, -u1);
        t0 += fast_exp2(k0 ? x0 : -__builtin_inff());
        t1 += fast_exp2(k1 ? x1 : -__builtin_inff());
      }
      stg0 += t0;
      stg1 += t1;
    }
  };
  auto exp_masked = [&](const Tile& t, int kb) __attribute__((always_inline)) {
    // key j = 32 kb + 8 (v / 4) + 4 h32 + v % 4 counts iff j <= min(i, S - 1),
    // i.e. iff the constant 8 (v / 4) + v % 4 <= lim
    const int lim0 = min(iq0, S - 1) - kb * kBlk - 4 * h32;
    const int lim1 = min(iq1, S - 1) - kb * kBlk - 4 * h32;
    const int lim2 = min(iq2, S - 1) - kb * kBlk - 4 * h32;
    float t0 = 0.f, t1 = 0.f, t2 = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 8 * (v >> 2) + (v & 3);
      const float x0 = __builtin_fmaf(t.s0[v], c, -u0);
      t0 += fast_exp2(r <= lim0 ? x0 : -__builtin_inff());
      if constexpr (NB >= 2) {
        const float x1 = __builtin_fmaf(t.s1[v], c, -u1);
        t1 += fast_exp2(r <= lim1 ? x1 : -__builtin_inff());
      }
      if constexpr (NB == 3) {
        const float x2 = __builtin_fmaf(t.s2[v], c, -u2);
        t2 += fast_exp2(r <= lim2 ? x2 : -__builtin_inff());
      }
    }
    stg0 += t0;
    if constexpr (NB >= 2) stg1 += t1;
    if constexpr (NB == 3) stg2 += t2;
  };
  // Shifts from the first key block (key 0 is valid for every row).
  auto set_shift = [&](const Tile& t) __attribute__((always_inline)) {
    float m0 = -__builtin_inff(), m1 = -__builtin_inff(), m2 = -__builtin_inff();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int j = mfma_row(v, lane);
      if (j <= iq0 && j < S) m0 = fmaxf(m0, t.s0[v]);
      if constexpr (NB >= 2)
        if (j <= iq1 && j < S) m1 = fmaxf(m1, t.s1[v]);
      if constexpr (NB == 3)
        if (j <= iq2 && j < S) m2 = fmaxf(m2, t.s2[v]);
    }
    m0 = fmaxf(m0, __shfl_xor(m0, 32));
    m1 = fmaxf(m1, __shfl_xor(m1, 32));
    u0 = m0 * c;
    u1 = m1 * c;
    if constexpr (NB == 3) u2 = fmaxf(m2, __shfl_xor(m2, 32)) * c;
  };
  // Exponentials of block kb (in cur) and MFMAs of block kb + 1 (into nxt).
  auto step = [&](Tile& cur, Tile& nxt, int kb, const unsigned char* nk, const int* nr, int nslot)
                  __attribute__((always_inline)) {
    const bool m_ok = kb + 1 < kb_end;
    // dense: blocks below every query; sparse: blocks also outside every window
    const bool fast = kSp ? kb < kb_rank_end : kb < kb_full;
    // VALU and transcendental (exp2) operations per MFMA: per value an fma
    // and an add (dense) or a clamped subtract and two fma (rank test), and
    // one exp2
    constexpr int kValuPerMfma = (kSp ? 3 : 2) * 16 * NB / C::kMfmaPerBlock;
    constexpr int kTransPerMfma = 16 * NB / C::kMfmaPerBlock;
    if (m_ok && fast) {
      mfma_block(nxt, nk, nr, nslot);
      if constexpr (kSp)
        exp_rank(cur);
      else
        exp_full(cur);
      // operand reads issued ahead: four with one block per wave (each read
      // then feeds a single MFMA), else two
      constexpr int kAhead = NB == 1 ? 4 : 2;
      __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
      for (int m = 0; m < C::kMfmaPerBlock; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
        __builtin_amdgcn_sched_group_barrier(0x400, kTransPerMfma, 0);
        // one operand read per key slice, i.e. after every NB-th MFMA
        if (NB == 1 ? m < C::kKSteps - kAhead : (m % NB == NB - 1 && m < NB * C::kKSteps - NB))
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (kSp && m == C::kKSteps - 1)  // the next block's four rank reads
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
    } else {
      if (m_ok) mfma_block(nxt, nk, nr, nslot);
      if (fast) {
        if constexpr (kSp)
          exp_rank(cur);
        else
          exp_full(cur);
      } else if (kb < kb_end) {
        if constexpr (kSp)
          exp_sparse(cur, kb);
        else
          exp_masked(cur, kb);
      }
    }
  };

  auto flush_partials = [&]() __attribute__((always_inline)) {
    sum0 += stg0;
    stg0 = 0.f;
    if constexpr (NB >= 2) {
      sum1 += stg1;
      stg1 = 0.f;
    }
    if constexpr (NB == 3) {
      sum2 += stg2;
      stg2 = 0.f;
    }
  };
  Tile t0, t1;
  // One stage: the exponentials of its kSlots key blocks, the MFMAs of each
  // next block one step ahead (the last step's from the other buffer, after
  // the barrier); the next stage's copies are stored in two halves.
  static_assert(C::kSlots % 2 == 0 && C::kSlots >= 4, "tile ping-pong needs an even stage");
  constexpr int kStoreA = C::kSlots == 8 ? 1 : 0;  // store half 0 after this step
  constexpr int kStoreB = C::kSlots == 8 ? 3 : 2;  // store half 1 after this step
  static_assert(kStoreA < kStoreB && kStoreB <= C::kSlots - 2,
                "both halves must be stored before the stage's last step");
  auto stage = [&](auto bufc, int st) __attribute__((always_inline)) {
    constexpr int kBuf = decltype(bufc)::value;
    unsigned char* ck = kBuf ? k_lds1 : k_lds0;
    unsigned char* nk = kBuf ? k_lds0 : k_lds1;
    int* cr = kBuf ? r_lds1 : r_lds0;
    int* nr = kBuf ? r_lds0 : r_lds1;
    const bool more = st + 1 < n_stages;
    if (more) issue_loads(st + 1, 0);
    const int kb0 = st * C::kSlots;
#pragma unroll
    for (int j = 0; j < C::kSlots - 1; ++j) {
      if (j & 1)
        step(t1, t0, kb0 + j, ck, cr, j + 1);
      else
        step(t0, t1, kb0 + j, ck, cr, j + 1);
      if (more && j == kStoreA) {
        store_half(st + 1, 0, nk, nr);
        issue_loads(st + 1, 1);
      }
      if (more && j == kStoreB) store_half(st + 1, 1, nk, nr);
    }
    __syncthreads();
    step(t1, t0, kb0 + C::kSlots - 1, nk, nr, 0);
    // key blocks 8 m .. 8 m + 7 done: one stage of eight, or two of four
    if (C::kSlots == 8 || (st & 1)) flush_partials();
  };

  issue_loads(0, 0);
  store_half(0, 0, k_lds0, r_lds0);
  issue_loads(0, 1);
  store_half(0, 1, k_lds0, r_lds0);
  __syncthreads();
  if (0 < kb_end) {
    mfma_block(t0, k_lds0, r_lds0, 0);
    set_shift(t0);
  }
  for (int st = 0; st < n_stages; st += 2) {
    stage(std::integral_constant<int, 0>{}, st);
    if (st + 1 >= n_stages) break;
    stage(std::integral_constant<int, 1>{}, st + 1);
  }

  flush_partials();  // the blocks after the last multiple of eight
  // Combine the two half-columns (lanes l and l^32 hold the same query).
  sum0 += __shfl_xor(sum0, 32);
  if constexpr (NB >= 2) sum1 += __shfl_xor(sum1, 32);
  if constexpr (NB == 3) sum2 += __shfl_xor(sum2, 32);
  // A non-finite sum (overflow) flags the row; in sparse mode so does a sum
  // too small to trust (the shift comes from every key of the first block,
  // kept or not) or an empty pattern.  Flagged rows are written below.
  const float lo = kSp ? 0x1p-60f : 0.f;
  const float l0 = (u0 + __log2f(sum0)) * kLn2;
  const bool ok0 = sum0 < __builtin_inff() && l0 == l0 && (!kSp || sum0 >= lo);
  float l1 = 0.f, l2 = 0.f;
  bool ok1 = true, ok2 = true;
  if constexpr (NB >= 2) {
    l1 = (u1 + __log2f(sum1)) * kLn2;
    ok1 = sum1 < __builtin_inff() && l1 == l1 && (!kSp || sum1 >= lo);
  }
  if constexpr (NB == 3) {
    l2 = (u2 + __log2f(sum2)) * kLn2;
    ok2 = sum2 < __builtin_inff() && l2 == l2;
  }
  const int gq = h * G + g;  // query head
  const bool own = active && lane < 32;
  if (own) {
    float* out = a.lse + (size_t)(b * a.Hq + gq) * S;
    if (iq0 < S && ok0) out[iq0] = l0;
    if (NB >= 2 && iq1 < S && ok1) out[iq1] = l1;
    if (NB == 3 && iq2 < S && ok2) out[iq2] = l2;
  }
  // The wave's flagged rows, one after another, recomputed exactly.
  uint64_t flagged[3] = {__ballot(own && iq0 < S && !ok0),
                         NB >= 2 ? __ballot(own && iq1 < S && !ok1) : 0ull,
                         NB == 3 ? __ballot(own && iq2 < S && !ok2) : 0ull};
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    uint64_t m = flagged[cb];
    while (m) {
      const int bit = __builtin_ctzll(m);
      m &= m - 1;
      exact_row<D, T, kSp>(a, b, h, gq, p0 + 32 * cb + bit, lane);
    }
  }
  }  // tiles of the workgroup
}

struct SparseIn {
  const int32_t* rank;
  const int32_t* cutoff;
  int window;
};

template <int D, typename T, int W, bool kSp, int NB>
hipError_t launch_lse_w(const void* q, const void* k, const Shape& sh, float scale, float* lse,
                        const SparseIn& sp, hipStream_t stream) {
  using C = LseCfg<D, W, NB>;
  LseArgs a;
  a.rank = sp.rank;
  a.cutoff = sp.cutoff;
  a.window = sp.window;
  a.q = q;
  a.k = k;
  a.lse = lse;
  a.B = sh.B;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.S = sh.S;
  a.G = sh.G;
  a.c = scale * kLog2e;
  a.scale = scale;
  const int64_t n_pb = (sh.S + C::kQueriesPerWave - 1) / C::kQueriesPerWave;
  a.n_wg = (int)((n_pb * sh.G + C::kWaves - 1) / C::kWaves);
  const int64_t units = (int64_t)sh.B * sh.Hkv;
  // One-workgroup-per-CU grids pair the tile of the longest rows with the
  // tile of the shortest when the equal-work pairs fill whole rounds of the
  // CUs (at least 95%).
  bool pair = false;
  if (W == 8 && a.n_wg >= 2) {
    const int64_t pairs = units * ((a.n_wg + 1) / 2);
    const int64_t rounds = (pairs + kNumCUs - 1) / kNumCUs;
    pair = pairs * 20 >= rounds * kNumCUs * 19;
  }
  const int64_t blocks = units * (pair ? (a.n_wg + 1) / 2 : a.n_wg);
  if constexpr (W == 8) {
    if (pair)
      hipLaunchKernelGGL((lse_kernel<D, T, W, kSp, true, NB>), dim3((unsigned)blocks),
                         dim3(C::kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((lse_kernel<D, T, W, kSp, false, NB>), dim3((unsigned)blocks),
                         dim3(C::kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL((lse_kernel<D, T, W, kSp, false, NB>), dim3((unsigned)blocks),
                       dim3(C::kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

// 8-wave workgroups (one per CU) when the grid holds at least two per CU;
// else 8-wave workgroups of one query block per wave, each taking a long and
// a short tile, when those pairs fill whole rounds of the CUs; else 4-wave
// workgroups (two per CU) with two query blocks per wave.  Three
// query blocks per wave only where they still give such a grid.  The number
// of blocks per wave does not change the result: every row sums the same key
// blocks in the same order.
template <int D, typename T, bool kSp>
hipError_t launch_lse_t(const void* q, const void* k, const Shape& sh, float scale, float* lse,
                        const SparseIn& sp, hipStream_t stream) {
  auto blocks8 = [&](int queries_per_wave) {
    const int64_t n_pb = (sh.S + queries_per_wave - 1) / queries_per_wave;
    return (n_pb * sh.G + 7) / 8 * sh.B * sh.Hkv;
  };
  if constexpr (lse_query_blocks<T, kSp>() == 3) {
    if (blocks8(LseCfg<D, 8, 3>::kQueriesPerWave) >= 2 * kNumCUs)
      return launch_lse_w<D, T, 8, kSp, 3>(q, k, sh, scale, lse, sp, stream);
  }
  if (blocks8(LseCfg<D, 8, 2>::kQueriesPerWave) >= 2 * kNumCUs)
    return launch_lse_w<D, T, 8, kSp, 2>(q, k, sh, scale, lse, sp, stream);
  if constexpr (!kSp) {
    // one query block per wave, workgroups pairing the longest rows with the
    // shortest, when those pairs fill whole rounds of the CUs
    const int64_t n_wg = (((int64_t)sh.S + kBlk - 1) / kBlk * sh.G + 7) / 8;
    const int64_t pairs = (int64_t)sh.B * sh.Hkv * ((n_wg + 1) / 2);
    const int64_t rounds = (pairs + kNumCUs - 1) / kNumCUs;
    if (n_wg >= 2 && pairs * 20 >= rounds * kNumCUs * 19)
      return launch_lse_w<D, T, 8, kSp, 1>(q, k, sh, scale, lse, sp, stream);
  }
  return launch_lse_w<D, T, 4, kSp, 2>(q, k, sh, scale, lse, sp, stream);
}

}  // namespace

hipError_t launch_lse(const void* q, const void* k, int dtype, const Shape& sh, float scale,
                      float* lse, hipStream_t stream) {
  if (dtype != 0) return launch_lse_f32(q, k, sh, scale, nullptr, nullptr, 0, lse, stream);
  const SparseIn none{nullptr, nullptr, 0};
  return sh.D == 128 ? launch_lse_t<128, uint16_t, false>(q, k, sh, scale, lse, none, stream)
                     : launch_lse_t<64, uint16_t, false>(q, k, sh, scale, lse, none, stream);
}

hipError_t launch_lse_sparse(const void* q, const void* k, int dtype, const Shape& sh, float scale,
                             const int32_t* rank, const int32_t* cutoff, int window, float* lse,
                             hipStream_t stream) {
  if (dtype != 0) return launch_lse_f32(q, k, sh, scale, rank, cutoff, window, lse, stream);
  const SparseIn sp{rank, cutoff, window};
  return sh.D == 128 ? launch_lse_t<128, uint16_t, true>(q, k, sh, scale, lse, sp, stream)
                     : launch_lse_t<64, uint16_t, true>(q, k, sh, scale, lse, sp, stream);
}

}  // namespace kvp
