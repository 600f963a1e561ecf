// Transposed future-attention-mass pass for gfx950.
//
// Computes, for every key j of every (batch, KV head),
//   mass[j] = sum over the G query heads g of the group,
//             sum over queries i >= j + window of exp2(c * <q_i, k_j> - lse2_i)
// (or, in per-head mode, the same sum for each query head on its own)
// with c = scale * log2(e) and lse2 = LSE * log2(e): the un-normalised future
// mass of KVpop (§3.1 Eq. 2, App. B.1) recovered from the per-query LSE as in
// its §3.2 Eq. 8, without any S x S map.
//
// Work decomposition (keys stationary, queries streamed):
//   * one workgroup = 8 waves = 512 consecutive keys of one (batch, KV head),
//     one workgroup per CU (two waves of the same workgroup per SIMD, so the
//     co-resident waves advance together and a tile's time follows its work;
//     two workgroups on one CU issue at very different rates, oldest first);
//     grids too small for two workgroups per CU use 4 waves = 256 keys, or,
//     where paired tiles fill whole rounds, 4 waves of one 32-row block
//     each = 128 keys (each step then takes two staged pairs, and the copies
//     go two stages ahead: one wave per SIMD has nothing to cover a wait);
//     each wave keeps its 64 (32) keys (32-row MFMA blocks, all of d) as
//     bf16 A operands in registers for the whole sweep;
//   * the workgroup sweeps the future (query block, head) pairs of its group
//     -- query blocks of 32 from the end of the sequence backwards, the G
//     heads of a block consecutively -- one pair per wave per LDS stage,
//     double buffered; wave w stages pair w of every stage, and every staged
//     pair feeds all keys of the workgroup;
//   * in LDS a pair is stored as the MFMA B operands themselves: per 16-wide
//     slice of d, 1 KB holding lane l's 16 bytes at 16 l, copied from HBM
//     through VGPRs in two halves, so every operand read is one contiguous,
//     bank-conflict-free ds_read_b128;
//   * per pair and wave: 16 MFMA 32x32x16 give a 64 x 32 logit tile; each
//     lane applies fma + exp2 + add to its 32 values and keeps 32 per-key
//     partial sums (its query column) in registers;
//   * software pipeline inside each wave: the MFMAs of pair p+1 are issued
//     between the VALU operations of pair p (one MFMA per six VALU
//     operations), so the matrix cores and the VALU work at the same time;
//   * at the end the 32 column partials of each key are added in LDS in a
//     fixed order and each key's mass is written once: no atomics, bitwise
//     reproducible.
// Blocks are mapped XCD-aware: all tiles of one (batch, KV head) run on the
// same XCD and sweep the same Q rows at the same time (shared L2).
// Grids of one workgroup per CU whose tile pairs fill whole rounds of the CUs
// give each workgroup two tiles, m and n_tiles - 1 - m (a long and a short
// band of the triangle: equal work for every workgroup, so no round waits on
// the order in which the hardware hands out workgroups); the second tile
// sweeps its query blocks upwards, which keeps the second tiles of all
// workgroups on the same rows at the same time.  Such grids take whole units
// per round of an XCD's CUs; other grids run single tiles, longest first, so
// the triangular work load balances.
#include <type_traits>

#include "kvp_device.h"
#include "kvp_launch.h"

namespace kvp {
namespace {

template <int D, int W, int KB>
struct MassCfg {
  static constexpr int kWaves = W;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kKeyBlocks = KB;                 // 32-row key blocks per wave
  static constexpr int kKeysPerWave = 32 * KB;
  static constexpr int kKeysPerWG = kWaves * kKeysPerWave;
  static constexpr int kKSteps = D / 16;                // 16-wide slices of d
  static constexpr int kFragBytes = kWave * 16;         // one B operand (1 KB)
  static constexpr int kSlotBytes = kKSteps * kFragBytes;
  static constexpr int kSlots = kWaves;                 // wave w stages slot w
  static constexpr int kStageBytes = kSlots * kSlotBytes;
  static constexpr int kMfmaPerPair = KB * kKSteps;
  // per value: fma and add on the VALU, exp2 on the transcendental unit
  static constexpr int kAluPerPair = 2 * 16 * KB;
  static constexpr int kTransPerPair = 16 * KB;
  // LDS reads issued before a pair's first MFMA (its lse2 and the first
  // operands); the rest go out one after every KB-th MFMA
  static constexpr int kReadsAhead = KB == 1 ? 4 : 3;
  // One key block per wave makes a step half as long, too short to cover
  // the copies' latency: they are issued two stages ahead instead.
  static constexpr bool kDeep = KB == 1;
  static constexpr int kRedStride = 33;                 // column partials per key (+1 pad)
  static constexpr int kRedWaveFloats = kKeysPerWave * kRedStride;
  // the final reduction reuses the two stage buffers when they hold every
  // wave's partials
  static constexpr int kRedWavesPerBuf = kStageBytes / (kRedWaveFloats * 4);
  static constexpr bool kRedInStage = 2 * kRedWavesPerBuf >= kWaves;
};

struct MassArgs {
  const void* q;
  const void* k;
  const float* lse;
  float* mass;
  int B, Hq, Hkv, S, G, window;
  int per_head;  // 0: one unit per (batch, KV head), masses summed over its G
                 // query heads; 1: one unit per (batch, query head)
  int head_split;  // 1, or 2: the G heads of a group in two halves, each added
                   // into the zeroed output by an atomic (two terms: the sum
                   // does not depend on their order)
  int n_tiles;     // key tiles per unit (paired mode: block x sweeps key tiles
                   // x' and n_tiles - 1 - x' of its unit, x' the tile index
                   // the block mapping gives)
  float c;       // scale * log2(e)
  // query-block mode: blocks [seg_start + t seg_len, ...) clipped to S, both
  // multiples of 32; per block the mean over its rows and the unit's heads
  // (seg_block, may be null) and its suffix maximum (seg_future)
  int seg_start, seg_len, n_seg;
  float* seg_block;
  float* seg_future;
  // query-chunk mode (chunk_pairs > 0, one tile per block, no head split):
  // the sweep of key tile t, n_t = (query blocks it sees) * G pairs, is cut
  // into ceil(n_t / chunk_pairs) chunks of chunk_pairs pairs (a multiple of
  // G: whole query blocks), from the last query block down; block x of the
  // grid takes chunk x / n_units of unit x % n_units (chunks of a unit
  // numbered tile by tile) and writes its tile's partial masses to
  // partial[(unit * chunks_per_unit + chunk) * kKeysPerWG + key - tile start]
  int chunk_pairs, chunks_per_unit;
  float* partial;
};

// Query blocks seen by key tile `tile` of kpt keys: [qb_lo, qb_hi], or none
// (returns 0).  Pairs = blocks * heads.
__host__ __device__ __forceinline__ int tile_query_blocks(int tile, int kpt, int S, int window) {
  const int q_first = tile * kpt + window;
  return q_first < S ? (S - 1) / kBlk - q_first / kBlk + 1 : 0;
}

struct Tile {
  f32x16_t s0, s1;  // logits of key blocks 0 / 1 (rows) x 32 queries (columns);
                    // one key block per wave: key block 0 x slots A / B
  float l2;         // lse2 of this lane's query column (slot A)
  float l2b;        // one key block per wave: the same for slot B
};

// Sum of a 16-value register row over the 32 lanes of a wave half (lanes
// l and l ^ 16, ^ 8, ... with equal bit 5) by halving exchanges: afterwards
// lane l holds the total of value v = (l & 31) >> 1 (lanes 2m and 2m+1 hold
// the same total).  The inputs are consumed.
__device__ __forceinline__ float reduce_columns(f32x16_t& x, int l32) {
#pragma unroll
  for (int half = 8, bit = 4; half >= 1; half >>= 1, --bit) {
    const bool upper = (l32 >> bit) & 1;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float lo = x[i], hi = x[i + half];
      const float send = upper ? lo : hi;
      const float keep = upper ? hi : lo;
      x[i] = keep + __shfl_xor(send, 1 << bit);
    }
  }
  return x[0] + __shfl_xor(x[0], 1);
}

// kSeg: 0 future masses; 1 query-block mode, a block's sums reduced and
// written after the step that ends it; 2 query-block mode with every block
// edge after the last step of a stage (blocks of whole stages of pairs; the
// sweep starts with as many uncomputed query blocks as that takes), so the
// steps carry no reduction and keep their MFMA/VALU interleave.
template <int D, typename T, int W, int KB, int kSeg, bool kPair>
__global__ __launch_bounds__(kWave * W, 8 / W) void mass_kernel(MassArgs a) {
  static_assert(KB == 2 || (KB == 1 && !kSeg), "one key block per wave: mass mode only");
  using C = MassCfg<D, W, KB>;
  __shared__ __attribute__((aligned(1024))) unsigned char q_lds0[C::kStageBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char q_lds1[C::kStageBytes];
  __shared__ float l_lds0[C::kSlots * kBlk];
  __shared__ float l_lds1[C::kSlots * kBlk];
  __shared__ float red_extra[C::kRedInStage ? 1 : C::kWaves * C::kRedWaveFloats];

  const int S = a.S, w = a.window;
  // A unit is a (batch, KV head) whose G query heads are swept together, or
  // in per-head mode a single (batch, query head) with the keys of its KV head.
  const int n_heads_out = a.per_head ? a.Hq : a.Hkv;
  const int split = a.head_split;
  const int G = a.per_head ? 1 : a.G / split;  // query heads swept per unit
  int unit, tile;
  // query-chunk mode: this block's chunk, its first query block from the
  // top of the tile's sweep and its number of query blocks
  int chunk_id = 0, chunk_qb_skip = 0, chunk_qbs = 0;
  // paired grids carry equal work per block: whole units per round of an
  // XCD; otherwise longest tiles first
  if constexpr (kPair) {
    xcd_map_units(blockIdx.x, a.B * n_heads_out * split, (a.n_tiles + 1) / 2, unit, tile);
  } else if (!kSeg && KB == 2 && a.chunk_pairs > 0) {
    const int n_units = a.B * n_heads_out;
    unit = (int)blockIdx.x % n_units;
    int local = (int)blockIdx.x / n_units;
    chunk_id = unit * a.chunks_per_unit + local;
    const int qb_per_chunk = a.chunk_pairs / G;
    tile = 0;
    for (int t = 0; t < a.n_tiles; ++t) {
      const int qbs = tile_query_blocks(t, C::kKeysPerWG, S, w);
      const int nc = (qbs + qb_per_chunk - 1) / qb_per_chunk;
      if (local < nc) {
        tile = t;
        chunk_qb_skip = local * qb_per_chunk;
        chunk_qbs = min(qb_per_chunk, qbs - chunk_qb_skip);
        break;
      }
      local -= nc;
    }
  } else {
    xcd_map(blockIdx.x, a.B * n_heads_out * split, unit, tile);
  }
  const bool chunked = !kSeg && !kPair && KB == 2 && a.chunk_pairs > 0;
  const int part = unit % split;
  unit /= split;
  const int b = unit / n_heads_out;
  const int ho = unit - b * n_heads_out;                  // output row within the batch
  const int h = a.per_head ? ho / a.G : ho;               // KV head
  const int g0 = a.per_head ? ho : ho * a.G + part * G;   // first query head swept
  // Paired mode: the workgroup sweeps key tile `tile` and then tile
  // n_tiles - 1 - tile of the same unit.  The two add up to the same work for
  // every workgroup (a long and a short column band of the triangle), so the
  // grid needs no second round whose start depends on the order in which the
  // hardware hands out workgroups.
  const int tile_last = kPair ? a.n_tiles - 1 - tile : tile;
  const int n_rep = tile_last != tile ? 2 : 1;
  // unrolled: each tile's sweep is compiled for its own direction, which
  // leaves the query-block modes room for their column reductions
#pragma unroll
  for (int rep = 0; rep < 2; ++rep) {
  if (rep == n_rep) break;
  // the previous tile's column reduction has read the stage buffers
  if (rep) __syncthreads();
  // lane indices are re-derived per tile from an opaque copy of the thread
  // id, so that nothing computed from them stays live across both tiles
  int tid = threadIdx.x;
  if constexpr (kPair) asm volatile("" : "+v"(tid));
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;  // query column / key row within a 32-block
  const int h32 = lane >> 5;  // which 8-element half of a 16-wide slice of d
  const int tile_key0 = (rep ? tile_last : tile) * C::kKeysPerWG;
  const int key0 = tile_key0 + wave * C::kKeysPerWave;

  const T* __restrict__ kbase = static_cast<const T*>(a.k) + (size_t)(b * a.Hkv + h) * S * D;
  const T* __restrict__ qgroup = static_cast<const T*>(a.q) + (size_t)(b * a.Hq + g0) * S * D;
  const float* __restrict__ lgroup = a.lse + (size_t)(b * a.Hq + g0) * S;
  const uint32_t head_bytes = (uint32_t)S * D * sizeof(T);

  // Stationary keys: A operands of the wave's 32-row blocks, all slices of d.
  u32x4_t kf[KB][C::kKSteps];
  {
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase, head_bytes);
#pragma unroll
    for (int rb = 0; rb < KB; ++rb)
#pragma unroll
      for (int ks = 0; ks < C::kKSteps; ++ks)  // keys >= S read 0
        kf[rb][ks] = buf_load8(kr, (uint32_t)(key0 + 32 * rb + l32) * D + 16 * ks + 8 * h32,
                               static_cast<const T*>(nullptr));
    // wait here once, so that no use of the keys inside the sweep waits on
    // the loads of the stage copies in flight
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  }

  f32x16_t acc0 = {}, acc1 = {};
  const float c = a.c;
  // first query any key of the tile can see (in query-block mode, and that
  // belongs to a block)
  const int q_first = kSeg ? max(tile_key0 + w, a.seg_start) : tile_key0 + w;

  // The query blocks are swept from the last one down, except in the second
  // tile of a paired workgroup, which sweeps them upwards from the first block
  // it sees: the second tiles of all workgroups start at staggered times, and
  // sweeping upwards puts all of them on the same query rows at the same time
  // (shared L2), as the first tiles are while they sweep down.
  const bool asc = kPair && rep == 1;

  // query-block mode: per-key running maxima of the blocks flushed so far
  // (block scores are >= 0), the lowest block flushed, and the key rows this
  // lane writes after a column reduction
  float fmax0 = 0.f, fmax1 = 0.f;
  int seg_low = a.n_seg;
  const int red_row = 8 * ((l32 >> 1) >> 2) + 4 * h32 + ((l32 >> 1) & 3);
  const size_t seg_row0 = (size_t)(b * n_heads_out + ho) * a.n_seg;
  // stores through buffer resources over one output row: the row base stays
  // scalar, keys >= S fall outside the resource and are dropped
  auto write_seg = [&](int t, float v0, float v1) __attribute__((always_inline)) {
    if (l32 & 1) return;
    const size_t o = (seg_row0 + t) * S;
    const uint32_t off0 = (uint32_t)(key0 + red_row) * 4u;
    const uint32_t row_bytes = (uint32_t)S * 4u;
    if (a.seg_block) {
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.seg_block + o, row_bytes);
      buf_store_f32(rb, off0, v0);
      buf_store_f32(rb, off0 + 128u, v1);
    }
    const __amdgpu_buffer_rsrc_t rf = make_rsrc(a.seg_future + o, row_bytes);
    buf_store_f32(rf, off0, fmax0);
    buf_store_f32(rf, off0 + 128u, fmax1);
  };
  // upward sweep: a block's mean is parked in its future row until the
  // running maximum can be taken from the last block down
  auto write_raw = [&](int t, float v0, float v1) __attribute__((always_inline)) {
    if (l32 & 1) return;
    const __amdgpu_buffer_rsrc_t rf = make_rsrc(a.seg_future + (seg_row0 + t) * S, (uint32_t)S * 4u);
    const uint32_t off0 = (uint32_t)(key0 + red_row) * 4u;
    buf_store_f32(rf, off0, v0);
    buf_store_f32(rf, off0 + 128u, v1);
  };
  auto flush_seg = [&](int t) __attribute__((always_inline)) {
    const int i0 = a.seg_start + t * a.seg_len;
    const int rows = min(S, i0 + a.seg_len) - i0;
    const float inv = 1.f / (float)(rows * G);
    const float v0 = reduce_columns(acc0, l32) * inv;
    const float v1 = reduce_columns(acc1, l32) * inv;
    acc0 = f32x16_t{};
    acc1 = f32x16_t{};
    if (asc) {
      write_raw(t, v0, v1);
    } else {
      fmax0 = fmaxf(fmax0, v0);
      fmax1 = fmaxf(fmax1, v1);
      write_seg(t, v0, v1);
    }
    seg_low = min(seg_low, t);
  };

  if (q_first < S && (!chunked || chunk_qbs > 0)) {
    // a chunk sweeps query blocks [qb_hi - skip - qbs + 1, qb_hi - skip]
    const int qb_last = (S - 1) / kBlk;
    const int qb_hi = chunked ? qb_last - chunk_qb_skip : qb_last;
    const int qb_lo = chunked ? qb_hi - chunk_qbs + 1 : q_first / kBlk;
    // Stage-aligned query-block mode: pad_qb query blocks beyond the sweep's
    // start (rows past S going down, below the first seen row going up),
    // staged but computed by no wave, make the first block's pairs, and so
    // every later block edge, end a stage.  seg_first: the block swept
    // first; first_qbs: its query blocks in the sweep.
    int pad_qb = 0, seg_first = 0, first_qbs = 0;
    if constexpr (kSeg == 2) {
      seg_first = ((asc ? qb_lo : qb_hi) * kBlk - a.seg_start) / a.seg_len;
      const int edge_qb = (a.seg_start + (seg_first + (asc ? 1 : 0)) * a.seg_len) / kBlk;
      first_qbs = asc ? edge_qb - qb_lo : qb_hi - edge_qb + 1;
      while (((pad_qb + first_qbs) * G) % C::kSlots) ++pad_qb;  // < kSlots steps
    }
    const int n_pairs = (qb_hi - qb_lo + 1 + pad_qb) * G;
    const int pad_pairs = pad_qb * G;
    // Pair p is (query block qb_first + qb_step * (p / G), head p % G).
    const int qb_step = asc ? 1 : -1;
    const int qb_first = asc ? qb_lo - pad_qb : qb_hi + pad_qb;
    // query-block mode: after the last pair of a block (its last head, and
    // its first query block going down or its last going up) or the last
    // pair of the sweep, reduce and write
    auto maybe_flush = [&](int p) __attribute__((always_inline)) {
      if constexpr (kSeg == 1) {
        if (p >= n_pairs) return;
        const int qrow = (qb_first + qb_step * (p / G)) * kBlk - a.seg_start;
        const bool edge = asc ? (qrow + kBlk) % a.seg_len == 0 : qrow % a.seg_len == 0;
        if (p == n_pairs - 1 || (p % G == G - 1 && edge)) flush_seg(qrow / a.seg_len);
      }
    };
    // stage-aligned query-block mode: after the last step of a stage, the
    // block whose last pair that is, or the sweep's last block
    int next_edge = (pad_qb + first_qbs) * G - 1, seg_cur = seg_first;
    const int pairs_per_seg = a.seg_len / kBlk * G;
    auto stage_flush = [&](int p_end) __attribute__((always_inline)) {
      if constexpr (kSeg == 2) {
        if (p_end >= next_edge || p_end >= n_pairs - 1) {
          flush_seg(seg_cur);
          seg_cur += qb_step;
          next_edge += pairs_per_seg;
        }
      }
    };
    const int n_stages = (n_pairs + C::kSlots - 1) / C::kSlots;
    // For this wave, pairs [p_vis_lo, p_vis_hi) see at least one query;
    // those in [p_full_lo, p_full_hi) see every key with every query (no
    // mask), the others need the mask.  A partial last block (rows >= S) is
    // masked too.
    // (the padding pairs lie before p_vis_lo)
    const int p_part = (S % kBlk) && qb_hi == qb_last ? G : 0;
    const int qb_full = (key0 + C::kKeysPerWave - 1 + w + kBlk - 1) / kBlk;
    const int qb_min = (key0 + w) / kBlk;  // first block with a query i >= key0 + w
    const int p_vis_lo = asc ? min(n_pairs, pad_pairs + max(0, qb_min - qb_lo) * G) : pad_pairs;
    const int p_vis_hi = asc ? n_pairs : max(0, min(n_pairs, (qb_first - qb_min + 1) * G));
    const int p_full_lo = asc ? min(n_pairs, pad_pairs + max(0, qb_full - qb_lo) * G)
                              : pad_pairs + p_part;
    const int p_full_hi = asc ? n_pairs - p_part : max(0, min(n_pairs, (qb_first - qb_full + 1) * G));

    // ---- staging: this wave copies pair kSlots * st + wave of stage st
    int ld_qb = qb_first + qb_step * (wave / G);
    int ld_g = wave % G;
    auto advance = [&](int& qb, int& g) __attribute__((always_inline)) {
      g += C::kSlots;
      while (g >= G) {
        g -= G;
        qb += qb_step;
      }
    };
    // Copies go HBM -> VGPR -> LDS in two halves of the d slices, so that
    // only 4 x 16 bytes per lane are in flight in registers at a time.
    constexpr int kHalf = C::kKSteps / 2;
    u32x4_t stage_regs[kHalf];
    float lse_pref = 0.f;
    auto issue_loads = [&](int st, int half) __attribute__((always_inline)) {
      if (st * C::kSlots + wave >= n_pairs) return;
      if (half == 0 && lane < kBlk) {
        const int i = ld_qb * kBlk + lane;  // < 0: padding below the sweep
        lse_pref = (kSeg != 2 || i >= 0) && i < S ? lgroup[(size_t)ld_g * S + i] : 0.f;
      }
      const __amdgpu_buffer_rsrc_t qr = make_rsrc(qgroup + (size_t)ld_g * S * D, head_bytes);
      const uint32_t e0 = (uint32_t)(ld_qb * kBlk + l32) * D + 8 * h32;
#pragma unroll
      for (int t = 0; t < kHalf; ++t)  // rows >= S read 0
        stage_regs[t] = buf_load8(qr, e0 + 16 * (half * kHalf + t), static_cast<const T*>(nullptr));
    };
    auto store_half = [&](int st, int half, unsigned char* qdst) __attribute__((always_inline)) {
      if (st * C::kSlots + wave >= n_pairs) return;
      unsigned char* slot = qdst + wave * C::kSlotBytes + lane * 16;
#pragma unroll
      for (int t = 0; t < kHalf; ++t)
        *reinterpret_cast<u32x4_t*>(slot + (half * kHalf + t) * C::kFragBytes) = stage_regs[t];
    };
    auto finish_loads = [&](int st, float* ldst) __attribute__((always_inline)) {
      const bool valid = st * C::kSlots + wave < n_pairs;
      if (lane < kBlk) {
        const int i = ld_qb * kBlk + lane;
        // no query (row beyond S or no pair): exp2(x - inf) = 0
        ldst[wave * kBlk + lane] =
            (valid && (kSeg != 2 || i >= 0) && i < S) ? lse_pref * kLog2e : __builtin_inff();
      }
      advance(ld_qb, ld_g);  // the pair this wave stages in the next stage
    };
    // Two stages ahead (one key block per wave): a stage's copies are issued
    // whole at the start of the stage two before it, into one of two register
    // sets, and stored to LDS just before the barrier of the stage before it.
    // Loads and stores are unconditional (a pair past the sweep reads zeros
    // through an empty resource and fills a slot no MFMA reads), so the
    // store waits only for its own set.
    u32x4_t deep_regs[2][C::kDeep ? C::kKSteps : 1];
    float deep_lse[2] = {0.f, 0.f};
    int deep_qb[2] = {0, 0};
    auto deep_issue = [&](auto setc, int st) __attribute__((always_inline)) {
      if constexpr (C::kDeep) {
        constexpr int kSet = decltype(setc)::value;
        const bool valid = st * C::kSlots + wave < n_pairs;
        deep_qb[kSet] = ld_qb;
        const __amdgpu_buffer_rsrc_t lr =
            make_rsrc(lgroup + (size_t)ld_g * S, valid ? (uint32_t)S * 4u : 0u);
        deep_lse[kSet] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(lr, (uint32_t)(ld_qb * kBlk + l32) * 4u, 0, 0));
        const __amdgpu_buffer_rsrc_t qr =
            make_rsrc(qgroup + (size_t)ld_g * S * D, valid ? head_bytes : 0u);
        const uint32_t e0 = (uint32_t)(ld_qb * kBlk + l32) * D + 8 * h32;
#pragma unroll
        for (int t = 0; t < C::kKSteps; ++t)  // rows >= S read 0
          deep_regs[kSet][t] = buf_load8(qr, e0 + 16 * t, static_cast<const T*>(nullptr));
        advance(ld_qb, ld_g);
      }
    };
    auto deep_store = [&](auto setc, int st, unsigned char* qdst, float* ldst)
                          __attribute__((always_inline)) {
      if constexpr (C::kDeep) {
        constexpr int kSet = decltype(setc)::value;
        const bool valid = st * C::kSlots + wave < n_pairs;
        unsigned char* slot = qdst + wave * C::kSlotBytes + lane * 16;
#pragma unroll
        for (int t = 0; t < C::kKSteps; ++t)
          *reinterpret_cast<u32x4_t*>(slot + t * C::kFragBytes) = deep_regs[kSet][t];
        if (lane < kBlk) {
          const int i = deep_qb[kSet] * kBlk + lane;
          ldst[wave * kBlk + lane] = (valid && i < S) ? deep_lse[kSet] * kLog2e : __builtin_inff();
        }
      }
    };

    // ---- compute
    auto mfma_pair = [&](Tile& t, const unsigned char* qsrc, const float* lsrc, int slot)
                         __attribute__((always_inline)) {
      const unsigned char* src = qsrc + slot * C::kSlotBytes + lane * 16;
      t.l2 = lsrc[slot * kBlk + l32];
#pragma unroll
      for (int ks = 0; ks < C::kKSteps; ++ks) {
        const u32x4_t bq = *reinterpret_cast<const u32x4_t*>(src + ks * C::kFragBytes);
        t.s0 = mfma_32x32x16(kf[0][ks], bq, ks ? t.s0 : f32x16_t{});
        if constexpr (KB == 2) t.s1 = mfma_32x32x16(kf[KB >= 2 ? 1 : 0][ks], bq, ks ? t.s1 : f32x16_t{});
      }
    };
    auto exp_full = [&](const Tile& t) __attribute__((always_inline)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc0[v] += fast_exp2(__builtin_fmaf(t.s0[v], c, -t.l2));
        if constexpr (KB == 2) acc1[v] += fast_exp2(__builtin_fmaf(t.s1[v], c, -t.l2));
      }
    };
    auto exp_masked = [&](const Tile& t, int p) __attribute__((always_inline)) {
      // query i counts for key j = key0 + 32 b + 8 (v / 4) + 4 h32 + v % 4 iff
      // i >= j + w, i.e. iff the constant 8 (v / 4) + v % 4 <= lim - 32 b
      const int lim = (qb_first + qb_step * (p / G)) * kBlk + l32 - key0 - w - 4 * h32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + (v & 3);
        const float x0 = __builtin_fmaf(t.s0[v], c, -t.l2);
        acc0[v] += fast_exp2(r <= lim ? x0 : -__builtin_inff());
        if constexpr (KB == 2) {
          const float x1 = __builtin_fmaf(t.s1[v], c, -t.l2);
          acc1[v] += fast_exp2(r + 32 <= lim ? x1 : -__builtin_inff());
        }
      }
    };
    // Exponentials of pair p (in cur) and MFMAs of pair p + 1 (into nxt).
    auto step = [&](Tile& cur, Tile& nxt, int p, const unsigned char* nq, const float* nl,
                    int nslot) __attribute__((always_inline)) {
      const bool m_ok = p + 1 >= p_vis_lo && p + 1 < p_vis_hi;
      const bool full = p >= p_full_lo && p < p_full_hi;
      if (m_ok && full) {
        mfma_pair(nxt, nq, nl, nslot);
        exp_full(cur);
        // issue order: operand reads ahead, then each MFMA followed by its
        // share of the VALU work (at d = 128: two fma, two add, two exp2),
        // one more operand read after every KB-th MFMA.  The scheduler
        // counts exp2 as transcendental (0x400), not VALU (0x002): without
        // its own group the exps ride along and the last MFMAs of the pair
        // go out with no VALU work beside them.
        __builtin_amdgcn_sched_group_barrier(0x100, C::kReadsAhead, 0);
#pragma unroll
        for (int m = 0; m < C::kMfmaPerPair; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, C::kAluPerPair / C::kMfmaPerPair, 0);
          __builtin_amdgcn_sched_group_barrier(0x400, C::kTransPerPair / C::kMfmaPerPair, 0);
          if (m % KB == KB - 1 && m < KB * (C::kKSteps + 1 - C::kReadsAhead))
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else {
        if (m_ok) mfma_pair(nxt, nq, nl, nslot);
        if (full)
          exp_full(cur);
        else if (p >= p_vis_lo && p < p_vis_hi)
          exp_masked(cur, p);
      }
    };

    // One key block per wave: a step takes two pairs (two staged slots), so
    // that each step has two independent MFMA chains (one per slot) like the
    // two key blocks of the other configurations; a single wave per SIMD
    // issues a lone accumulation chain about 40% slower.  The exponentials of
    // slot B go to the second set of accumulators.
    auto mfma_two = [&](Tile& t, const unsigned char* qsrc, const float* lsrc, int slot)
                        __attribute__((always_inline)) {
      const unsigned char* src = qsrc + slot * C::kSlotBytes + lane * 16;
      t.l2 = lsrc[slot * kBlk + l32];
      t.l2b = lsrc[(slot + 1) * kBlk + l32];
#pragma unroll
      for (int ks = 0; ks < C::kKSteps; ++ks) {
        const u32x4_t ba = *reinterpret_cast<const u32x4_t*>(src + ks * C::kFragBytes);
        const u32x4_t bb = *reinterpret_cast<const u32x4_t*>(src + C::kSlotBytes + ks * C::kFragBytes);
        t.s0 = mfma_32x32x16(kf[0][ks], ba, ks ? t.s0 : f32x16_t{});
        t.s1 = mfma_32x32x16(kf[0][ks], bb, ks ? t.s1 : f32x16_t{});
      }
    };
    auto exp_two_full = [&](const Tile& t) __attribute__((always_inline)) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc0[v] += fast_exp2(__builtin_fmaf(t.s0[v], c, -t.l2));
        acc1[v] += fast_exp2(__builtin_fmaf(t.s1[v], c, -t.l2b));
      }
    };
    // one slot of a two-slot tile: B selects s1 / l2b / acc1
    auto exp_one = [&](const Tile& t, bool b_slot, int p, bool full) __attribute__((always_inline)) {
      const int lim = (qb_first + qb_step * (p / G)) * kBlk + l32 - key0 - w - 4 * h32;
      const float l2 = b_slot ? t.l2b : t.l2;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 8 * (v >> 2) + (v & 3);
        const float x = __builtin_fmaf(b_slot ? t.s1[v] : t.s0[v], c, -l2);
        const float e = fast_exp2(full || r <= lim ? x : -__builtin_inff());
        if (b_slot)
          acc1[v] += e;
        else
          acc0[v] += e;
      }
    };
    // Exponentials of pairs p, p + 1 (in cur) and MFMAs of pairs p + 2, p + 3
    // (slots nslot, nslot + 1, into nxt).
    auto step2 = [&](Tile& cur, Tile& nxt, int p, const unsigned char* nq, const float* nl,
                     int nslot) __attribute__((always_inline)) {
      if constexpr (KB == 1) {
        auto vis = [&](int x) { return x >= p_vis_lo && x < p_vis_hi; };
        auto ful = [&](int x) { return x >= p_full_lo && x < p_full_hi; };
        const bool m_a = vis(p + 2), m_b = vis(p + 3);
        if (m_a && m_b && ful(p) && ful(p + 1)) {
          mfma_two(nxt, nq, nl, nslot);
          exp_two_full(cur);
          // issue order: six reads ahead (both lse2 and the first two
          // slices of each slot), then each MFMA with its share of the VALU
          // work and one more read
          __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
          for (int m = 0; m < 2 * C::kKSteps; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);
            if (m < 2 * C::kKSteps - 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        } else {
          // pairs past the sweep compute on whatever the slot holds, unused
          if (m_a || m_b) mfma_two(nxt, nq, nl, nslot);
          if (vis(p)) exp_one(cur, false, p, ful(p));
          if (vis(p + 1)) exp_one(cur, true, p + 1, ful(p + 1));
        }
      }
    };

    Tile t0, t1;
    // One stage: the exponentials of its kSlots pairs; the MFMAs of each next
    // pair are issued one step ahead, the last step's from the other buffer
    // once the barrier has published it.  The copies for the next stage are
    // issued at the start and stored in two halves further on, so each half
    // has a few steps to arrive.
    static_assert(C::kSlots % 2 == 0 && C::kSlots >= 4, "tile ping-pong needs an even stage");
    constexpr int kStoreA = C::kSlots == 8 ? 1 : 0;  // store half 0 after this step
    constexpr int kStoreB = C::kSlots == 8 ? 3 : 2;  // store half 1 after this step
    static_assert(kStoreA < kStoreB && kStoreB <= C::kSlots - 2,
                  "both halves must be stored before the stage's last step");
    auto stage = [&](auto bufc, int st) __attribute__((always_inline)) {
      constexpr int kBuf = decltype(bufc)::value;
      unsigned char* cq = kBuf ? q_lds1 : q_lds0;
      unsigned char* nq = kBuf ? q_lds0 : q_lds1;
      float* cl = kBuf ? l_lds1 : l_lds0;
      float* nl = kBuf ? l_lds0 : l_lds1;
      const bool more = st + 1 < n_stages;
      const int p0 = st * C::kSlots;
      if constexpr (C::kDeep) {
        // register set kBuf is free (stored at the end of the previous
        // stage); set 1 - kBuf holds the next stage's copies.  No condition
        // on either: past the last stage they read and store nothing used.
        deep_issue(bufc, st + 2);
        // two steps of two slots: the first's MFMAs take slots 2 and 3, the
        // second's slots 0 and 1 of the next stage, after the barrier
        static_assert(C::kSlots == 4, "one key block per wave: four-wave workgroups");
        step2(t0, t1, p0, cq, cl, 2);
        deep_store(std::integral_constant<int, 1 - kBuf>{}, st + 1, nq, nl);
        __syncthreads();
        step2(t1, t0, p0 + 2, nq, nl, 0);
        return;
      }
      if (more) issue_loads(st + 1, 0);
#pragma unroll
      for (int j = 0; j < C::kSlots - 1; ++j) {
        if (j & 1)
          step(t1, t0, p0 + j, cq, cl, j + 1);
        else
          step(t0, t1, p0 + j, cq, cl, j + 1);
        maybe_flush(p0 + j);
        if (more && j == kStoreA) {
          store_half(st + 1, 0, nq);
          issue_loads(st + 1, 1);
        }
        if (more && j == kStoreB) {
          store_half(st + 1, 1, nq);
          finish_loads(st + 1, nl);
        }
      }
      __syncthreads();
      step(t1, t0, p0 + C::kSlots - 1, nq, nl, 0);
      maybe_flush(p0 + C::kSlots - 1);
      stage_flush(p0 + C::kSlots - 1);
    };

    if constexpr (C::kDeep) {
      deep_issue(std::integral_constant<int, 0>{}, 0);
      deep_issue(std::integral_constant<int, 1>{}, 1);
      deep_store(std::integral_constant<int, 0>{}, 0, q_lds0, l_lds0);
    } else {
      issue_loads(0, 0);
      store_half(0, 0, q_lds0);
      issue_loads(0, 1);
      store_half(0, 1, q_lds0);
      finish_loads(0, l_lds0);
    }
    __syncthreads();
    if constexpr (C::kDeep) {
      if (p_vis_lo <= 1 && 0 < p_vis_hi) mfma_two(t0, q_lds0, l_lds0, 0);
    } else {
      if (p_vis_lo <= 0 && 0 < p_vis_hi) mfma_pair(t0, q_lds0, l_lds0, 0);
    }
    for (int st = 0; st < n_stages; st += 2) {
      stage(std::integral_constant<int, 0>{}, st);
      if (st + 1 >= n_stages) break;
      stage(std::integral_constant<int, 1>{}, st + 1);
    }
  }

  if constexpr (kSeg) {
    if (asc && seg_low < a.n_seg) {
      // upward sweep: wait for the parked block means, read them back (the
      // stores have reached L2; this wave never read those lines before) and
      // write block scores and running maxima from the last block down,
      // sixteen blocks' loads in flight at a time
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      const uint32_t off0 = (uint32_t)(key0 + red_row) * 4u;
      constexpr int kBatch = 16;
      for (int t_hi = a.n_seg - 1; t_hi >= seg_low; t_hi -= kBatch) {
        float p0[kBatch], p1[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int t = max(t_hi - u, seg_low);
          const __amdgpu_buffer_rsrc_t rf =
              make_rsrc(a.seg_future + (seg_row0 + t) * S, (uint32_t)S * 4u);
          p0[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rf, off0, 0, 0));
          p1[u] = __builtin_bit_cast(float,
                                     __builtin_amdgcn_raw_buffer_load_b32(rf, off0 + 128u, 0, 0));
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int t = t_hi - u;
          if (t < seg_low) break;
          fmax0 = fmaxf(fmax0, p0[u]);
          fmax1 = fmaxf(fmax1, p1[u]);
          write_seg(t, p0[u], p1[u]);
        }
      }
    }
    // blocks wholly before the first query the tile sees: no attention, and
    // the future score is the maximum of the later blocks
    for (int t = seg_low - 1; t >= 0; --t) write_seg(t, 0.f, 0.f);
    continue;
  }

  // Column reduction: each lane holds one query column's partial sums for 32
  // keys per block; add the 32 columns of every key in LDS in a fixed order.
  __syncthreads();
  float* red;
  if constexpr (C::kRedInStage) {
    constexpr int kPer = C::kRedWavesPerBuf;
    red = reinterpret_cast<float*>(wave < kPer ? q_lds0 : q_lds1) +
          (wave < kPer ? wave : wave - kPer) * C::kRedWaveFloats;
  } else
    red = red_extra + wave * C::kRedWaveFloats;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int kl = mfma_row(v, lane);
    if constexpr (KB == 2) {
      red[kl * C::kRedStride + l32] = acc0[v];
      red[(kl + 32) * C::kRedStride + l32] = acc1[v];
    } else {
      red[kl * C::kRedStride + l32] = acc0[v] + acc1[v];  // slots A and B
    }
  }
  __syncthreads();
  // lane = key within the wave's keys
  const int key = key0 + lane;
  if (lane < C::kKeysPerWave && key < S) {
    float tot = 0.f;
#pragma unroll
    for (int col = 0; col < 32; ++col) tot += red[lane * C::kRedStride + col];
    if (chunked) {
      if (chunk_qbs > 0) a.partial[(size_t)chunk_id * C::kKeysPerWG + (key - tile_key0)] = tot;
    } else {
      float* dst = a.mass + (size_t)(b * n_heads_out + ho) * S + key;
      if (split > 1)
        atomicAdd(dst, tot);
      else
        *dst = tot;
    }
  }
  }  // tiles of the workgroup
}

// Query-chunk mode: the mass of every key is the sum of its tile's chunk
// partials, added in chunk order (bitwise reproducible).  Keys of tiles with
// no chunk (no future query) get 0.
template <int kKeysPerTile>
__global__ __launch_bounds__(256) void mass_chunk_sum_kernel(MassArgs a, int n_units) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)n_units * a.S) return;
  const int unit = (int)(i / a.S);
  const int key = (int)(i - (int64_t)unit * a.S);
  const int t = key / kKeysPerTile;
  const int qpc = a.chunk_pairs / (a.per_head ? 1 : a.G);  // query blocks per chunk
  int off = 0;
  for (int u = 0; u < t; ++u)
    off += (tile_query_blocks(u, kKeysPerTile, a.S, a.window) + qpc - 1) / qpc;
  const int nc = (tile_query_blocks(t, kKeysPerTile, a.S, a.window) + qpc - 1) / qpc;
  const float* p = a.partial + ((size_t)unit * a.chunks_per_unit + off) * kKeysPerTile +
                   (key - t * kKeysPerTile);
  float sum = 0.f;
  for (int c = 0; c < nc; ++c) sum += p[(size_t)c * kKeysPerTile];
  a.mass[i] = sum;
}

__global__ __launch_bounds__(256) void zero_fill_kernel(float* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0.f;
}

template <int D, typename T, int W, int KB, bool kSeg>
hipError_t launch_mass_w(const void* q, const void* k, const float* lse, const Shape& sh,
                         float scale, int window, int per_head, int split, float* mass,
                         const SegOut& seg, hipStream_t stream) {
  using C = MassCfg<D, W, KB>;
  MassArgs a;
  a.q = q;
  a.k = k;
  a.lse = lse;
  a.mass = mass;
  a.B = sh.B;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.S = sh.S;
  a.G = sh.G;
  a.window = window;
  a.per_head = per_head;
  a.head_split = split;
  a.c = scale * kLog2e;
  a.seg_start = seg.start;
  a.seg_len = seg.len;
  a.n_seg = seg.n;
  a.seg_block = seg.block;
  a.seg_future = seg.future;
  a.chunk_pairs = 0;
  a.chunks_per_unit = 0;
  a.partial = nullptr;
  const int64_t n_tiles = (sh.S + C::kKeysPerWG - 1) / C::kKeysPerWG;
  const int64_t units = (int64_t)sh.B * (per_head ? sh.Hq : sh.Hkv) * split;
  a.n_tiles = (int)n_tiles;
  // One-workgroup-per-CU grids (and the one-block-per-wave grids) pair each
  // long key tile with a short one when the equal-work pairs fill whole
  // rounds of the CUs (at least 95%).
  bool pair = false;
  if ((W == 8 || KB == 1) && n_tiles >= 2) {
    const int64_t pairs = units * ((n_tiles + 1) / 2);
    const int64_t rounds = (pairs + kNumCUs - 1) / kNumCUs;
    pair = pairs * 20 >= rounds * kNumCUs * 19;
  }
  const int64_t blocks = units * (pair ? (n_tiles + 1) / 2 : n_tiles);
  if (split > 1) {
    const int64_t n = (int64_t)sh.B * sh.Hkv * sh.S;
    const int64_t fill_blocks = min((n + 255) / 256, (int64_t)4 * kNumCUs);
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)fill_blocks), dim3(256), 0, stream, mass, n);
  }
  // query-block mode with blocks of whole stages of pairs: the stage-aligned
  // kernel (block edges after the last step of a stage)
  const int g_unit = per_head ? 1 : sh.G / split;
  const bool aligned = kSeg && (int64_t)seg.len / kBlk * g_unit % C::kSlots == 0;
  auto go = [&](auto modec) -> hipError_t {
    constexpr int kMode = decltype(modec)::value;
    if constexpr (W == 8 || KB == 1) {
      if (pair) {
        hipLaunchKernelGGL((mass_kernel<D, T, W, KB, kMode, true>), dim3((unsigned)blocks),
                           dim3(C::kThreads), 0, stream, a);
        return hipGetLastError();
      }
    }
    if constexpr (KB == 2) {
      hipLaunchKernelGGL((mass_kernel<D, T, W, KB, kMode, false>), dim3((unsigned)blocks),
                         dim3(C::kThreads), 0, stream, a);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;  // one block per wave is chosen for paired grids only
  };
  if constexpr (kSeg) {
    if (aligned) return go(std::integral_constant<int, 2>{});
    return go(std::integral_constant<int, 1>{});
  } else {
    return go(std::integral_constant<int, 0>{});
  }
}

// 512-key workgroups (one per CU) when the grid has at least two per CU.
// Shorter sequences: 128-key workgroups of four waves with one key block per
// wave, each taking a long and a short tile, when those pairs fill whole
// rounds of the CUs (every wave then has the same work); otherwise 256-key
// workgroups (two per CU).  Group sums whose 256-key grid has fewer than two
// workgroups per CU also split each group's heads in two halves.
template <int D, typename T, bool kSeg>
hipError_t launch_mass_t(const void* q, const void* k, const float* lse, const Shape& sh,
                         float scale, int window, int per_head, float* mass, const SegOut& seg,
                         hipStream_t stream) {
  using C4 = MassCfg<D, 4, 2>;
  using C8 = MassCfg<D, 8, 2>;
  using C1 = MassCfg<D, 4, 1>;
  int64_t units = (int64_t)sh.B * (per_head ? sh.Hq : sh.Hkv);
  int split = 1;
  if (!kSeg && !per_head && sh.G % 2 == 0 &&
      units * ((sh.S + C4::kKeysPerWG - 1) / C4::kKeysPerWG) < 2 * kNumCUs)
    split = 2;
  units *= split;
  const int64_t blocks8 = units * ((sh.S + C8::kKeysPerWG - 1) / C8::kKeysPerWG);
  if (blocks8 >= 2 * kNumCUs)
    return launch_mass_w<D, T, 8, 2, kSeg>(q, k, lse, sh, scale, window, per_head, split, mass,
                                           seg, stream);
  if constexpr (!kSeg) {
    const int64_t tiles1 = (sh.S + C1::kKeysPerWG - 1) / C1::kKeysPerWG;
    const int64_t pairs = units * ((tiles1 + 1) / 2);
    const int64_t rounds = (pairs + kNumCUs - 1) / kNumCUs;
    if (tiles1 >= 2 && pairs * 20 >= rounds * kNumCUs * 19)
      return launch_mass_w<D, T, 4, 1, kSeg>(q, k, lse, sh, scale, window, per_head, split, mass,
                                             seg, stream);
  }
  return launch_mass_w<D, T, 4, 2, kSeg>(q, k, lse, sh, scale, window, per_head, split, mass, seg,
                                         stream);
}

// Query-chunk plan of a short-sequence launch of group sums: key tiles whose
// sweeps are cut into chunks of equal query blocks.  For one to four rounds
// of the CUs (kChunkPerRound workgroups each) the smallest chunk that fits is
// found; the plan taken has the least rounds x (chunk + a per-workgroup
// overhead of two query blocks).  chunk_qbs = 0: no chunking (large grids,
// fp32 input, or nothing to sweep).
struct ChunkPlan {
  int chunk_qbs, chunks_per_unit;
  int64_t units, n_tiles;
};
// waves per chunk workgroup (two key blocks each): 4 -> 256-key tiles, two
// workgroups per CU (measured a little faster at 4K tokens than 8 waves and
// 512-key tiles, one per CU)
constexpr int kChunkWaves = 4;
constexpr int kChunkTile = kChunkWaves * 64;
constexpr int kChunkPerRound = kNumCUs * (8 / kChunkWaves);

ChunkPlan mass_chunk_plan(int dtype, const Shape& sh, int window, int per_head) {
  ChunkPlan pl{0, 0, 0, 0};
  // per-head masses already spread over G times the units (the paired
  // one-block grid, two workgroups per CU): no chunking
  if (dtype != 0 || sh.S <= 0 || per_head) return pl;
  pl.units = (int64_t)sh.B * (per_head ? sh.Hq : sh.Hkv);
  pl.n_tiles = (sh.S + kChunkTile - 1) / kChunkTile;
  // grids of at least two 512-key tiles per CU run the paired 8-wave launch
  if (pl.units * ((sh.S + 511) / 512) >= 2 * kNumCUs) return pl;
  int64_t qmax = 0;
  for (int64_t t = 0; t < pl.n_tiles; ++t)
    qmax = max(qmax, (int64_t)tile_query_blocks((int)t, kChunkTile, sh.S, window));
  if (qmax == 0) return pl;
  auto chunks = [&](int64_t qpc) {
    int64_t n = 0;
    for (int64_t t = 0; t < pl.n_tiles; ++t)
      n += (tile_query_blocks((int)t, kChunkTile, sh.S, window) + qpc - 1) / qpc;
    return n;
  };
  int64_t best_q = qmax, best_cost = -1;
  for (int64_t rounds = 1; rounds <= 4; ++rounds) {
    // smallest chunk (in query blocks) whose grid fits `rounds` rounds;
    // the chunk count does not grow with the chunk size
    int64_t lo = 1, hi = qmax;
    if (pl.units * chunks(hi) > rounds * kChunkPerRound) continue;
    while (lo < hi) {
      const int64_t mid = (lo + hi) / 2;
      if (pl.units * chunks(mid) <= rounds * kChunkPerRound)
        hi = mid;
      else
        lo = mid + 1;
    }
    const int64_t cost = rounds * (lo + 2);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best_q = lo;
    }
  }
  pl.chunk_qbs = (int)best_q;
  pl.chunks_per_unit = (int)chunks(best_q);
  return pl;
}

template <int D, typename T>
hipError_t launch_mass_chunked_t(const void* q, const void* k, const float* lse, const Shape& sh,
                                 float scale, int window, int per_head, float* mass,
                                 const ChunkPlan& pl, void* workspace, hipStream_t stream) {
  using C = MassCfg<D, kChunkWaves, 2>;
  static_assert(C::kKeysPerWG == kChunkTile, "chunk tiles: two key blocks per wave");
  MassArgs a;
  a.q = q;
  a.k = k;
  a.lse = lse;
  a.mass = mass;
  a.B = sh.B;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.S = sh.S;
  a.G = sh.G;
  a.window = window;
  a.per_head = per_head;
  a.head_split = 1;
  a.n_tiles = (int)pl.n_tiles;
  a.c = scale * kLog2e;
  a.seg_start = 0;
  a.seg_len = 32;
  a.n_seg = 0;
  a.seg_block = nullptr;
  a.seg_future = nullptr;
  a.chunk_pairs = pl.chunk_qbs * (per_head ? 1 : sh.G);
  a.chunks_per_unit = pl.chunks_per_unit;
  a.partial = static_cast<float*>(workspace);
  const int64_t blocks = pl.units * pl.chunks_per_unit;
  hipLaunchKernelGGL((mass_kernel<D, T, kChunkWaves, 2, false, false>), dim3((unsigned)blocks),
                     dim3(C::kThreads), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t n = pl.units * sh.S;
  hipLaunchKernelGGL((mass_chunk_sum_kernel<kChunkTile>), dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, stream, a, (int)pl.units);
  return hipGetLastError();
}

}  // namespace

size_t mass_workspace_bytes(int dtype, const Shape& sh, int window, int per_head) {
  const ChunkPlan pl = mass_chunk_plan(dtype, sh, window, per_head);
  if (pl.chunk_qbs == 0) return 0;
  return (size_t)pl.units * pl.chunks_per_unit * kChunkTile * sizeof(float);
}

hipError_t launch_mass_ws(const void* q, const void* k, const float* lse, int dtype,
                          const Shape& sh, float scale, int window, int per_head, float* mass,
                          void* workspace, hipStream_t stream) {
  const ChunkPlan pl = mass_chunk_plan(dtype, sh, window, per_head);
  if (pl.chunk_qbs == 0 || workspace == nullptr)
    return launch_mass(q, k, lse, dtype, sh, scale, window, per_head, mass, stream);
  return sh.D == 128 ? launch_mass_chunked_t<128, uint16_t>(q, k, lse, sh, scale, window, per_head,
                                                            mass, pl, workspace, stream)
                     : launch_mass_chunked_t<64, uint16_t>(q, k, lse, sh, scale, window, per_head,
                                                           mass, pl, workspace, stream);
}

hipError_t launch_mass(const void* q, const void* k, const float* lse, int dtype, const Shape& sh,
                       float scale, int window, int per_head, float* mass, hipStream_t stream) {
  const SegOut none{0, 32, 0, nullptr, nullptr};
  if (dtype != 0)
    return launch_mass_f32(q, k, lse, sh, scale, window, per_head, mass, none, stream);
  return sh.D == 128 ? launch_mass_t<128, uint16_t, false>(q, k, lse, sh, scale, window, per_head,
                                                           mass, none, stream)
                     : launch_mass_t<64, uint16_t, false>(q, k, lse, sh, scale, window, per_head,
                                                          mass, none, stream);
}

hipError_t launch_block_scores(const void* q, const void* k, const float* lse, int dtype,
                               const Shape& sh, float scale, int window, int per_head,
                               const SegOut& seg, hipStream_t stream) {
  if (seg.n == 0) return hipSuccess;
  if (dtype != 0)
    return launch_mass_f32(q, k, lse, sh, scale, window, per_head, nullptr, seg, stream);
  return sh.D == 128 ? launch_mass_t<128, uint16_t, true>(q, k, lse, sh, scale, window, per_head,
                                                          nullptr, seg, stream)
                     : launch_mass_t<64, uint16_t, true>(q, k, lse, sh, scale, window, per_head,
                                                         nullptr, seg, stream);
}

}  // namespace kvp
