// Transposed future-attention-mass pass for gfx950.
//
// Computes, for every key j of every (batch, KV head),
//   mass[j] = sum over the G query heads g of the group,
//             sum over queries i >= j + window of exp2(c * <q_i, k_j> - lse2_i)
// with c = scale * log2(e) and lse2 = LSE * log2(e): the un-normalised future
// mass of KVpop (§3.1 Eq. 2, App. B.1) recovered from the per-query LSE as in
// its §3.2 Eq. 8, without any S x S map.
//
// Work decomposition (keys stationary, queries streamed):
//   * one workgroup = 4 waves = 256 consecutive keys of one (batch, KV head);
//     each wave keeps its 64 keys (two 32-row MFMA blocks) as bf16 A-operands
//     in registers for the whole sweep;
//   * the workgroup sweeps the future query blocks (32 queries each) of all G
//     heads of the group, from the end of the sequence backwards, staging
//     4 (query block, head) pairs per LDS stage, double buffered;
//   * per pair and wave: 16 MFMA 32x32x16 give a 64 x 32 logit tile; each
//     lane applies fma + exp2 + add to its 32 values and keeps 32 per-key
//     partial sums (its query column) in registers;
//   * at the end the 32 column partials of each key are added in LDS in a
//     fixed order and each key's mass is written once: no atomics, bitwise
//     reproducible.
// Blocks are mapped XCD-aware: all tiles of one (batch, KV head) run on the
// same XCD and sweep the same Q rows in the same order (shared L2), longest
// tiles first so the triangular work load balances.
#include "kvp_device.h"
#include "kvp_launch.h"

namespace kvp {
namespace {

template <int D>
struct MassCfg {
  static constexpr int kWaves = 4;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kKeysPerWave = 64;
  static constexpr int kKeysPerWG = kWaves * kKeysPerWave;
  static constexpr int kSlots = 4;  // (query block, head) pairs per LDS stage
  static constexpr int kKSteps = D / 16;
  static constexpr int kChunks = D / 8;               // 16-byte chunks per row
  static constexpr int kRowStride = D * 2 + 16;       // padded row pitch (bytes)
  static constexpr int kSlotBytes = kBlk * kRowStride;
  static constexpr int kStageBytes = kSlots * kSlotBytes;
  static constexpr int kStageChunks = kSlots * kBlk * kChunks;
  static constexpr int kChunksPerThread = kStageChunks / kThreads;
  static_assert(kStageChunks % kThreads == 0, "stage must split evenly");
};

struct MassArgs {
  const void* q;
  const void* k;
  const float* lse;
  float* mass;
  int B, Hq, Hkv, S, G, window;
  float c;  // scale * log2(e)
};

template <int D, typename T>
__global__ __launch_bounds__(256, 2) void mass_kernel(MassArgs a) {
  using C = MassCfg<D>;
  __shared__ __attribute__((aligned(16))) unsigned char q_lds[2][C::kStageBytes];
  __shared__ float l_lds[2][C::kSlots * kBlk];

  const int S = a.S, G = a.G, w = a.window;
  int unit, tile;
  xcd_map(blockIdx.x, a.B * a.Hkv, unit, tile);
  const int b = unit / a.Hkv;
  const int h = unit - b * a.Hkv;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int tile_key0 = tile * C::kKeysPerWG;
  const int key0 = tile_key0 + wave * C::kKeysPerWave;

  const T* __restrict__ kbase = static_cast<const T*>(a.k) + (size_t)(b * a.Hkv + h) * S * D;
  const T* __restrict__ qbase = static_cast<const T*>(a.q) + (size_t)(b * a.Hq + h * G) * S * D;
  const float* __restrict__ lbase = a.lse + (size_t)(b * a.Hq + h * G) * S;

  // Stationary keys: A-operands of the two 32-row blocks, all k-steps.
  u32x4_t kf[2][C::kKSteps];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int key = key0 + 32 * rb + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < C::kKSteps; ++ks) {
      const int col = 16 * ks + 8 * (lane >> 5);
      kf[rb][ks] = key < S ? load8(kbase + (size_t)key * D + col) : u32x4_t{0, 0, 0, 0};
    }
  }

  f32x16_t acc0 = {}, acc1 = {};
  const float c = a.c;
  const int q_first = tile_key0 + w;  // first query any key of the tile can see

  if (q_first < S) {
    const int qb_hi = (S - 1) / kBlk;
    const int qb_lo = q_first / kBlk;
    const int n_pairs = (qb_hi - qb_lo + 1) * G;
    const int n_stages = (n_pairs + C::kSlots - 1) / C::kSlots;

    // Stage loader: pair p -> query block qb_hi - p / G, head p % G.
    u32x4_t stage_regs[C::kChunksPerThread];
    auto load_stage = [&](int st) {
#pragma unroll
      for (int t = 0; t < C::kChunksPerThread; ++t) {
        const int cidx = tid + t * C::kThreads;
        const int slot = cidx / (kBlk * C::kChunks);
        const int row = (cidx / C::kChunks) % kBlk;
        const int ch = cidx % C::kChunks;
        const int p = st * C::kSlots + slot;
        u32x4_t v = {0, 0, 0, 0};
        if (p < n_pairs) {
          const int qb = qb_hi - p / G;
          const int g = p - (p / G) * G;
          const int i = qb * kBlk + row;
          if (i < S) v = load8(qbase + ((size_t)g * S + i) * D + ch * 8);
        }
        stage_regs[t] = v;
      }
    };
    auto store_stage = [&](int st, int buf) {
#pragma unroll
      for (int t = 0; t < C::kChunksPerThread; ++t) {
        const int cidx = tid + t * C::kThreads;
        const int slot = cidx / (kBlk * C::kChunks);
        const int row = (cidx / C::kChunks) % kBlk;
        const int ch = cidx % C::kChunks;
        *reinterpret_cast<u32x4_t*>(&q_lds[buf][slot * C::kSlotBytes + row * C::kRowStride + ch * 16]) =
            stage_regs[t];
      }
      if (tid < C::kSlots * kBlk) {
        const int slot = tid / kBlk;
        const int row = tid % kBlk;
        const int p = st * C::kSlots + slot;
        float l2 = __builtin_inff();  // no query: exp2(x - inf) = 0
        if (p < n_pairs) {
          const int qb = qb_hi - p / G;
          const int g = p - (p / G) * G;
          const int i = qb * kBlk + row;
          if (i < S) l2 = lbase[(size_t)g * S + i] * kLog2e;
        }
        l_lds[buf][tid] = l2;
      }
    };

    load_stage(0);
    store_stage(0, 0);
    __syncthreads();

    for (int st = 0; st < n_stages; ++st) {
      const int buf = st & 1;
      if (st + 1 < n_stages) load_stage(st + 1);

#pragma unroll
      for (int slot = 0; slot < C::kSlots; ++slot) {
        const int p = st * C::kSlots + slot;
        if (p >= n_pairs) break;
        const int q0 = (qb_hi - p / G) * kBlk;
        if (q0 + kBlk - 1 < key0 + w) continue;           // no query of this block reaches these keys
        const bool full = q0 >= key0 + C::kKeysPerWave - 1 + w;

        const unsigned char* sbase = &q_lds[buf][slot * C::kSlotBytes + (lane & 31) * C::kRowStride];
        f32x16_t s0 = {}, s1 = {};
#pragma unroll
        for (int ks = 0; ks < C::kKSteps; ++ks) {
          const u32x4_t bq = *reinterpret_cast<const u32x4_t*>(sbase + (2 * ks + (lane >> 5)) * 16);
          s0 = mfma_32x32x16(kf[0][ks], bq, s0);
          s1 = mfma_32x32x16(kf[1][ks], bq, s1);
        }
        const float l2 = l_lds[buf][slot * kBlk + (lane & 31)];
        if (full) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            acc0[v] += fast_exp2(__builtin_fmaf(s0[v], c, -l2));
            acc1[v] += fast_exp2(__builtin_fmaf(s1[v], c, -l2));
          }
        } else {
          const int i = q0 + (lane & 31);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int j = key0 + mfma_row(v, lane);
            const float x0 = __builtin_fmaf(s0[v], c, -l2);
            const float x1 = __builtin_fmaf(s1[v], c, -l2);
            acc0[v] += fast_exp2(i >= j + w ? x0 : -__builtin_inff());
            acc1[v] += fast_exp2(i >= j + 32 + w ? x1 : -__builtin_inff());
          }
        }
      }

      if (st + 1 < n_stages) store_stage(st + 1, buf ^ 1);
      __syncthreads();
    }
  }

  // Column reduction: each lane holds one query column's partial sums for 32
  // keys; add the 32 columns of every key in LDS in a fixed order.
  __syncthreads();
  float* red = reinterpret_cast<float*>(&q_lds[0][0]) + wave * (C::kKeysPerWave * 33);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int kl = mfma_row(v, lane);
    red[kl * 33 + (lane & 31)] = acc0[v];
    red[(kl + 32) * 33 + (lane & 31)] = acc1[v];
  }
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int cidx = 0; cidx < 32; ++cidx) tot += red[lane * 33 + cidx];
  const int key = key0 + lane;
  if (key < S) a.mass[(size_t)(b * a.Hkv + h) * S + key] = tot;
}

template <int D, typename T>
hipError_t launch_mass_t(const void* q, const void* k, const float* lse, const Shape& sh,
                         float scale, int window, float* mass, hipStream_t stream) {
  using C = MassCfg<D>;
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
  a.c = scale * kLog2e;
  const int64_t n_tiles = (sh.S + C::kKeysPerWG - 1) / C::kKeysPerWG;
  const int64_t blocks = n_tiles * (int64_t)sh.B * sh.Hkv;
  hipLaunchKernelGGL((mass_kernel<D, T>), dim3((unsigned)blocks), dim3(C::kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mass(const void* q, const void* k, const float* lse, int dtype, const Shape& sh,
                       float scale, int window, float* mass, hipStream_t stream) {
  if (sh.D == 128)
    return dtype == 0 ? launch_mass_t<128, uint16_t>(q, k, lse, sh, scale, window, mass, stream)
                      : launch_mass_t<128, float>(q, k, lse, sh, scale, window, mass, stream);
  return dtype == 0 ? launch_mass_t<64, uint16_t>(q, k, lse, sh, scale, window, mass, stream)
                    : launch_mass_t<64, float>(q, k, lse, sh, scale, window, mass, stream);
}

}  // namespace kvp
