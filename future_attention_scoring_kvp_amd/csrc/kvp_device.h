// Device-side building blocks shared by the gfx950 kernels of libkvp.
//
// Matrix-core tile (both dense kernels put KEYS on the rows = A operand and
// QUERIES on the columns = B operand):
//   v_mfma_f32_32x32x16_bf16, D = A (32 x 16) * B (16 x 32):
//     lane l supplies A[l % 32][8*(l/32) + e] and B[8*(l/32) + e][l % 32],
//     e = 0..7, and receives D[8*(v/4) + 4*(l/32) + (v%4)][l % 32] in result
//     register v = 0..15.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kNumCUs = 256;     // MI355X: 8 XCDs x 32 compute units
constexpr int kBlk = 32;          // MFMA tile edge (rows = keys, cols = queries)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Row index (within a 32-row tile) of result register v of lane l.
__device__ __forceinline__ int mfma_row(int v, int lane) {
  return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Buffer resource (raw, stride 0) over `bytes` bytes from `base`.  Loads whose
// per-lane offset is at or beyond `bytes` return zeros instead of touching
// memory (the check covers the per-lane offset only, so every offset here is
// passed per lane with a zero scalar offset).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// One fp32 store through a buffer resource; offsets at or past the range of
// the resource are dropped by the hardware bounds check.
__device__ __forceinline__ void buf_store_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_offset,
                                              float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, byte_offset, 0, 0);
}

// Eight bf16 elements at element offset `elem` of a buffer (16 bytes).
// Out-of-range reads give zeros.
__device__ __forceinline__ u32x4_t buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t elem,
                                             const uint16_t*) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, elem * 2, 0, 0));
}

// Eight consecutive bf16 input elements (16 bytes).
__device__ __forceinline__ u32x4_t load8(const uint16_t* __restrict__ p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Blocks are dispatched round-robin over the 8 XCDs (each with its own L2).
// Map block `bid` to (unit, tile) so that every tile of a unit runs on one
// XCD (units u with u % 8 == bid % 8) and each XCD receives tiles in order
// 0, 1, 2, ... (tile 0 = the longest).  Falls back to tile-major order when
// the unit count is not a multiple of 8.
__device__ __forceinline__ void xcd_map(int bid, int n_units, int& unit, int& tile) {
  if ((n_units & 7) == 0) {
    const int xcd = bid & 7;
    const int slot = bid >> 3;
    const int per_xcd = n_units >> 3;
    tile = slot / per_xcd;
    unit = (slot - tile * per_xcd) * 8 + xcd;
  } else {
    tile = bid / n_units;
    unit = bid - tile * n_units;
  }
}

// Unit-major variant for grids whose blocks all carry the same work: block
// `bid` of an XCD takes tile `bid / 8 % n_per_unit` of the XCD's
// `bid / 8 / n_per_unit`-th unit, so each round of an XCD's CUs covers whole
// units and every tile of a unit sweeps the unit's rows together (one L2).
// Falls back to unit-major order over the grid when the unit count is not a
// multiple of 8.
__device__ __forceinline__ void xcd_map_units(int bid, int n_units, int n_per_unit, int& unit,
                                              int& tile) {
  if ((n_units & 7) == 0) {
    const int slot = bid >> 3;
    const int u_local = slot / n_per_unit;
    tile = slot - u_local * n_per_unit;
    unit = u_local * 8 + (bid & 7);
  } else {
    unit = bid / n_per_unit;
    tile = bid - unit * n_per_unit;
  }
}

}  // namespace kvp
