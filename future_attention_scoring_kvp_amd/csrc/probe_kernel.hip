// Matrix-core throughput probe for gfx950: the sustained bf16 MFMA rate of
// the whole chip and the core clock it runs at, the yardstick beside the
// datasheet peak for the transposed mass pass (an MFMA-bound contraction).
//
// Every wave issues back-to-back v_mfma_f32_32x32x16_bf16 on four independent
// accumulator chains (no memory traffic, no VALU work in the loop), with
// operands of pseudo-random bf16 values in [-2, 2) so that the datapath
// toggles like it does on real data.  Two waves per SIMD (512-thread
// workgroups, one per CU), as in the mass kernel.  Lane 0 of each workgroup
// records the core-clock and constant-rate counters at its start and end.
#include "kvp_probe.h"

#include "kvp_device.h"

namespace kvp {
namespace {

constexpr int kProbeThreads = 512;

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// Two bf16 values in [-2, 2) from 32 random bits: sign, exponent 126 or 127,
// random 7-bit mantissa.
__device__ __forceinline__ uint32_t bf16_pair(uint32_t r) {
  const uint32_t lo = ((r & 1u) << 15) | ((126u + ((r >> 1) & 1u)) << 7) | ((r >> 2) & 0x7Fu);
  const uint32_t hi = (((r >> 9) & 1u) << 15) | ((126u + ((r >> 10) & 1u)) << 7) | ((r >> 11) & 0x7Fu);
  return lo | (hi << 16);
}

__global__ __launch_bounds__(kProbeThreads, 1) void mfma_probe_kernel(int iters, float* sink,
                                                                      long long* stamps) {
  const uint32_t seed = mix(blockIdx.x * kProbeThreads + threadIdx.x + 1u);
  u32x4_t a, b;
  for (int i = 0; i < 4; ++i) {
    a[i] = bf16_pair(mix(seed + 2 * i));
    b[i] = bf16_pair(mix(seed + 2 * i + 1));
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  long long t0 = 0, w0 = 0;
  if (threadIdx.x == 0) {
    t0 = clock64();
    w0 = wall_clock64();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      c0 = mfma_32x32x16(a, b, c0);
      c1 = mfma_32x32x16(b, a, c1);
      c2 = mfma_32x32x16(a, a, c2);
      c3 = mfma_32x32x16(b, b, c3);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  sink[blockIdx.x * kProbeThreads + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    const long long t1 = clock64(), w1 = wall_clock64();
    long long* st = stamps + 4 * (size_t)blockIdx.x;
    st[0] = t0;
    st[1] = t1;
    st[2] = w0;
    st[3] = w1;
  }
}

// Read probe: every thread reads 16-byte pieces through a buffer resource,
// as the matrix-core kernels stage their operands (raw buffer loads of 16
// bytes, consecutive lanes on consecutive pieces), and writes one word, so
// the bytes the memory counters see can be compared with a known read.
__global__ __launch_bounds__(256) void read16_probe_kernel(const unsigned char* src,
                                                           uint32_t bytes, uint32_t* sink) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(src, bytes);
  const uint32_t n16 = bytes / 16;
  uint32_t x = 0;
  for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < n16; i += gridDim.x * 256) {
    const u32x4_t v =
        __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, i * 16u, 0, 0));
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[blockIdx.x * 256 + threadIdx.x] = x;
}

}  // namespace
}  // namespace kvp

extern "C" {

int kvp_probe_read16(const void* src, uint32_t bytes, int blocks, uint32_t* sink,
                     hipStream_t stream) {
  if (!src || !sink || blocks < 1 || bytes % 16 != 0) return 1;
  hipLaunchKernelGGL(kvp::read16_probe_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const unsigned char*>(src), bytes, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}


int kvp_probe_mfma_bf16(int blocks, int iters, float* sink, long long* stamps,
                        hipStream_t stream) {
  if (blocks < 1 || iters < 1 || !sink || !stamps) return 1;
  hipLaunchKernelGGL(kvp::mfma_probe_kernel, dim3(blocks), dim3(kvp::kProbeThreads), 0, stream,
                     iters, sink, stamps);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

double kvp_probe_flops(int blocks, int iters) {
  // per wave and iteration: 16 MFMAs of 32 x 32 x 16 (2 flop per product)
  return (double)blocks * (kvp::kProbeThreads / 64) * iters * 16.0 * 32 * 32 * 16 * 2;
}

int kvp_probe_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

}  // extern "C"
