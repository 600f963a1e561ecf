/*
 * kvp_probe.h — measurement probe shipped beside libkvp (libkvp_probe.so):
 * the sustained bf16 matrix-core rate of the GPU it runs on and the core
 * clock during that load.  Used to state the mass pass's throughput against
 * a measured peak as well as against the datasheet one; it computes nothing
 * of the method.
 */
#ifndef KVP_PROBE_H_
#define KVP_PROBE_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue the probe on `stream`: `blocks` workgroups of 8 waves (one per
 * CU), each wave issuing 16 * iters back-to-back v_mfma_f32_32x32x16_bf16 on
 * register operands (no memory traffic in the loop).
 *   sink   : device fp32 [blocks * 512], written (keeps the results live).
 *   stamps : device int64 [blocks * 4], per workgroup: core-clock counter at
 *            start and end, constant-rate counter at start and end.
 * Returns 0, 1 for invalid arguments, 4 if the launch failed.  Time it with
 * events on `stream`; flops come from kvp_probe_flops. */
int kvp_probe_mfma_bf16(int blocks, int iters, float* sink, long long* stamps,
                        hipStream_t stream);

/* Flops of one probe launch (2 per multiply-add). */
double kvp_probe_flops(int blocks, int iters);

/* Read probe for memory-counter scaling: `blocks` workgroups of 256 threads
 * read the `bytes` bytes at `src` (device, a multiple of 16, below 4 GiB)
 * through 16-byte raw buffer loads, consecutive lanes on consecutive 16-byte
 * pieces, and write one uint32 per thread to `sink` (device, blocks * 256).
 * Returns 0, 1 for invalid arguments, 4 if the launch failed. */
int kvp_probe_read16(const void* src, uint32_t bytes, int blocks, uint32_t* sink,
                     hipStream_t stream);

/* Rate of the constant-rate counter in kHz (0 on error): core clock =
 * d(core counter) / d(constant counter) * rate. */
int kvp_probe_wall_clock_khz(void);

#ifdef __cplusplus
}
#endif

#endif /* KVP_PROBE_H_ */
