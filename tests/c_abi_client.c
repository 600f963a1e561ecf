/*
 * c_abi_client — libkvp.so used from C through include/kvp.h alone: no
 * Python, no torch.  Test infrastructure: tests/test_c_abi_client.py builds
 * nothing and runs the binary that the build step compiles next to this file.
 *
 *   c_abi_client host
 *       Host-side checks only (no GPU call): ABI version, keep count,
 *       workspace sizes, status strings, and arguments that every stage
 *       rejects before launching anything.  Exit status 0 when all hold.
 *
 *   c_abi_client run B Hq Hkv S D window n_sink top_k q.bin k.bin out_dir
 *       Reads Q [B,Hq,S,D] and K [B,Hkv,S,D] as bf16 bit patterns, runs the
 *       path on a stream of its own with device memory from hipMalloc —
 *       kvp_lse_fwd, kvp_future_mass, kvp_future_mass_chunked (with its
 *       workspace when it takes one), kvp_select_topk (with its workspace) —
 *       and writes lse.bin, mass.bin, mass_chunked.bin and keep.bin (raw fp32
 *       / int32) to out_dir.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvp.h"

static int failures = 0;

#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");              \
      ++failures;                         \
    }                                     \
  } while (0)

#define HIP_OK(call)                                                             \
  do {                                                                           \
    hipError_t e_ = (call);                                                      \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));          \
      exit(2);                                                                   \
    }                                                                            \
  } while (0)

static kvp_dims_t dims_of(int b, int hq, int hkv, int s, int d) {
  kvp_dims_t x;
  x.batch = b;
  x.n_q_heads = hq;
  x.n_kv_heads = hkv;
  x.seq_len = s;
  x.head_dim = d;
  return x;
}

static int host_checks(void) {
  CHECK(kvp_abi_version() == 8, "abi version %d", (int)kvp_abi_version());
  /* budget s + w + k clipped to the sequence */
  CHECK(kvp_keep_count(1000, 100, 4, 50) == 154, "keep count");
  CHECK(kvp_keep_count(10, 100, 4, 50) == 10, "keep count, short row");
  CHECK(kvp_keep_count(-1, 0, 0, 0) == -1, "keep count, negative size");
  CHECK(kvp_select_workspace_bytes(dims_of(8, 1, 1, 32768, 128), 100) == 0,
        "select workspace, register path");
  CHECK(kvp_select_workspace_bytes(dims_of(8, 1, 1, 131072, 128), 2048) > 0,
        "select workspace, split path");
  for (int st = KVP_OK; st <= KVP_EHIP; ++st)
    CHECK(kvp_status_string((kvp_status_t)st) != NULL && kvp_status_string((kvp_status_t)st)[0],
          "status string %d", st);
  /* rejected before any launch: no device memory or stream is touched */
  _Alignas(256) float dummy[64];
  const kvp_dims_t ok = dims_of(1, 4, 2, 256, 128);
  CHECK(kvp_lse_fwd(NULL, dummy, KVP_BF16, ok, 0.f, dummy, NULL) == KVP_EINVAL, "lse: null q");
  CHECK(kvp_lse_fwd(dummy, dummy, KVP_BF16, dims_of(1, 4, 2, 256, 96), 0.f, dummy, NULL) ==
            KVP_EUNSUPPORTED,
        "lse: head_dim 96");
  CHECK(kvp_lse_fwd(dummy, dummy, KVP_BF16, dims_of(1, 5, 2, 256, 128), 0.f, dummy, NULL) ==
            KVP_EINVAL,
        "lse: Hq not a multiple of Hkv");
  CHECK(kvp_future_mass(dummy, dummy, dummy, KVP_BF16, ok, 0.f, -1, dummy, NULL) == KVP_EINVAL,
        "mass: negative window");
  CHECK(kvp_future_mass_chunked(dummy, dummy, dummy, KVP_BF16, ok, 0.f, 8, 2, dummy, NULL, 0,
                                NULL) == KVP_EINVAL,
        "chunked mass: per_head 2");
  CHECK(kvp_select_topk(dummy, dims_of(1, 1, 1, 256, 128), -3, 4, 10, (int32_t*)dummy, NULL, 0,
                        NULL) == KVP_EINVAL,
        "select: negative window");
  CHECK(kvp_select_topk(dummy, dims_of(1, 1, 1, 131072, 128), 1024, 4, 2048, (int32_t*)dummy,
                        NULL, 0, NULL) == KVP_EWORKSPACE,
        "select: long rows without a workspace");
  return failures;
}

static void* read_file(const char* path, size_t bytes) {
  FILE* f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    exit(2);
  }
  void* p = malloc(bytes ? bytes : 1);
  if (fread(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "short read %s\n", path);
    exit(2);
  }
  fclose(f);
  return p;
}

static void write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    exit(2);
  }
  fclose(f);
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  HIP_OK(hipMalloc(&p, bytes ? bytes : 256));
  return p;
}

static int run(int argc, char** argv) {
  if (argc != 13) {
    fprintf(stderr, "usage: %s run B Hq Hkv S D window n_sink top_k q.bin k.bin out_dir\n",
            argv[0]);
    return 2;
  }
  const int B = atoi(argv[2]), Hq = atoi(argv[3]), Hkv = atoi(argv[4]), S = atoi(argv[5]);
  const int D = atoi(argv[6]), w = atoi(argv[7]), s = atoi(argv[8]), k = atoi(argv[9]);
  const kvp_dims_t dims = dims_of(B, Hq, Hkv, S, D);
  const size_t q_bytes = (size_t)B * Hq * S * D * 2, k_bytes = (size_t)B * Hkv * S * D * 2;
  const size_t lse_bytes = (size_t)B * Hq * S * 4, mass_bytes = (size_t)B * Hkv * S * 4;
  const int64_t n_keep = kvp_keep_count(S, w, s, k);
  const size_t keep_bytes = (size_t)B * Hkv * (size_t)n_keep * 4;
  void* hq = read_file(argv[10], q_bytes);
  void* hk = read_file(argv[11], k_bytes);

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  void* dq = dev_alloc(q_bytes);
  void* dk = dev_alloc(k_bytes);
  float* dlse = (float*)dev_alloc(lse_bytes);
  float* dmass = (float*)dev_alloc(mass_bytes);
  float* dmass2 = (float*)dev_alloc(mass_bytes);
  int32_t* dkeep = (int32_t*)dev_alloc(keep_bytes);
  const size_t mws = kvp_future_mass_workspace_bytes(dims, KVP_BF16, w, 0);
  kvp_dims_t rows = dims_of(B * Hkv, 1, 1, S, D);
  const size_t sws = kvp_select_workspace_bytes(rows, k);
  void* dmws = mws ? dev_alloc(mws) : NULL;  /* hipMalloc: 256-byte aligned */
  void* dsws = sws ? dev_alloc(sws) : NULL;
  HIP_OK(hipMemcpyAsync(dq, hq, q_bytes, hipMemcpyHostToDevice, st));
  HIP_OK(hipMemcpyAsync(dk, hk, k_bytes, hipMemcpyHostToDevice, st));

  kvp_status_t r = kvp_lse_fwd(dq, dk, KVP_BF16, dims, 0.f, dlse, st);
  CHECK(r == KVP_OK, "kvp_lse_fwd: %s", kvp_status_string(r));
  r = kvp_future_mass(dq, dk, dlse, KVP_BF16, dims, 0.f, w, dmass, st);
  CHECK(r == KVP_OK, "kvp_future_mass: %s", kvp_status_string(r));
  r = kvp_future_mass_chunked(dq, dk, dlse, KVP_BF16, dims, 0.f, w, 0, dmass2, dmws, mws, st);
  CHECK(r == KVP_OK, "kvp_future_mass_chunked: %s", kvp_status_string(r));
  r = kvp_select_topk(dmass, rows, w, s, k, dkeep, dsws, sws, st);
  CHECK(r == KVP_OK, "kvp_select_topk: %s", kvp_status_string(r));
  HIP_OK(hipStreamSynchronize(st));

  void* out = malloc(lse_bytes > keep_bytes ? (lse_bytes > mass_bytes ? lse_bytes : mass_bytes)
                                            : (keep_bytes > mass_bytes ? keep_bytes : mass_bytes));
  HIP_OK(hipMemcpy(out, dlse, lse_bytes, hipMemcpyDeviceToHost));
  write_file(argv[12], "lse.bin", out, lse_bytes);
  HIP_OK(hipMemcpy(out, dmass, mass_bytes, hipMemcpyDeviceToHost));
  write_file(argv[12], "mass.bin", out, mass_bytes);
  HIP_OK(hipMemcpy(out, dmass2, mass_bytes, hipMemcpyDeviceToHost));
  write_file(argv[12], "mass_chunked.bin", out, mass_bytes);
  HIP_OK(hipMemcpy(out, dkeep, keep_bytes, hipMemcpyDeviceToHost));
  write_file(argv[12], "keep.bin", out, keep_bytes);

  free(out);
  free(hq);
  free(hk);
  hipFree(dq);
  hipFree(dk);
  hipFree(dlse);
  hipFree(dmass);
  hipFree(dmass2);
  hipFree(dkeep);
  if (dmws) hipFree(dmws);
  if (dsws) hipFree(dsws);
  HIP_OK(hipStreamDestroy(st));
  printf("c_abi_client: ran %d x %d/%d heads x %d, workspaces %zu and %zu bytes\n", B, Hq, Hkv, S,
         mws, sws);
  return failures;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "host") == 0) {
    const int f = host_checks();
    printf("c_abi_client: host checks %s\n", f ? "FAILED" : "ok");
    return f ? 1 : 0;
  }
  if (argc >= 2 && strcmp(argv[1], "run") == 0) return run(argc, argv) ? 1 : 0;
  fprintf(stderr, "usage: %s host | run ...\n", argv[0]);
  return 2;
}
