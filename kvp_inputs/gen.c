/* Seeded synthetic inputs for the future-attention-mass path.
 *
 * This module only makes input data (Q and K tensors and the small recipe
 * arrays that shape them).  It holds none of the method's arithmetic: no
 * logits, no softmax, no mass, no selection.  Both the CPU oracle and the GPU
 * path consume the bytes it writes.
 *
 * Random numbers come from a counter-based SplitMix64 (Vigna's published
 * SplitMix64 finaliser applied to key + (n+1)*golden_gamma), so element n of a
 * stream can be produced independently of every other element, by any thread.
 * Normal deviates use the Box-Muller transform on pairs (2p, 2p+1).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* n-th output of a SplitMix64 generator whose state starts at `key`. */
static inline uint64_t sm64_at(uint64_t key, uint64_t n) {
  return mix64(key + (n + 1) * GAMMA);
}

uint64_t kvpgen_stream_key(uint64_t seed, uint64_t tag) {
  return mix64(seed ^ mix64(tag * 0xD1B54A32D192ED03ULL + GAMMA));
}

uint64_t kvpgen_u64(uint64_t key, uint64_t n) { return sm64_at(key, n); }

/* Standard normal number n of stream `key` (Box-Muller on the pair n/2). */
static inline double normal_at(uint64_t key, uint64_t n) {
  const uint64_t p = n >> 1;
  const uint64_t a = sm64_at(key, 2 * p);
  const uint64_t b = sm64_at(key, 2 * p + 1);
  const double u1 = (double)((a >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
  const double u2 = (double)(b >> 11) * 0x1.0p-53;       /* [0, 1) */
  const double r = sqrt(-2.0 * log(u1));
  const double th = 6.283185307179586476925286766559 * u2;
  return (n & 1) ? r * sin(th) : r * cos(th);
}

double kvpgen_normal(uint64_t key, uint64_t n) { return normal_at(key, n); }

void kvpgen_normals_f64(uint64_t key, uint64_t offset, int64_t count, double* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = normal_at(key, offset + (uint64_t)i);
}

/* float -> bfloat16 bit pattern, round to nearest even.  Input values here
 * are finite by construction. */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* `count` distinct positions drawn uniformly from [lo, hi), seeded by key,
 * via a partial Fisher-Yates shuffle; written in draw order. */
int kvpgen_choose(uint64_t key, int64_t lo, int64_t hi, int64_t count, int64_t* out) {
  const int64_t n = hi - lo;
  if (n < 0 || count < 0 || count > n) return 1;
  int64_t* pool = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  if (!pool) return 2;
  for (int64_t i = 0; i < n; ++i) pool[i] = lo + i;
  for (int64_t i = 0; i < count; ++i) {
    const uint64_t r = sm64_at(key, (uint64_t)i);
    /* multiply-shift maps r to [0, n - i) */
    const int64_t span = n - i;
    const int64_t pick = i + (int64_t)(((unsigned __int128)r * (uint64_t)span) >> 64);
    const int64_t t = pool[i];
    pool[i] = pool[pick];
    pool[pick] = t;
    out[i] = pool[i];
  }
  free(pool);
  return 0;
}

/* One [B, H, S, D] tensor:
 *   x[b,h,t,c] = (z[b,h,t,c] + lr_scale * sum_r U[h / u_head_div, c, r] * a[b, t, r]) * pos_scale[t]
 * with z the standard normal stream `key` at flat index ((b*H + h)*S + t)*D + c.
 * U ([n_u_heads, D, R]) and a ([B, S, R]) are optional (R = 0 disables);
 * pos_scale ([S]) is optional (NULL = 1).  out_bf16 != 0 writes bfloat16 bit
 * patterns (round to nearest even) into uint16 out, else float32. */
typedef struct {
  uint64_t key;
  int64_t B, H, S, D;
  const float* pos_scale;
  const double* U;
  const double* a;
  int R;
  double lr_scale;
  int64_t u_head_div;
  int out_bf16;
  void* out;
  int64_t row_begin, row_end; /* rows = (b, h, t) flattened */
} gen_job;

static void* gen_worker(void* arg) {
  const gen_job* j = (const gen_job*)arg;
  const int64_t D = j->D;
  for (int64_t row = j->row_begin; row < j->row_end; ++row) {
    const int64_t t = row % j->S;
    const int64_t bh = row / j->S;
    const int64_t h = bh % j->H;
    const int64_t b = bh / j->H;
    const double ps = j->pos_scale ? (double)j->pos_scale[t] : 1.0;
    const double* arow = j->R ? j->a + ((size_t)b * j->S + t) * j->R : NULL;
    const double* Uh = j->R ? j->U + (size_t)(h / j->u_head_div) * D * j->R : NULL;
    for (int64_t c = 0; c < D; ++c) {
      double v = normal_at(j->key, (uint64_t)(row * D + c));
      if (j->R) {
        double lr = 0.0;
        for (int r = 0; r < j->R; ++r) lr += Uh[c * j->R + r] * arow[r];
        v += j->lr_scale * lr;
      }
      v *= ps;
      const float f = (float)v;
      if (j->out_bf16)
        ((uint16_t*)j->out)[row * D + c] = f32_to_bf16_rne(f);
      else
        ((float*)j->out)[row * D + c] = f;
    }
  }
  return NULL;
}

int kvpgen_tensor(uint64_t key, int64_t B, int64_t H, int64_t S, int64_t D,
                  const float* pos_scale, const double* U, const double* a, int R,
                  double lr_scale, int64_t u_head_div, int out_bf16, void* out,
                  int nthreads) {
  if (B < 0 || H < 0 || S < 0 || D < 0 || !out || u_head_div < 1 || R < 0) return 1;
  if (R > 0 && (!U || !a)) return 1;
  const int64_t rows = B * H * S;
  if (rows == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > rows) nthreads = (int)rows;
  pthread_t tid[256];
  gen_job jobs[256];
  for (int i = 0; i < nthreads; ++i) {
    gen_job j = {key, B, H, S, D, pos_scale, U, a, R, lr_scale, u_head_div, out_bf16, out,
                 rows * i / nthreads, rows * (i + 1) / nthreads};
    jobs[i] = j;
  }
  int started = 0;
  for (int i = 1; i < nthreads; ++i) {
    if (pthread_create(&tid[i], NULL, gen_worker, &jobs[i]) != 0) break;
    started = i;
  }
  gen_worker(&jobs[0]);
  for (int i = 1; i <= started; ++i) pthread_join(tid[i], NULL);
  for (int i = started + 1; i < nthreads; ++i) gen_worker(&jobs[i]);
  return 0;
}
