// KVpop target scores from future-attention masses, for gfx950.
//
//   r[b, h, t] = Agg over the query heads g of KV head h of log(eps + m_g[t] / N_t)
// with N_t = max(1, S - (t + w)) when normalising (KVpop §3.1 Eq. 2 and
// App. B.2) and N_t = 1 otherwise (App. B.1), where Agg is
//   LOG_MEAN  log(eps + mean_g m_g[t] / N_t)     (App. B.1, log of the group mean)
//   MEAN_LOG  mean_g log(eps + m_g[t] / N_t)     (§3.1 Eq. 3 with Agg = mean)
//   MAX_LOG   max_g  log(eps + m_g[t] / N_t)     (§3.1 Eq. 3 with Agg = max)
// and, when a query position q >= 0 is given, the decayed score of App. B.3
//   r(q)[t] = r[t] + floor((q - t) / n) * log(gamma_h)   for t <= q,
// and -inf for tokens t > q, which do not exist yet at query q.
//
// One thread per output score; the G masses of a group are read with a
// stride of S floats (coalesced across neighbouring t).  The kernel is bound
// by HBM bandwidth: it reads G (or 1) floats and writes 1 float per score.
#include "kvp_device.h"
#include "kvp_launch.h"

namespace kvp {
namespace {

struct TargetArgs {
  const float* mass;
  const float* log_gamma;
  float* score;
  int B, Hq, Hkv, S, G;
  int per_head, window, normalize, agg, query, decay_step;
  float eps;
};

__global__ __launch_bounds__(256) void target_kernel(TargetArgs a) {
  const int64_t n = (int64_t)a.B * a.Hkv * a.S;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int S = a.S;
  const int t = (int)(idx % S);
  const int64_t bh = idx / S;
  const int h = (int)(bh % a.Hkv);
  const int b = (int)(bh / a.Hkv);
  const int nt = S - (t + a.window);
  const float inv_n = a.normalize ? 1.0f / (float)(nt > 1 ? nt : 1) : 1.0f;

  float r;
  if (a.per_head) {
    const float* m = a.mass + ((int64_t)b * a.Hq + (int64_t)h * a.G) * S + t;
    if (a.agg == 0) {  // log of the group mean
      float sum = 0.f;
      for (int g = 0; g < a.G; ++g) sum += m[(int64_t)g * S];
      r = __logf(a.eps + sum * inv_n / (float)a.G);
    } else if (a.agg == 1) {  // mean of the logs
      float sum = 0.f;
      for (int g = 0; g < a.G; ++g) sum += __logf(a.eps + m[(int64_t)g * S] * inv_n);
      r = sum / (float)a.G;
    } else {  // max of the logs
      r = -__builtin_inff();
      for (int g = 0; g < a.G; ++g) r = fmaxf(r, __logf(a.eps + m[(int64_t)g * S] * inv_n));
    }
  } else {  // group sums: only the log of the group mean is defined
    r = __logf(a.eps + a.mass[idx] * inv_n / (float)a.G);
  }
  if (a.query >= 0) {
    if (t > a.query)
      r = -__builtin_inff();
    else
      r += (float)((a.query - t) / a.decay_step) * a.log_gamma[h];
  }
  a.score[idx] = r;
}

// Static priorities of the running top-k (KVpop §3.2 with App. B.3): the
// decayed score at query q is r[t] + floor((q - t) / n) log gamma_h, whose
// query-dependent part floor(q / n) log gamma_h is shared by every token up
// to one decay step, so tokens are ranked once by
//   pi[b, h, t] = r[b, h, t] - floor(t / n) * log gamma_h
// (one fused multiply-add, correctly rounded; in place allowed).
__global__ __launch_bounds__(256) void priority_kernel(const float* score, const float* log_gamma,
                                                       float* pri, int64_t n, int Hkv, int S,
                                                       int decay_step) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int t = (int)(idx % S);
  const int h = (int)((idx / S) % Hkv);
  pri[idx] = __builtin_fmaf(-(float)(t / decay_step), log_gamma[h], score[idx]);
}

}  // namespace

hipError_t launch_priority(const float* score, const Shape& sh, int decay_step,
                           const float* log_gamma, float* priority, hipStream_t stream) {
  const int64_t n = (int64_t)sh.B * sh.Hkv * sh.S;
  hipLaunchKernelGGL(priority_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     score, log_gamma, priority, n, sh.Hkv, sh.S, decay_step);
  return hipGetLastError();
}

hipError_t launch_target(const float* mass, int per_head, const Shape& sh, int window,
                         int normalize, int agg, float eps, int query, int decay_step,
                         const float* log_gamma, float* score, hipStream_t stream) {
  TargetArgs a;
  a.mass = mass;
  a.log_gamma = log_gamma;
  a.score = score;
  a.B = sh.B;
  a.Hq = sh.Hq;
  a.Hkv = sh.Hkv;
  a.S = sh.S;
  a.G = sh.G;
  a.per_head = per_head;
  a.window = window;
  a.normalize = normalize;
  a.agg = agg;
  a.query = query;
  a.decay_step = decay_step;
  a.eps = eps;
  const int64_t n = (int64_t)sh.B * sh.Hkv * sh.S;
  hipLaunchKernelGGL(target_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvp
