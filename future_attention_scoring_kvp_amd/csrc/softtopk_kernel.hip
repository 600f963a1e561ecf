// LKV's Soft-TopK for gfx950: forward (closed-form threshold) and backward.
//
// Per row of n scores x and budget k in (0, n), with z = x / tau:
//   y_i = f(z_i - lam),  f(u) = 1 - e^{-u}/2 (u >= 0), e^{u}/2 (u < 0)
// (the Laplace CDF), lam chosen so that sum_i y_i = k ("LKV: End-to-End
// Learning of Head-wise Budgets and Token Selection for LLM KV Cache
// Eviction", §3.2 and App. A.1).  For the split m (the elements z_i >= lam),
// e^{lam} solves S1 y^2 + 2 (k - m) y - S2 = 0 with S1 = sum_{z_i >= lam}
// e^{-z_i}, S2 = sum_{z_i < lam} e^{z_i}.
//
// One workgroup per row, no sort: F(t) = sum_i f(z_i - t) decreases in t and
// F(lam) = k, so the split is the set of elements whose value satisfies
// F(z_i) <= k.  Its boundary is found by bisection on the order-preserving
// 32-bit keys of x (at most 32 block reductions), then one pass forms S1, S2
// relative to the smallest element of the split (every term <= 1) and the
// closed form gives lam.  All per-row arithmetic is fp64.
//
// Backward (App. A.2): with f'(u) = e^{-|u|} / 2 and u_i = z_i - lam,
//   dz_j = f'(u_j) (dy_j - A / B),  A = sum_i dy_i f'(u_i),  B = sum_i f'(u_i),
//   dx = dz / tau,  dk = A / B.
#include "kvp_device.h"
#include "kvp_launch.h"

namespace kvp {
namespace {

constexpr int kStThreads = 256;
constexpr int kStWaves = kStThreads / kWave;

__device__ __forceinline__ uint32_t st_key(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if (u == 0x80000000u) u = 0u;  // -0 ties +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float st_value(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __builtin_bit_cast(float, u);
}

__device__ __forceinline__ double laplace_cdf(double u) {
  return u >= 0.0 ? 1.0 - 0.5 * exp(-u) : 0.5 * exp(u);
}

// Workgroup sum of a double (every thread gets the total).
__device__ double block_sum(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red free from any previous use
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kStWaves; ++w) t += red[w];
  return t;
}

__device__ uint32_t block_min_u32(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, off));
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  uint32_t t = red[0];
#pragma unroll
  for (int w = 1; w < kStWaves; ++w) t = min(t, red[w]);
  return t;
}

struct StArgs {
  const float* x;
  const float* k;    // [rows]
  const float* lam;  // backward input [rows]
  const float* dy;
  float* y;
  float* lam_out;    // [rows] or null
  float* dx;
  float* dk;         // [rows] or null
  int n;
  double inv_tau;
};

__global__ __launch_bounds__(kStThreads) void soft_topk_fwd_kernel(StArgs a) {
  __shared__ double red[kStWaves];
  __shared__ uint32_t redu[kStWaves];
  const int n = a.n;
  const float* __restrict__ x = a.x + (size_t)blockIdx.x * n;
  float* __restrict__ y = a.y + (size_t)blockIdx.x * n;
  const double kk = (double)a.k[blockIdx.x];
  const double it = a.inv_tau;
  const int tid = threadIdx.x;

  // key range of the row
  uint32_t kmin = 0xFFFFFFFFu, kmax_inv = 0xFFFFFFFFu;
  for (int i = tid; i < n; i += kStThreads) {
    const uint32_t kv = st_key(x[i]);
    kmin = min(kmin, kv);
    kmax_inv = min(kmax_inv, ~kv);
  }
  kmin = block_min_u32(kmin, redu);
  const uint32_t kmax = ~block_min_u32(kmax_inv, redu);

  auto F = [&](double t) {  // sum_i f(z_i - t)
    double s = 0.0;
    for (int i = tid; i < n; i += kStThreads) s += laplace_cdf((double)x[i] * it - t);
    return block_sum(s, red);
  };

  double lam;
  if (!(kk > 0.0)) {
    lam = __builtin_inf();  // no budget: every y = 0
  } else if (!(kk < (double)n)) {
    lam = -__builtin_inf();  // the whole row: every y = 1
  } else {
    const double zmax = (double)st_value(kmax) * it;
    const double zmin = (double)st_value(kmin) * it;
    int case_m;  // 0: lam above every element, 2: below every element, 1: split inside
    uint32_t hi = kmax;
    if (F(zmax) > kk) {
      case_m = 0;
    } else if (F(zmin) <= kk) {
      case_m = 2;
      hi = kmin;
    } else {
      case_m = 1;
      uint32_t lo = kmin;  // F > k at lo, F <= k at hi
      while (hi - lo > 1u) {
        const uint32_t mid = lo + (hi - lo) / 2u;
        if (F((double)st_value(mid) * it) <= kk)
          hi = mid;
        else
          lo = mid;
      }
    }
    // split: elements with key >= hi; shift c = value at hi (case 0: the
    // maximum, every element is below the threshold)
    const double c = (double)st_value(hi) * it;
    double m = 0.0, s1 = 0.0, s2 = 0.0;
    for (int i = tid; i < n; i += kStThreads) {
      const float xi = x[i];
      const double z = (double)xi * it;
      if (case_m != 0 && st_key(xi) >= hi) {
        m += 1.0;
        s1 += exp(-(z - c));
      } else {
        s2 += exp(z - c);
      }
    }
    m = block_sum(m, red);
    s1 = block_sum(s1, red);
    s2 = block_sum(s2, red);
    const double av = kk - m;
    if (case_m == 0) {
      lam = c + log(s2 / (2.0 * kk));
    } else if (case_m == 2) {
      lam = c + log(2.0 * ((double)n - kk) / s1);
    } else {
      const double p = s1 * s2;  // <= m (n - m)
      const double root = sqrt(av * av + p);
      // y s1 = sqrt(a^2 + p) - a, without cancellation for a > 0
      const double ys1 = av > 0.0 ? p / (root + av) : root - av;
      lam = c + log(ys1) - log(s1);
    }
  }
  if (tid == 0 && a.lam_out) a.lam_out[blockIdx.x] = (float)lam;
  for (int i = tid; i < n; i += kStThreads) y[i] = (float)laplace_cdf((double)x[i] * it - lam);
}

__global__ __launch_bounds__(kStThreads) void soft_topk_bwd_kernel(StArgs a) {
  __shared__ double red[kStWaves];
  const int n = a.n;
  const size_t o = (size_t)blockIdx.x * n;
  const double lam = (double)a.lam[blockIdx.x];
  const double it = a.inv_tau;
  const int tid = threadIdx.x;
  double sa = 0.0, sb = 0.0;
  for (int i = tid; i < n; i += kStThreads) {
    const double fp = 0.5 * exp(-fabs((double)a.x[o + i] * it - lam));
    sa += (double)a.dy[o + i] * fp;
    sb += fp;
  }
  sa = block_sum(sa, red);
  sb = block_sum(sb, red);
  const double r = sb > 0.0 ? sa / sb : 0.0;
  if (tid == 0 && a.dk) a.dk[blockIdx.x] = (float)r;
  for (int i = tid; i < n; i += kStThreads) {
    const double fp = 0.5 * exp(-fabs((double)a.x[o + i] * it - lam));
    a.dx[o + i] = (float)(fp * ((double)a.dy[o + i] - r) * it);
  }
}

}  // namespace

hipError_t launch_soft_topk_fwd(const float* x, const float* k, int64_t rows, int n, float tau,
                                float* y, float* lam, hipStream_t stream) {
  StArgs a{};
  a.x = x;
  a.k = k;
  a.y = y;
  a.lam_out = lam;
  a.n = n;
  a.inv_tau = 1.0 / (double)tau;
  hipLaunchKernelGGL(soft_topk_fwd_kernel, dim3((unsigned)rows), dim3(kStThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_soft_topk_bwd(const float* x, const float* lam, const float* dy, int64_t rows,
                                int n, float tau, float* dx, float* dk, hipStream_t stream) {
  StArgs a{};
  a.x = x;
  a.lam = lam;
  a.dy = dy;
  a.dx = dx;
  a.dk = dk;
  a.n = n;
  a.inv_tau = 1.0 / (double)tau;
  hipLaunchKernelGGL(soft_topk_bwd_kernel, dim3((unsigned)rows), dim3(kStThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvp
