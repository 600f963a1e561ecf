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
// F(z_i) <= k, and the closed form over that split gives lam.
//   * Rows of up to 32768 (soft_topk_fwd_lds_kernel): the row sits in LDS; a
//     Newton search in fp32 brackets the split, and one fp64 pass over the
//     snapped bracket checks it and forms the sums (details below).
//   * Longer rows (soft_topk_fwd_kernel): bisection on the order-preserving
//     32-bit keys of x (at most 32 block reductions in fp64), then one pass
//     forms S1, S2 relative to the smallest element of the split (every term
//     <= 1).
// The sums, the closed form and y are fp64 in both.
//
// Backward (App. A.2): with f'(u) = e^{-|u|} / 2 and u_i = z_i - lam,
//   dz_j = f'(u_j) (dy_j - A / B),  A = sum_i dy_i f'(u_i),  B = sum_i f'(u_i),
//   dx = dz / tau,  dk = A / B.
#include <utility>

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

// Workgroup maximum of a double (every thread gets it).
__device__ double block_max(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red free from any previous use
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  double t = red[0];
#pragma unroll
  for (int w = 1; w < kStWaves; ++w) t = fmax(t, red[w]);
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
    // split: elements with key >= hi (case 0: none; case 2: all).  Its
    // smallest element c and the largest other element lop are the
    // references: split terms e^{-(z - c)}, the others e^{z - lop}, each side
    // holding a term equal to 1, so the sums neither overflow nor vanish.
    auto in_split = [&](float xi) { return case_m == 2 || (case_m == 1 && st_key(xi) >= hi); };
    double cneg = -__builtin_inf(), lop = -__builtin_inf();
    for (int i = tid; i < n; i += kStThreads) {
      const float xi = x[i];
      const double z = (double)xi * it;
      if (in_split(xi))
        cneg = fmax(cneg, -z);
      else
        lop = fmax(lop, z);
    }
    cneg = block_max(cneg, red);
    lop = block_max(lop, red);
    const double c = -cneg;
    double m = 0.0, sa = 0.0, sb = 0.0;
    for (int i = tid; i < n; i += kStThreads) {
      const float xi = x[i];
      const double z = (double)xi * it;
      if (in_split(xi)) {
        m += 1.0;
        sa += exp(-(z - c));
      } else {
        sb += exp(z - lop);
      }
    }
    m = block_sum(m, red);
    sa = block_sum(sa, red);
    sb = block_sum(sb, red);
    if (case_m == 0) {
      lam = lop + log(sb / (2.0 * kk));  // lop is the row maximum
    } else if (case_m == 2) {
      lam = c + log(2.0 * ((double)n - kk) / sa);  // c is the row minimum
    } else {
      // with Y = e^{lam - c}: A Y^2 + 2 (k - m) Y - B = 0, A = sa,
      // B = e^{-(c - lop)} sb; taken in logs so that A B may underflow
      const double av = kk - m;
      const double log_a = log(sa), log_b = log(sb) - (c - lop);
      const double root = sqrt(av * av + exp(log_a + log_b));
      if (av > 0.0)
        lam = c + log_b - log(root + av);  // Y A = A B / (root + a)
      else if (av < 0.0)
        lam = c + log(root - av) - log_a;
      else
        lam = c + 0.5 * (log_b - log_a);
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


// ---- rows of up to kStMaxLds scores, held in LDS (soft_topk_fwd_lds_kernel).
// The threshold is bracketed by a safeguarded Newton iteration on F(t) = k
// (F' = -sum_i f'(z_i - t) comes from the same exponential; a bisection
// step is taken when Newton leaves the bracket and every fourth step).  The
// search runs in fp32 in the units of x, so its bracket ends are floats and
// its element tests exact: it ends with no element strictly inside the
// bracket (at worst, two adjacent floats).  The bracket is then snapped to
// the elements around it (lop <= lo, c >= hi) and one fp64 pass gives the
// split size m, A = sum_{z >= c} e^{-(z - c)}, B' = sum_{z < c} e^{z - lop}
// and from them F(c), F(lop):
//   F(c) <= k < F(lop)               -> split = {z >= c}, closed form in logs
//   F(c) > k and c the row maximum   -> lam above every element
//   F(lop) <= k and lop the row min  -> lam below every element
// Anything else (fp32 misjudged a step) reruns the search in fp64 on z.

constexpr int kStRegThreads = 512;
constexpr int kStRegWaves = kStRegThreads / kWave;
constexpr int kStMaxLds = 32768;

// Workgroup sums of N doubles at once (every thread gets the totals).
template <int N>
__device__ void block_sums(double* v, double (*red)[8]) {
  static_assert(N <= 8, "reduction table holds 8 values per wave");
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v[i] += __shfl_xor(v[i], off);
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red free from any previous use
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int i = 0; i < N; ++i) red[wave][i] = v[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kStRegWaves; ++w) t += red[w][i];
    v[i] = t;
  }
}

// Workgroup maxima of two floats (every thread gets them).
__device__ void block_max2f(float& a0, float& a1, double (*red)[8]) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a0 = fmaxf(a0, __shfl_xor(a0, off));
    a1 = fmaxf(a1, __shfl_xor(a1, off));
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red[wave][0] = a0;
    red[wave][1] = a1;
  }
  __syncthreads();
  a0 = (float)red[0][0];
  a1 = (float)red[0][1];
#pragma unroll
  for (int w = 1; w < kStRegWaves; ++w) {
    a0 = fmaxf(a0, (float)red[w][0]);
    a1 = fmaxf(a1, (float)red[w][1]);
  }
}

// Workgroup maxima of two doubles (every thread gets them).
__device__ void block_max2(double& a0, double& a1, double (*red)[8]) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a0 = fmax(a0, __shfl_xor(a0, off));
    a1 = fmax(a1, __shfl_xor(a1, off));
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    red[wave][0] = a0;
    red[wave][1] = a1;
  }
  __syncthreads();
  a0 = red[0][0];
  a1 = red[0][1];
#pragma unroll
  for (int w = 1; w < kStRegWaves; ++w) {
    a0 = fmax(a0, red[w][0]);
    a1 = fmax(a1, red[w][1]);
  }
}

__global__ __launch_bounds__(kStRegThreads) void soft_topk_fwd_lds_kernel(StArgs a) {
  __shared__ double red[kStRegWaves][8];
  __shared__ float xs[kStMaxLds];
  const int n = a.n;
  const float* __restrict__ x = a.x + (size_t)blockIdx.x * n;
  float* __restrict__ y = a.y + (size_t)blockIdx.x * n;
  const double kk = (double)a.k[blockIdx.x];
  const double it = a.inv_tau;
  const float it32 = (float)it;
  const int tid = threadIdx.x;

  float xmin_neg = -__builtin_inff(), xmax = -__builtin_inff();
  for (int i = tid; i < n; i += kStRegThreads) {
    const float xi = x[i];
    xs[i] = xi;
    xmin_neg = fmaxf(xmin_neg, -xi);
    xmax = fmaxf(xmax, xi);
  }
  block_max2f(xmin_neg, xmax, red);  // its barriers also publish xs
  const float xmin = -xmin_neg;
  const double zmin = (double)xmin * it, zmax = (double)xmax * it;

  // fp32 search pass at tx (x units): F, |dF/dz| and the elements in
  // (lo, tx) and (tx, hi)
  auto eval32 = [&](float tx, float lo, float hi, double (&r)[8]) __attribute__((always_inline)) {
    float f = 0.f, d = 0.f;
    int c_lo = 0, c_hi = 0;
#pragma unroll 4
    for (int i = tid; i < n; i += kStRegThreads) {
      const float xi = xs[i];
      const float u = (xi - tx) * it32;
      const float ex = __expf(-fabsf(u));
      f += u >= 0.f ? 1.f - 0.5f * ex : 0.5f * ex;
      d += 0.5f * ex;
      c_lo += (xi > lo && xi < tx) ? 1 : 0;
      c_hi += (xi > tx && xi < hi) ? 1 : 0;
    }
    r[0] = f;
    r[1] = d;
    r[2] = c_lo;
    r[3] = c_hi;
    block_sums<4>(r, red);
  };
  // fp64 search pass at t (z units), the same quantities
  auto eval64 = [&](double t, double lo, double hi, double (&r)[8]) __attribute__((always_inline)) {
    double f = 0.0, d = 0.0, c_lo = 0.0, c_hi = 0.0;
#pragma unroll 4
    for (int i = tid; i < n; i += kStRegThreads) {
      const double z = (double)xs[i] * it;
      const double u = z - t;
      const double ex = exp(-fabs(u));
      f += u >= 0.0 ? 1.0 - 0.5 * ex : 0.5 * ex;
      d += 0.5 * ex;
      c_lo += (z > lo && z < t) ? 1.0 : 0.0;
      c_hi += (z > t && z < hi) ? 1.0 : 0.0;
    }
    r[0] = f;
    r[1] = d;
    r[2] = c_lo;
    r[3] = c_hi;
    block_sums<4>(r, red);
  };
  // Safeguarded Newton in the bracket (lo, hi), from t with g = F(t) - k and
  // dabs = |F'(t)| in z units (tscale = z units per unit of T); returns with
  // no element strictly inside.  Bounded: the bracket at least halves every
  // fourth step and empties when no value of T lies strictly inside.
  auto search = [&](auto lo, auto hi, auto t, double g, double dabs, double tscale,
                    auto&& eval) __attribute__((always_inline)) {
    using T = decltype(t);
    double r[8];
    for (int step = 0; step < 4096; ++step) {
      T tn = (T)((double)t + g / (dabs * tscale));  // t - g / F'(t)
      if (!(tn > lo && tn < hi) || (step & 3) == 3) tn = (T)(0.5 * ((double)lo + (double)hi));
      if (!(tn > lo && tn < hi)) break;  // no value strictly inside: no element either
      t = tn;
      eval(t, lo, hi, r);
      g = r[0] - kk;
      dabs = r[1];
      bool empty;
      if (g > 0.0) {
        lo = t;
        empty = r[3] == 0.0;  // elements in (t, hi)
      } else {
        hi = t;
        empty = r[2] == 0.0;  // elements in (lo, t)
      }
      if (empty) break;
    }
    return std::pair<T, T>(lo, hi);
  };

  double lam;
  if (!(kk > 0.0)) {
    lam = __builtin_inf();  // no budget: every y = 0
  } else if (!(kk < (double)n)) {
    lam = -__builtin_inf();  // the whole row: every y = 1
  } else {
    // fp32 search from the middle of the row's range
    double r[8];
    const float tx0 = 0.5f * (xmin + xmax);
    float lo_x = xmin, hi_x = xmax;
    if (tx0 > xmin && tx0 < xmax) {
      eval32(tx0, xmin, xmax, r);
      const double g0 = r[0] - kk;
      bool empty;
      if (g0 > 0.0) {
        lo_x = tx0;
        empty = r[3] == 0.0;
      } else {
        hi_x = tx0;
        empty = r[2] == 0.0;
      }
      if (!empty) {
        const auto b = search(lo_x, hi_x, tx0, g0, r[1], it, eval32);
        lo_x = b.first;
        hi_x = b.second;
      }
    }
    double lo = (double)lo_x * it, hi = (double)hi_x * it;
    // Snap the bracket to the elements around it: lop = the largest z <= lo,
    // c = the smallest z >= hi (no element lies between them, and F(lop) >=
    // F(lo), F(c) <= F(hi)).  One fp64 pass then takes split terms relative
    // to c and the others relative to lop, each side holding a term equal
    // to 1, and gives F(c) and F(lop) with the factor e^{-(c - lop)} <= 1.
    // On a misjudged fp32 bracket it runs once more after an fp64 search.
    for (int attempt = 0;; ++attempt) {
      double lop_v = -__builtin_inf(), cneg = -__builtin_inf();
      for (int i = tid; i < n; i += kStRegThreads) {
        const double z = (double)xs[i] * it;
        if (z <= lo) lop_v = fmax(lop_v, z);
        if (z >= hi) cneg = fmax(cneg, -z);
      }
      block_max2(lop_v, cneg, red);  // both exist: lo >= zmin and hi <= zmax
      const double lop = lop_v, c = -cneg;
      double s[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};  // m, A, B'
#pragma unroll 4
      for (int i = tid; i < n; i += kStRegThreads) {
        const double z = (double)xs[i] * it;
        if (z >= c) {
          s[0] += 1.0;
          s[1] += exp(-(z - c));
        } else {
          s[2] += exp(z - lop);
        }
      }
      block_sums<3>(s, red);
      const double m = s[0], A = s[1], Bp = s[2];
      const double eg = exp(-(c - lop));
      const double f_c = m - 0.5 * A + 0.5 * eg * Bp;
      const double f_lo = m - 0.5 * eg * A + 0.5 * Bp;
      if (f_c <= kk && f_lo > kk) {
        // split {z >= c}: with Y = e^{lam - c}, A Y^2 + 2 (k - m) Y - B = 0,
        // B = e^{-(c - lop)} B'; taken in logs so that A B may underflow
        const double av = kk - m;
        const double log_a = log(A), log_b = log(Bp) - (c - lop);
        const double root = sqrt(av * av + exp(log_a + log_b));
        if (av > 0.0)
          lam = c + log_b - log(root + av);  // Y A = A B / (root + a)
        else if (av < 0.0)
          lam = c + log(root - av) - log_a;
        else
          lam = c + 0.5 * (log_b - log_a);
        break;
      }
      if (f_c > kk && c >= zmax) {  // above every element: sum_i e^{z_i - zmax}
        lam = zmax + log((m + eg * Bp) / (2.0 * kk));
        break;
      }
      if (f_lo <= kk && lop <= zmin) {  // below every element: sum_i e^{-(z_i - zmin)}
        lam = zmin + log(2.0 * ((double)n - kk) / (((double)n - m) + eg * A));
        break;
      }
      if (attempt > 0) {  // not reached: an fp64 bracket meets one of the above
        lam = __builtin_nan("");
        break;
      }
      // fp64 search in z units: the ends first, then Newton inside
      eval64(zmax, zmin, zmax, r);
      if (r[0] > kk) {
        lo = hi = zmax;
        continue;
      }
      double r2[8];
      eval64(zmin, zmin, zmax, r2);
      if (r2[0] <= kk) {
        lo = hi = zmin;
        continue;
      }
      const auto b = search(zmin, zmax, zmin, r2[0] - kk, r2[1], 1.0, eval64);
      lo = b.first;
      hi = b.second;
    }
  }
  if (tid == 0 && a.lam_out) a.lam_out[blockIdx.x] = (float)lam;
#pragma unroll 4
  for (int i = tid; i < n; i += kStRegThreads) y[i] = (float)laplace_cdf((double)xs[i] * it - lam);
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
  if (n <= kStMaxLds)
    hipLaunchKernelGGL(soft_topk_fwd_lds_kernel, dim3((unsigned)rows), dim3(kStRegThreads), 0, stream, a);
  else
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
