/*
 * CPU ORACLE for the future-attention-mass path — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow fp64 implementation of what the GPU library computes, used
 * only to check it: the tests, the smoke check and the benchmark's CPU
 * baseline load it; the library itself never does.  It shares no code,
 * header, table or constant with the HIP path.
 *
 * Sources (cited by page title and section/equation):
 *   [KVpop] "KVpop — Key-Value Cache Compression with Predictive Online
 *           Pruning" (arXiv 2607.05061).
 *   [LKV]   "LKV: End-to-End Learning of Head-wise Budgets and Token Selection
 *           for LLM KV Cache Eviction" (arXiv 2605.06676).
 *   [Tut]   the KV-compression tutorial page of the "transformer math" series
 *           (aicassindra), sections "H2O: evict by accumulated attention" and
 *           "StreamingLLM and the attention-sink surprise".
 *
 * What is computed, and from where:
 *   logits  l(i,j) = scale * <q_i, k_j>, scale = 1/sqrt(d) by default, over
 *           the causal prefix j <= i: the scaled dot-product causal softmax of
 *           [LKV] §3 Preliminaries ("The KV Cache Bottleneck", Eq. 1).
 *   LSE_i   log of the dense causal softmax normaliser of row i, the
 *           "log-normalizer" that [KVpop] §3.2 (Eq. 8) reuses.
 *   p(i->j) = softmax row i at column j = exp(l(i,j) - LSE_i).
 *   mass    [KVpop] §3.1 Eq. 2 future-attention mass in its un-normalised form
 *           of App. B.1 (sum of p(d->t) over d = t+w .. S-1, no 1/N_t), summed
 *           over the G query heads that share KV head h.  App. B.1 averages
 *           over the G heads; the plain sum ranks identically.
 *   keep    [KVpop] §3 Eq. 1 (budget B = s + w + k per KV head) with Fig. 1
 *           (sinks and protected recent window always kept, remaining slots to
 *           the top-k long-range tokens) and Eq. 4 (eligible set at the last
 *           query q = S-1: s <= t <= S-1-w).  Ties in mass go to the lower
 *           index (no page addresses ties).
 *
 * Input dtypes: 0 = bfloat16 bit patterns; 1 = float32, rounded to bfloat16
 * (round to nearest even) by this file's own routine before use, i.e. the
 * values a bf16 kernel consumes; 2 = float32 used exactly.
 *
 * Parallelism does not change the arithmetic of a sum: the query rows of each
 * (batch, query head) are split into a fixed number of interleaved row
 * partitions, each with its own fp64 column buffer, and the buffers are added
 * in a fixed order (query head, then partition).  Results do not depend on
 * the thread count.
 */
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <utility>
#include <vector>

namespace {

constexpr int kRowBlock = 64;    // rows per block inside a partition
constexpr int kPartitions = 16;  // fixed row partitions per (b, query head)

// bfloat16 (bit pattern) -> double, exact.
double bf16_to_double(uint16_t h) {
  uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

// float32 -> bfloat16 bit pattern, round to nearest, ties to even.
uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) {  // inf / nan: keep class
    uint16_t r = static_cast<uint16_t>(u >> 16);
    if ((u & 0x007FFFFFu) != 0) r |= 0x0040u;
    return r;
  }
  uint32_t upper = u >> 16;
  uint32_t lower = u & 0xFFFFu;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1;
  return static_cast<uint16_t>(upper);
}

double load_elem(const void* base, int dtype, int64_t idx) {
  if (dtype == 0) return bf16_to_double(static_cast<const uint16_t*>(base)[idx]);
  const float f = static_cast<const float*>(base)[idx];
  if (dtype == 1) return bf16_to_double(float_to_bf16_rne(f));
  return static_cast<double>(f);
}

struct Dims {
  int64_t B, Hq, Hkv, S, D;
};

// One causal softmax row: logits l(i, 0..i), the LSE and p(i->j) = e_j / Z.
// kt is K of the row's KV head, transposed to [D][S] (so the dot products
// for all j are formed column by column; each l(i,j) still accumulates
// q[0]k[0] + q[1]k[1] + ... in index order).
struct RowResult {
  double lse;
  double rowsum;
};

RowResult softmax_row(const double* qi, const double* kt, int64_t S, int64_t D, int64_t i,
                      double scale, std::vector<double>& logit) {
  const int64_t n = i + 1;
  for (int64_t j = 0; j < n; ++j) logit[j] = 0.0;
  for (int64_t c = 0; c < D; ++c) {
    const double qc = qi[c];
    const double* kc = kt + c * S;
    for (int64_t j = 0; j < n; ++j) logit[j] += qc * kc[j];
  }
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j) {
    logit[j] *= scale;
    m = std::max(m, logit[j]);
  }
  double z = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    logit[j] = std::exp(logit[j] - m);  // now e_j
    z += logit[j];
  }
  double rowsum = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    logit[j] /= z;  // now p(i->j)
    rowsum += logit[j];
  }
  return {m + std::log(z), rowsum};
}

void widen_head(const void* src, int dtype, int64_t head_offset, int64_t S, int64_t D,
                std::vector<double>& dst) {
  dst.resize(static_cast<size_t>(S * D));
  for (int64_t t = 0; t < S * D; ++t) dst[t] = load_elem(src, dtype, head_offset + t);
}

void transpose_head(const std::vector<double>& k, int64_t S, int64_t D, std::vector<double>& kt) {
  kt.resize(static_cast<size_t>(S * D));
  for (int64_t j = 0; j < S; ++j)
    for (int64_t c = 0; c < D; ++c) kt[c * S + j] = k[j * D + c];
}

template <typename F>
void parallel_items(int64_t n_items, int nthreads, F&& fn) {
  if (nthreads < 1) nthreads = 1;
  if (n_items < nthreads) nthreads = static_cast<int>(std::max<int64_t>(n_items, 1));
  std::atomic<int64_t> next{0};
  auto worker = [&]() {
    for (;;) {
      const int64_t it = next.fetch_add(1);
      if (it >= n_items) break;
      fn(it);
    }
  };
  std::vector<std::thread> pool;
  for (int t = 1; t < nthreads; ++t) pool.emplace_back(worker);
  worker();
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

int kvp_oracle_abi_version() { return 1; }

int oracle_round_bf16(const float* x, int64_t n, uint16_t* out) {
  if ((!x || !out) && n > 0) return 1;
  for (int64_t i = 0; i < n; ++i) out[i] = float_to_bf16_rne(x[i]);
  return 0;
}

/* Dense causal softmax of every query row, its LSE, and the future mass.
 *
 *   lse[b,g,i]     = ln sum_{j<=i} exp(l_g(i,j))                  ([B,Hq,S])
 *   mass[b,h,j]    = sum_{g: g/G = h} sum_{i >= j+window} p_g(i->j)  ([B,Hkv,S])
 *   mass_heads[b,g,j] = sum_{i >= j+window} p_g(i->j), each query head on its
 *                    own: the per-head mass m^(h,g) of [KVpop] §3.1 Eq. 2 in
 *                    the un-normalised form of App. B.1     ([B,Hq,S]; optional)
 *   rowsum[b,g,i]  = sum_{j<=i} p_g(i->j)          (should be 1; optional)
 *   winmass[b,g,i] = sum_{i-window < j <= i} p_g(i->j)  (in-window mass; optional)
 *
 * b_only / h_only >= 0 restrict the work to one batch element / KV head (the
 * other outputs are left untouched); rows below row_lo are skipped, which
 * leaves mass[j] exact for every j >= row_lo - window.  Any output pointer may
 * be NULL.  Returns 0, or 1 on invalid arguments. */
int oracle_future_mass(const void* q, const void* k, int dtype, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t S, int64_t D, double scale, int64_t window,
                       int64_t b_only, int64_t h_only, int64_t row_lo, int nthreads,
                       double* lse, double* mass, double* rowsum, double* winmass,
                       double* mass_heads) {
  if (!q || !k || B < 0 || Hq < 1 || Hkv < 1 || S < 0 || D < 1 || Hq % Hkv != 0 ||
      window < 0 || dtype < 0 || dtype > 2 || row_lo < 0)
    return 1;
  if (!(scale > 0.0)) scale = 1.0 / std::sqrt(static_cast<double>(D));
  const int64_t G = Hq / Hkv;
  const Dims dm{B, Hq, Hkv, S, D};

  for (int64_t b = 0; b < dm.B; ++b) {
    if (b_only >= 0 && b != b_only) continue;
    for (int64_t h = 0; h < dm.Hkv; ++h) {
      if (h_only >= 0 && h != h_only) continue;
      std::vector<double> kh, kt;
      widen_head(k, dtype, (b * Hkv + h) * S * D, S, D, kh);
      transpose_head(kh, S, D, kt);
      std::vector<std::vector<double>> qheads(static_cast<size_t>(G));
      for (int64_t gg = 0; gg < G; ++gg)
        widen_head(q, dtype, (b * Hq + h * G + gg) * S * D, S, D, qheads[gg]);

      const int64_t n_items = G * kPartitions;
      std::vector<std::vector<double>> colbuf(static_cast<size_t>(n_items));
      parallel_items(n_items, nthreads, [&](int64_t item) {
        const int64_t gg = item / kPartitions;
        const int64_t part = item % kPartitions;
        const int64_t g = h * G + gg;  // query head g uses KV head g / G
        std::vector<double>& col = colbuf[item];
        col.assign(static_cast<size_t>(S), 0.0);
        std::vector<double> p(static_cast<size_t>(S > 0 ? S : 1));
        const double* qbase = qheads[gg].data();
        for (int64_t blk = part; blk * kRowBlock < S; blk += kPartitions) {
          const int64_t i0 = blk * kRowBlock;
          const int64_t i1 = std::min(S, i0 + kRowBlock);
          for (int64_t i = std::max(i0, row_lo); i < i1; ++i) {
            const RowResult rr = softmax_row(qbase + i * D, kt.data(), S, D, i, scale, p);
            const int64_t o = (b * Hq + g) * S + i;
            if (lse) lse[o] = rr.lse;
            if (rowsum) rowsum[o] = rr.rowsum;
            double win = 0.0;
            // query i counts for key j iff i >= j + window ([KVpop] Eq. 2 lower limit d = t + w)
            for (int64_t j = 0; j <= i; ++j) {
              if (j + window <= i)
                col[j] += p[j];
              else
                win += p[j];
            }
            if (winmass) winmass[o] = win;
          }
        }
      });
      if (mass) {
        double* out = mass + (b * Hkv + h) * S;
        for (int64_t j = 0; j < S; ++j) {
          double acc = 0.0;
          for (int64_t it = 0; it < n_items; ++it) acc += colbuf[it][j];
          out[j] = acc;
        }
      }
      if (mass_heads) {
        for (int64_t gg = 0; gg < G; ++gg) {
          double* out = mass_heads + (b * Hq + h * G + gg) * S;
          for (int64_t j = 0; j < S; ++j) {
            double acc = 0.0;
            for (int64_t part = 0; part < kPartitions; ++part) acc += colbuf[gg * kPartitions + part][j];
            out[j] = acc;
          }
        }
      }
    }
  }
  return 0;
}

/* LSE of selected rows only: rows[3r .. 3r+2] = (b, g, i).  Each costs one
 * causal row, O(i * D). */
int oracle_lse_rows(const void* q, const void* k, int dtype, int64_t B, int64_t Hq, int64_t Hkv,
                    int64_t S, int64_t D, double scale, const int64_t* rows, int64_t n_rows,
                    int nthreads, double* lse_out) {
  if (!q || !k || !rows || !lse_out || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D < 1 ||
      dtype < 0 || dtype > 2)
    return 1;
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t b = rows[3 * r], g = rows[3 * r + 1], i = rows[3 * r + 2];
    if (b < 0 || b >= B || g < 0 || g >= Hq || i < 0 || i >= S) return 1;
  }
  if (!(scale > 0.0)) scale = 1.0 / std::sqrt(static_cast<double>(D));
  const int64_t G = Hq / Hkv;
  parallel_items(n_rows, nthreads, [&](int64_t r) {
    const int64_t b = rows[3 * r], g = rows[3 * r + 1], i = rows[3 * r + 2];
    const int64_t h = g / G;
    std::vector<double> qi(static_cast<size_t>(D));
    for (int64_t c = 0; c < D; ++c) qi[c] = load_elem(q, dtype, ((b * Hq + g) * S + i) * D + c);
    std::vector<double> logit(static_cast<size_t>(i + 1));
    double m = -INFINITY;
    for (int64_t j = 0; j <= i; ++j) {
      double dot = 0.0;
      for (int64_t c = 0; c < D; ++c) dot += qi[c] * load_elem(k, dtype, ((b * Hkv + h) * S + j) * D + c);
      logit[j] = scale * dot;
      m = std::max(m, logit[j]);
    }
    double z = 0.0;
    for (int64_t j = 0; j <= i; ++j) z += std::exp(logit[j] - m);
    lse_out[r] = m + std::log(z);
  });
  return 0;
}

/* Size of every KV head's keep-set: sinks [0, min(s,S)), window
 * [max(0, S-w), S) and min(k, |eligible|) winners from [s, S-w). */
int64_t oracle_keep_count(int64_t S, int64_t window, int64_t n_sink, int64_t top_k) {
  if (S < 0 || window < 0 || n_sink < 0 || top_k < 0) return -1;
  std::vector<char> kept(static_cast<size_t>(S), 0);
  for (int64_t j = 0; j < S; ++j) {
    if (j < n_sink) kept[j] = 1;
    if (j >= S - window) kept[j] = 1;
  }
  int64_t eligible = 0;
  for (int64_t j = n_sink; j < S - window; ++j) ++eligible;
  int64_t n = std::min(top_k, eligible);
  for (int64_t j = 0; j < S; ++j) n += kept[j];
  return n;
}

/* Keep-set of every (b, KV head): ascending indices, n_keep per head.
 * Eligible tokens are ordered by (mass descending, index ascending) with a
 * full sort; the first min(k, |eligible|) are kept. */
int oracle_select(const double* mass, int64_t B, int64_t Hkv, int64_t S, int64_t window,
                  int64_t n_sink, int64_t top_k, int32_t* keep) {
  if (B < 0 || Hkv < 1 || S < 0 || window < 0 || n_sink < 0 || top_k < 0) return 1;
  if (S > 0 && B > 0 && (!mass || !keep)) return 1;
  const int64_t n_keep = oracle_keep_count(S, window, n_sink, top_k);
  for (int64_t bh = 0; bh < B * Hkv; ++bh) {
    const double* m = mass + bh * S;
    std::vector<char> kept(static_cast<size_t>(S), 0);
    for (int64_t j = 0; j < std::min(n_sink, S); ++j) kept[j] = 1;
    for (int64_t j = std::max<int64_t>(0, S - window); j < S; ++j) kept[j] = 1;
    std::vector<std::pair<double, int64_t>> elig;
    for (int64_t j = n_sink; j < S - window; ++j) elig.emplace_back(m[j], j);
    std::sort(elig.begin(), elig.end(), [](const std::pair<double, int64_t>& a,
                                           const std::pair<double, int64_t>& b) {
      if (a.first != b.first) return a.first > b.first;
      return a.second < b.second;
    });
    const int64_t take = std::min<int64_t>(top_k, static_cast<int64_t>(elig.size()));
    for (int64_t r = 0; r < take; ++r) kept[elig[r].second] = 1;
    int64_t w = 0;
    for (int64_t j = 0; j < S; ++j)
      if (kept[j]) {
        if (w >= n_keep) return 2;
        keep[bh * n_keep + w++] = static_cast<int32_t>(j);
      }
    if (w != n_keep) return 2;
  }
  return 0;
}

/* Running top-k cutoff of [KVpop] §3.2 ("Running top-k sparse attention"),
 * per (b, KV head) row of static priorities score[b,h,:]:
 *   1. sort the tokens t in [s, S) once by priority (descending; equal
 *      priorities by ascending index) and give each its rank (0 = best);
 *      tokens t < s (sinks) get rank -1;
 *   2. for q = 0 .. S-1 the token t = q - w becomes eligible (Eq. 4,
 *      E(q) = {s <= t <= q - w}); its rank is inserted into a Fenwick tree
 *      over ranks, and the rank of the k-th best eligible token is found by
 *      binary lifting: cutoff[q].  With fewer than k eligible tokens every
 *      eligible token is retained and cutoff[q] = S; with k = 0 none is and
 *      cutoff[q] = -1.
 * At query q an eligible token t is retained iff rank[t] <= cutoff[q].
 * Returns 0, or 1 on invalid arguments. */
int oracle_running_cutoff(const double* score, int64_t B, int64_t Hkv, int64_t S, int64_t window,
                          int64_t n_sink, int64_t top_k, int32_t* rank, int32_t* cutoff) {
  if (B < 0 || Hkv < 1 || S < 0 || window < 0 || n_sink < 0 || top_k < 0) return 1;
  if (S > 0 && B > 0 && (!score || !rank || !cutoff)) return 1;
  const int64_t s = std::min(n_sink, S);
  const int64_t n = S - s;  // rankable tokens
  for (int64_t bh = 0; bh < B * Hkv; ++bh) {
    const double* m = score + bh * S;
    int32_t* rk = rank + bh * S;
    int32_t* cut = cutoff + bh * S;
    std::vector<int64_t> order;
    for (int64_t t = s; t < S; ++t) order.push_back(t);
    std::sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
      if (m[a] != m[b]) return m[a] > m[b];
      return a < b;
    });
    for (int64_t t = 0; t < s; ++t) rk[t] = -1;
    for (int64_t r = 0; r < n; ++r) rk[order[r]] = static_cast<int32_t>(r);
    // Fenwick tree over ranks 1..n (rank r stored at index r + 1)
    std::vector<int64_t> tree(static_cast<size_t>(n + 1), 0);
    int64_t top = 1;
    while (top * 2 <= n) top *= 2;
    int64_t eligible = 0;
    for (int64_t q = 0; q < S; ++q) {
      const int64_t t = q - window;
      if (t >= s) {
        for (int64_t i = rk[t] + 1; i <= n; i += i & -i) tree[i] += 1;
        ++eligible;
      }
      if (top_k == 0) {  // no long-range token is retained
        cut[q] = -1;
        continue;
      }
      if (eligible < top_k) {  // every eligible token is retained
        cut[q] = static_cast<int32_t>(S);
        continue;
      }
      // binary lifting: largest position p with prefix(p) < k; rank p is the k-th
      int64_t pos = 0, acc = 0;
      for (int64_t step = top; step > 0; step /= 2) {
        if (pos + step <= n && acc + tree[pos + step] < top_k) {
          pos += step;
          acc += tree[pos];
        }
      }
      cut[q] = static_cast<int32_t>(pos);  // the k-th best eligible token has rank pos
    }
  }
  return 0;
}

/* Log-normaliser of the running top-k sparse attention ([KVpop] §3.2: the
 * student's sparse attention keeps, at query q, the sinks, the protected
 * window and the eligible tokens of rank at most the cutoff tau_q; its
 * per-query log-normalisers stand in for the dense ones in the target):
 *   lse[b,g,i] = ln sum_{j in K(i)} exp(l_g(i,j)),
 *   K(i) = { j <= i : i - j < window  or  rank[b,h,j] <= cutoff[b,h,i] }
 * with rank / cutoff as oracle_running_cutoff writes them (rank -1 for the
 * sinks, so they are always kept; cutoff S keeps every eligible token, -1
 * none).  An empty K(i) gives -inf.  Returns 0, or 1 on invalid arguments. */
int oracle_sparse_lse(const void* q, const void* k, int dtype, int64_t B, int64_t Hq, int64_t Hkv,
                      int64_t S, int64_t D, double scale, int64_t window, const int32_t* rank,
                      const int32_t* cutoff, int nthreads, double* lse) {
  if (!q || !k || !rank || !cutoff || !lse || B < 0 || Hq < 1 || Hkv < 1 || S < 0 || D < 1 ||
      Hq % Hkv != 0 || window < 0 || dtype < 0 || dtype > 2)
    return 1;
  if (!(scale > 0.0)) scale = 1.0 / std::sqrt(static_cast<double>(D));
  const int64_t G = Hq / Hkv;
  parallel_items(B * Hq, nthreads, [&](int64_t item) {
    const int64_t b = item / Hq, g = item % Hq, h = g / G;
    std::vector<double> qg, kh;
    widen_head(q, dtype, (b * Hq + g) * S * D, S, D, qg);
    widen_head(k, dtype, (b * Hkv + h) * S * D, S, D, kh);
    const int32_t* rk = rank + (b * Hkv + h) * S;
    const int32_t* cut = cutoff + (b * Hkv + h) * S;
    std::vector<double> logit(static_cast<size_t>(S > 0 ? S : 1));
    for (int64_t i = 0; i < S; ++i) {
      double m = -INFINITY;
      for (int64_t j = 0; j <= i; ++j) {
        const bool keep = (i - j < window) || (rk[j] <= cut[i]);
        if (!keep) continue;
        double dot = 0.0;
        for (int64_t c = 0; c < D; ++c) dot += qg[i * D + c] * kh[j * D + c];
        logit[j] = scale * dot;
        m = std::max(m, logit[j]);
      }
      double z = 0.0;
      for (int64_t j = 0; j <= i; ++j) {
        const bool keep = (i - j < window) || (rk[j] <= cut[i]);
        if (keep) z += std::exp(logit[j] - m);
      }
      lse[(b * Hq + g) * S + i] = z > 0.0 ? m + std::log(z) : -INFINITY;
    }
  });
  return 0;
}

/* ForesightKV Golden-Eviction block scores and future scores ("ForesightKV:
 * Optimizing KV Cache Eviction for Reasoning Models by Learning Long-Term
 * Contribution", §3.2 "Golden Eviction" and the appendix's block-level
 * surrogate; the introduction states the future score as the maximum of the
 * block scores of future steps).
 *
 * Query blocks: block t holds the query rows [block_start + t*block_len,
 * block_start + (t+1)*block_len) clipped to S; rows below block_start belong
 * to no block.  n_blocks = ceil((S - block_start) / block_len) (0 if
 * S <= block_start).
 *   block[b,u,t,j]  = mean over the query heads g of unit u and the rows i of
 *                     block t of p_g(i->j), counting only i >= j + window;
 *                     unit u is a KV head (its G query heads; per_head = 0)
 *                     or a single query head (per_head = 1)
 *   future[b,u,t,j] = max over t' >= t of block[b,u,t',j]
 * Either output may be NULL.  Returns 0, or 1 on invalid arguments. */
int oracle_block_scores(const void* q, const void* k, int dtype, int64_t B, int64_t Hq,
                        int64_t Hkv, int64_t S, int64_t D, double scale, int64_t window,
                        int64_t block_start, int64_t block_len, int per_head, int nthreads,
                        double* block, double* future) {
  if (!q || !k || B < 0 || Hq < 1 || Hkv < 1 || S < 0 || D < 1 || Hq % Hkv != 0 ||
      window < 0 || dtype < 0 || dtype > 2 || block_start < 0 || block_len < 1 ||
      (per_head != 0 && per_head != 1))
    return 1;
  if (!(scale > 0.0)) scale = 1.0 / std::sqrt(static_cast<double>(D));
  const int64_t G = Hq / Hkv;
  const int64_t n_blocks = S > block_start ? (S - block_start + block_len - 1) / block_len : 0;
  const int64_t n_units = per_head ? Hq : Hkv;
  const int64_t heads_per_unit = per_head ? 1 : G;

  for (int64_t b = 0; b < B; ++b) {
    for (int64_t h = 0; h < Hkv; ++h) {
      std::vector<double> kh, kt;
      widen_head(k, dtype, (b * Hkv + h) * S * D, S, D, kh);
      transpose_head(kh, S, D, kt);
      // column sums of every (query head of the group, block): one item each
      const int64_t n_items = G * n_blocks;
      std::vector<std::vector<double>> colsum(static_cast<size_t>(n_items));
      parallel_items(n_items, nthreads, [&](int64_t item) {
        const int64_t gg = item / n_blocks;
        const int64_t t = item % n_blocks;
        const int64_t g = h * G + gg;
        std::vector<double> qg;
        widen_head(q, dtype, (b * Hq + g) * S * D, S, D, qg);
        std::vector<double>& col = colsum[item];
        col.assign(static_cast<size_t>(S), 0.0);
        std::vector<double> p(static_cast<size_t>(S));
        const int64_t i0 = block_start + t * block_len;
        const int64_t i1 = std::min(S, i0 + block_len);
        for (int64_t i = i0; i < i1; ++i) {
          softmax_row(qg.data() + i * D, kt.data(), S, D, i, scale, p);
          for (int64_t j = 0; j + window <= i; ++j) col[j] += p[j];
        }
      });
      for (int64_t gg0 = 0; gg0 < G; gg0 += heads_per_unit) {
        const int64_t u = per_head ? h * G + gg0 : h;
        for (int64_t t = n_blocks - 1; t >= 0; --t) {
          const int64_t i0 = block_start + t * block_len;
          const double rows = static_cast<double>(std::min(S, i0 + block_len) - i0);
          const int64_t o = ((b * n_units + u) * n_blocks + t) * S;
          for (int64_t j = 0; j < S; ++j) {
            double acc = 0.0;
            for (int64_t gg = gg0; gg < gg0 + heads_per_unit; ++gg) acc += colsum[gg * n_blocks + t][j];
            const double mean = acc / (rows * static_cast<double>(heads_per_unit));
            if (block) block[o + j] = mean;
            if (future) {
              const double later = t + 1 < n_blocks ? future[o + S + j] : -INFINITY;
              future[o + j] = std::max(mean, later);
            }
          }
        }
      }
    }
  }
  return 0;
}

}  // extern "C"
