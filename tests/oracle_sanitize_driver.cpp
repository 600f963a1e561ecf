// Host-only driver that runs every C entry point of the CPU oracle on small
// shapes, including the degenerate ones (one token, a window longer than the
// sequence, no sinks, k = 0 and k beyond the eligible count, several threads).
// The test that compiles it links the oracle source with AddressSanitizer and
// UndefinedBehaviorSanitizer, so an out-of-bounds access, a use after free or
// undefined arithmetic anywhere in the oracle aborts the run.  It also checks
// the return codes and two identities (softmax rows sum to one; the keep-set
// size), so a sanitizer build that computes nonsense does not pass silently.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

extern "C" {
int oracle_round_bf16(const float* x, int64_t n, uint16_t* out);
int oracle_future_mass(const void* q, const void* k, int dtype, int64_t B, int64_t Hq,
                       int64_t Hkv, int64_t S, int64_t D, double scale, int64_t window,
                       int64_t b_only, int64_t h_only, int64_t row_lo, int nthreads, double* lse,
                       double* mass, double* rowsum, double* winmass, double* mass_heads);
int oracle_lse_rows(const void* q, const void* k, int dtype, int64_t B, int64_t Hq, int64_t Hkv,
                    int64_t S, int64_t D, double scale, const int64_t* rows, int64_t n_rows,
                    int nthreads, double* lse_out);
int64_t oracle_keep_count(int64_t S, int64_t window, int64_t n_sink, int64_t top_k);
int oracle_select(const double* mass, int64_t B, int64_t Hkv, int64_t S, int64_t window,
                  int64_t n_sink, int64_t top_k, int32_t* keep);
int oracle_running_cutoff(const double* score, int64_t B, int64_t Hkv, int64_t S, int64_t window,
                          int64_t n_sink, int64_t top_k, int32_t* rank, int32_t* cutoff);
int oracle_sparse_lse(const void* q, const void* k, int dtype, int64_t B, int64_t Hq, int64_t Hkv,
                      int64_t S, int64_t D, double scale, int64_t window, const int32_t* rank,
                      const int32_t* cutoff, int nthreads, double* lse);
int oracle_block_scores(const void* q, const void* k, int dtype, int64_t B, int64_t Hq,
                        int64_t Hkv, int64_t S, int64_t D, double scale, int64_t window,
                        int64_t block_start, int64_t block_len, int per_head, int nthreads,
                        double* block, double* future);
}

static int failures = 0;

static void expect(bool ok, const char* what, int64_t S) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s (S=%lld)\n", what, static_cast<long long>(S));
    ++failures;
  }
}

struct Case {
  int64_t B, Hq, Hkv, S, D, w, s, k, block_start, block_len;
};

static void run_case(const Case& c, int dtype, int nthreads, std::mt19937_64& rng) {
  std::normal_distribution<float> nd(0.f, 1.f);
  const int64_t nq = c.B * c.Hq * c.S * c.D, nk = c.B * c.Hkv * c.S * c.D;
  std::vector<float> qf(static_cast<size_t>(nq)), kf(static_cast<size_t>(nk));
  for (auto& x : qf) x = nd(rng);
  for (auto& x : kf) x = nd(rng);
  std::vector<uint16_t> qb(qf.size()), kb(kf.size());
  expect(oracle_round_bf16(qf.data(), nq, qb.data()) == 0, "round q", c.S);
  expect(oracle_round_bf16(kf.data(), nk, kb.data()) == 0, "round k", c.S);
  const void* q = dtype == 0 ? static_cast<const void*>(qb.data()) : qf.data();
  const void* k = dtype == 0 ? static_cast<const void*>(kb.data()) : kf.data();

  const int64_t rows_q = c.B * c.Hq * c.S, rows_kv = c.B * c.Hkv * c.S;
  std::vector<double> lse(rows_q), mass(rows_kv), rowsum(rows_q), win(rows_q), heads(rows_q);
  expect(oracle_future_mass(q, k, dtype, c.B, c.Hq, c.Hkv, c.S, c.D, 0.0, c.w, -1, -1, 0,
                            nthreads, lse.data(), mass.data(), rowsum.data(), win.data(),
                            heads.data()) == 0,
         "future_mass", c.S);
  for (double r : rowsum) expect(std::fabs(r - 1.0) < 1e-12, "row sums to one", c.S);
  // restricted to one unit and the tail rows
  expect(oracle_future_mass(q, k, dtype, c.B, c.Hq, c.Hkv, c.S, c.D, 0.0, c.w, c.B - 1,
                            c.Hkv - 1, c.S / 2, nthreads, lse.data(), mass.data(), nullptr,
                            nullptr, nullptr) == 0,
         "future_mass restricted", c.S);

  std::vector<int64_t> rows;
  for (int64_t r = 0; r < 5 && c.S > 0; ++r) {
    rows.push_back(static_cast<int64_t>(rng() % c.B));
    rows.push_back(static_cast<int64_t>(rng() % c.Hq));
    rows.push_back(static_cast<int64_t>(rng() % c.S));
  }
  std::vector<double> lse_r(rows.size() / 3 + 1);
  expect(oracle_lse_rows(q, k, dtype, c.B, c.Hq, c.Hkv, c.S, c.D, 0.0, rows.data(),
                         static_cast<int64_t>(rows.size() / 3), nthreads, lse_r.data()) == 0,
         "lse_rows", c.S);

  const int64_t n_keep = oracle_keep_count(c.S, c.w, c.s, c.k);
  expect(n_keep >= 0 && n_keep <= c.S, "keep count in range", c.S);
  std::vector<int32_t> keep(static_cast<size_t>(c.B * c.Hkv * n_keep + 1));
  expect(oracle_select(mass.data(), c.B, c.Hkv, c.S, c.w, c.s, c.k, keep.data()) == 0, "select",
         c.S);
  for (int64_t u = 0; u < c.B * c.Hkv; ++u)
    for (int64_t t = 1; t < n_keep; ++t)
      expect(keep[u * n_keep + t - 1] < keep[u * n_keep + t], "keep ascending", c.S);

  std::vector<int32_t> rank(rows_kv + 1), cut(rows_kv + 1);
  expect(oracle_running_cutoff(mass.data(), c.B, c.Hkv, c.S, c.w, c.s, c.k, rank.data(),
                               cut.data()) == 0,
         "running_cutoff", c.S);
  std::vector<double> lse_sp(rows_q + 1);
  expect(oracle_sparse_lse(q, k, dtype, c.B, c.Hq, c.Hkv, c.S, c.D, 0.0, c.w, rank.data(),
                           cut.data(), nthreads, lse_sp.data()) == 0,
         "sparse_lse", c.S);

  const int64_t nb =
      c.S > c.block_start ? (c.S - c.block_start + c.block_len - 1) / c.block_len : 0;
  for (int per_head = 0; per_head <= 1; ++per_head) {
    const int64_t units = per_head ? c.Hq : c.Hkv;
    std::vector<double> blk(static_cast<size_t>(c.B * units * nb * c.S + 1));
    std::vector<double> fut(blk.size());
    expect(oracle_block_scores(q, k, dtype, c.B, c.Hq, c.Hkv, c.S, c.D, 0.0, c.w, c.block_start,
                               c.block_len, per_head, nthreads, blk.data(), fut.data()) == 0,
           "block_scores", c.S);
  }
}

int main() {
  std::mt19937_64 rng(20261203);
  const Case cases[] = {
      {1, 1, 1, 1, 64, 0, 0, 1, 0, 32},        // one token
      {2, 4, 2, 37, 16, 5, 2, 7, 8, 8},        // ragged, batch 2
      {1, 4, 1, 50, 8, 60, 4, 10, 0, 64},      // window beyond the sequence
      {1, 2, 2, 41, 8, 0, 0, 0, 40, 1},        // w = 0, no sinks, k = 0
      {1, 6, 3, 33, 12, 3, 40, 100, 1, 5},     // sinks beyond S - w, k beyond eligible
  };
  for (const Case& c : cases)
    for (int dtype = 0; dtype <= 2; ++dtype)
      for (int nthreads : {1, 4}) run_case(c, dtype, nthreads, rng);
  // invalid arguments are rejected, not dereferenced
  expect(oracle_future_mass(nullptr, nullptr, 0, 1, 1, 1, 4, 8, 0.0, 0, -1, -1, 0, 1, nullptr,
                            nullptr, nullptr, nullptr, nullptr) == 1,
         "null inputs rejected", 4);
  expect(oracle_select(nullptr, 1, 1, 4, 0, 0, 1, nullptr) == 1, "null select rejected", 4);
  std::printf("oracle sanitizer driver: %s\n", failures ? "FAILED" : "ok");
  return failures ? 1 : 0;
}
