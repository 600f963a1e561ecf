/*
 * kvp.h — C ABI of the future-attention-mass library (libkvp.so), AMD
 * Instinct MI355X (gfx950).
 *
 * Three entry points compute the hot path of KVpop-style KV-cache eviction
 * scoring for one attention layer, from its post-RoPE queries Q and keys K:
 *
 *   kvp_lse_fwd      per-query log-sum-exp of the dense causal attention row;
 *   kvp_future_mass  future-attention mass of every key, summed over the query
 *                    heads of its GQA group, without an S x S map;
 *   kvp_select_topk  per-KV-head keep-set: sinks, recent window and the top-k
 *                    older tokens by mass.
 *
 * kvp_future_mass_chunked computes the same masses with a caller workspace,
 * which lets short sequences spread each key tile's queries over several
 * workgroups.
 *
 * Two more turn the masses into KVpop's training target:
 *
 *   kvp_future_mass_per_head  the future mass of every key for each query head
 *                             on its own (no group sum);
 *   kvp_target_scores         count normalisation, log(eps + m), aggregation
 *                             over the group and the temporal decay.
 *
 * And one gives the keep-set of every query position rather than only the
 * last one, with the normaliser of the attention that keeps it:
 *
 *   kvp_running_cutoff        static ranks and the per-query cutoff rank of
 *                             the running top-k (the sparse mask predicate);
 *   kvp_lse_sparse            the per-query LSE over that sparse pattern.
 *
 * A query-block variant of the transposed pass gives ForesightKV's labels:
 *
 *   kvp_block_future_scores   Golden-Eviction block scores (attention pooled
 *                             over the rows of each query block and the heads
 *                             of a group) and future scores (their maximum
 *                             over the current and later blocks).
 *
 * And a differentiable stand-in for the top-k selection:
 *
 *   kvp_soft_topk_fwd / _bwd  LKV's Soft-TopK soft mask (closed-form
 *                             threshold) and its gradients.
 *
 * Sources, cited by page title and section/equation:
 *   [KVpop] "KVpop — Key-Value Cache Compression with Predictive Online
 *           Pruning" (arXiv 2607.05061);
 *   [LKV]   "LKV: End-to-End Learning of Head-wise Budgets and Token
 *           Selection for LLM KV Cache Eviction" (arXiv 2605.06676);
 *   [Tut]   the "transformer math" KV-compression tutorial (aicassindra),
 *           sections "H2O: evict by accumulated attention" and
 *           "StreamingLLM and the attention-sink surprise";
 *   [FKV]   "ForesightKV: Optimizing KV Cache Eviction for Reasoning Models by
 *           Learning Long-Term Contribution" (arXiv 2602.03203).
 *
 * Common conventions
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises device memory; every call only
 *     enqueues kernels on `stream` (NULL = the default stream) and returns.
 *     Results are valid once the caller has synchronised that stream.
 *   - Layouts are dense row-major: Q [B, Hq, S, d], K [B, Hkv, S, d] (d
 *     fastest), LSE [B, Hq, S], mass [B, Hkv, S], keep [B, Hkv, n_keep].
 *   - GQA: query head g reads KV head g / G, G = Hq / Hkv (contiguous groups;
 *     [LKV] §3 "Problem Formulation": one retention mask per KV head, shared
 *     by the query heads of its group).
 *   - Logits are l(i, j) = scale * <q_i, k_j> with scale = 1/sqrt(d) when the
 *     `scale` argument is <= 0 ([LKV] §3 Eq. 1).
 *   - bf16 inputs are multiplied exactly and accumulated in fp32 on the
 *     matrix cores.  fp32 inputs are used as given: their logits are fp32
 *     dot products on the vector ALUs (fused multiply-adds), for callers who
 *     need the fp32 problem exactly rather than the matrix cores' speed.
 *   - Validation is synchronous and happens before any launch; a rejected
 *     call enqueues nothing.  No function prints, throws or aborts, and all
 *     are thread-safe; only kvp_select_topk_noalloc keeps state (its
 *     per-GPU device array, see there).
 *   - Sizes: batch >= 0 and 0 <= seq_len <= 2^22 (0 = empty input: nothing
 *     to do, KVP_OK; longer sequences give KVP_EUNSUPPORTED);
 *     n_q_heads, n_kv_heads >= 1 and n_q_heads % n_kv_heads == 0; head_dim
 *     in {64, 128}.  Pointers must be 16-byte aligned.
 */
#ifndef KVP_H_
#define KVP_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVP_OK = 0,
  KVP_EINVAL = 1,        /* null/misaligned pointer, negative size, Hq % Hkv != 0, ... */
  KVP_EUNSUPPORTED = 2,  /* head_dim not in {64, 128}, unknown dtype, size beyond limits */
  KVP_EWORKSPACE = 3,    /* workspace too small */
  KVP_EHIP = 4           /* a kernel launch failed (hipGetLastError) */
} kvp_status_t;

typedef enum { KVP_BF16 = 0, KVP_F32 = 1 } kvp_dtype_t;

typedef struct {
  int32_t batch;       /* B  */
  int32_t n_q_heads;   /* Hq */
  int32_t n_kv_heads;  /* Hkv */
  int32_t seq_len;     /* S  */
  int32_t head_dim;    /* d  */
} kvp_dims_t;

/* Stage 1 — causal log-sum-exp.
 *   lse[b, g, i] = ln sum_{j <= i} exp(scale * <q[b,g,i], k[b, g/G, j]>)
 * The dense causal normaliser of each query row: the per-query
 * log-normaliser that [KVpop] §3.2 (Eq. 8) reuses to recover attention
 * probabilities, computed here for the dense causal softmax of [LKV] §3 Eq. 1
 * (keys j <= i, diagonal included).  Natural log.
 *   q, k  : device, dtype `dtype`, layouts above.
 *   lse   : device fp32 [B, Hq, S], written entirely.
 * Rows whose logits span more than the fp32 exponent range are recomputed by
 * an exact per-row fallback, so every finite input yields a finite LSE. */
kvp_status_t kvp_lse_fwd(const void* q, const void* k, kvp_dtype_t dtype, kvp_dims_t dims,
                         float scale, float* lse, hipStream_t stream);

/* Stage 1, sparse — the log-normaliser of the running top-k sparse attention
 * ([KVpop] §3.2: the student's sparse attention keeps, at query q, the sink
 * tokens, the protected window and the top-k eligible tokens, and the
 * per-query log-normalisers it returns stand in for the dense ones in the
 * target; pass the result to kvp_future_mass in place of kvp_lse_fwd's):
 *   lse[b,g,i] = ln sum_{j in K(i)} exp(scale * <q[b,g,i], k[b,g/G,j]>),
 *   K(i) = { j <= i : i - j < window  or  rank[b,h,j] <= cutoff[b,h,i] }.
 *   rank, cutoff : device int32 [B, Hkv, S] as written by kvp_running_cutoff
 *                  with the same window (sinks have rank -1 and are always
 *                  kept; cutoff S keeps every eligible token, -1 none).
 *   lse          : device fp32 [B, Hq, S], natural log; -inf for an empty K(i)
 *                  (window 0, no sinks and no budget).
 * The same MFMA pass as kvp_lse_fwd with the pattern tested per (query, key)
 * pair; rows whose sum leaves the fp32 range are recomputed exactly. */
kvp_status_t kvp_lse_sparse(const void* q, const void* k, kvp_dtype_t dtype, kvp_dims_t dims,
                            float scale, const int32_t* rank, const int32_t* cutoff, int32_t window,
                            float* lse, hipStream_t stream);

/* Stage 2 — transposed future-attention-mass pass.
 *   mass[b, h, j] = sum_{g : g/G = h} sum_{i = j + window}^{S-1}
 *                     exp(scale * <q[b,g,i], k[b,h,j]> - lse[b,g,i])
 * [KVpop] §3.1 Eq. 2 in the un-normalised form of App. B.1 (no 1/N_t),
 * recovered from the LSE as in §3.2 Eq. 8, and summed over the G query heads
 * of the group (App. B.1 averages; the sum ranks identically).  Query i
 * counts for key j iff i >= j + window; mass[j] = 0 for j >= S - window.
 * With window = 0 this is H2O accumulated attention ([Tut], "H2O").
 *   lse    : device fp32 [B, Hq, S] as written by kvp_lse_fwd (natural log).
 *   window : w >= 0.
 *   mass   : device fp32 [B, Hkv, S], written entirely.
 * Each key is owned by one workgroup, which reduces over all its future
 * queries on chip and writes it once.  When the grid is too small to fill the
 * GPU (short sequences), each group's heads are split over two workgroups
 * that add into the output after a zero fill: two terms, so the sum does not
 * depend on their order.  Either way the result is bitwise reproducible. */
kvp_status_t kvp_future_mass(const void* q, const void* k, const float* lse, kvp_dtype_t dtype,
                             kvp_dims_t dims, float scale, int32_t window, float* mass,
                             hipStream_t stream);

/* Stage 2, per query head.
 *   mass[b, g, j] = sum_{i = j + window}^{S-1} exp(scale * <q[b,g,i], k[b,g/G,j]> - lse[b,g,i])
 * The same pass as kvp_future_mass without the sum over the group: the
 * un-normalised per-head mass m^(h,g) of [KVpop] §3.1 Eq. 2 / App. B.1, the
 * input of the per-head aggregation of Eq. 3.  Arguments as kvp_future_mass
 * except mass: device fp32 [B, Hq, S], written entirely. */
kvp_status_t kvp_future_mass_per_head(const void* q, const void* k, const float* lse,
                                      kvp_dtype_t dtype, kvp_dims_t dims, float scale,
                                      int32_t window, float* mass, hipStream_t stream);

/* Stage 2 with a caller workspace, for short sequences.
 * The same masses as kvp_future_mass (per_head = 0, mass [B, Hkv, S]) or
 * kvp_future_mass_per_head (per_head = 1, mass [B, Hq, S]), same definition
 * ([KVpop] §3.1 Eq. 2 / App. B.1, recovered from the LSE as in §3.2 Eq. 8).
 * Where the one-tile-per-workgroup launch would leave compute units idle,
 * each key tile's sweep over its future queries is cut into chunks of equal
 * length, one workgroup each; the chunks' partial masses go to the workspace
 * and a second kernel adds them per key in chunk order.  The result is
 * bitwise reproducible; it can differ from kvp_future_mass's in the last bits
 * (another order of the same sum).
 *   workspace : device memory of at least kvp_future_mass_workspace_bytes(
 *               dims, dtype, window, per_head) bytes, 256-byte aligned, owned
 *               by the caller, clobbered; may be null when that size is 0
 *               (long sequences, fp32 input and per-head masses, whose grid
 *               already has G times the units: the call then runs the
 *               kvp_future_mass / kvp_future_mass_per_head launch).
 * Errors as kvp_future_mass; per_head not 0 or 1 -> KVP_EINVAL;
 * workspace_bytes below the size -> KVP_EWORKSPACE; a null or misaligned
 * workspace where the size is not 0 -> KVP_EINVAL. */
size_t kvp_future_mass_workspace_bytes(kvp_dims_t dims, kvp_dtype_t dtype, int32_t window,
                                       int32_t per_head);
kvp_status_t kvp_future_mass_chunked(const void* q, const void* k, const float* lse,
                                     kvp_dtype_t dtype, kvp_dims_t dims, float scale,
                                     int32_t window, int32_t per_head, float* mass, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* Aggregation of the per-head log masses over the query heads of a group
 * ([KVpop] §3.1 Eq. 3 leaves Agg open; App. B.1 uses the log of the mean). */
typedef enum {
  KVP_AGG_LOG_MEAN = 0,  /* log(eps + (1/G) sum_g m_g)      App. B.1            */
  KVP_AGG_MEAN_LOG = 1,  /* (1/G) sum_g log(eps + m_g)      Eq. 3, Agg = mean   */
  KVP_AGG_MAX_LOG = 2    /* max_g log(eps + m_g)            Eq. 3, Agg = max    */
} kvp_agg_t;

/* KVpop target scores ([KVpop] §3.1 Eq. 2-3, App. B.1-B.3), one per key:
 *   m_g[t]  = mass[b, g, t] / N_t (per_head = 1) or the group sum / G
 *             (per_head = 0, only with KVP_AGG_LOG_MEAN), where
 *             N_t = max(1, S - (t + window)) if normalize (Eq. 2 / B.2), else 1;
 *   r[t]    = Agg_g log(eps + m_g[t])                    (Eq. 3 / B.1);
 *   with query >= 0 the decayed score of App. B.3 at query position q:
 *   r(q)[t] = r[t] + floor((q - t) / decay_step) * log_gamma[h]  for t <= q,
 *             -inf for t > q (not yet generated).
 *   mass      : device fp32 [B, Hq, S] (per_head = 1) or [B, Hkv, S] (0), as
 *               written by kvp_future_mass_per_head / kvp_future_mass.
 *   eps       : >= 0 (eps = 0 gives -inf for zero mass).
 *   query     : < 0 for no decay; else decay_step >= 1 and log_gamma is a
 *               device fp32 [Hkv] array of log(gamma_h) (gamma_h in (0, 1)).
 *   score     : device fp32 [B, Hkv, S], written entirely.
 *   dims      : head_dim is not read.
 * Natural logs in fp32.  The scores can be passed to kvp_select_topk. */
kvp_status_t kvp_target_scores(const float* mass, int32_t per_head, kvp_dims_t dims, int32_t window,
                               int32_t normalize, kvp_agg_t agg, float eps, int32_t query,
                               int32_t decay_step, const float* log_gamma, float* score,
                               hipStream_t stream);

/* Static token priorities of the running top-k ([KVpop] §3.2 "Running top-k
 * sparse attention": tokens are sorted once by a static priority because the
 * query-dependent part of the decayed score is shared across eligible tokens
 * up to the decay-step discretization; App. B.3 "Temporal Decay and Static
 * Priorities"):
 *   priority[b, h, t] = score[b, h, t] - floor(t / decay_step) * log_gamma[h]
 * At query q, App. B.3's decayed score score[t] + floor((q - t) / n) log_gamma
 * equals priority[t] + floor(q / n) log_gamma (shared by every token) plus at
 * most one step |log_gamma| for tokens with t mod n > q mod n; the order is
 * exact for n = 1 and at every q with q mod n = n - 1.  Pass the result to
 * kvp_running_cutoff.
 *   score     : device fp32 [B, Hkv, S] undecayed scores (e.g. kvp_target_scores
 *               with query < 0); priority may alias it (computed in place).
 *   log_gamma : device fp32 [Hkv], log(gamma_h) with gamma_h in (0, 1].
 *   decay_step: n >= 1.   dims: batch, n_kv_heads and seq_len are read.
 * One fp32 fused multiply-add per token (correctly rounded). */
kvp_status_t kvp_static_priority(const float* score, kvp_dims_t dims, int32_t decay_step,
                                 const float* log_gamma, float* priority, hipStream_t stream);

/* Size of every KV head's keep-set ([KVpop] §3 Eq. 1, budget B = s + w + k,
 * clipped to the sequence):
 *   min(s, S) + |[max(s, S - w), S)| + min(k, max(0, S - w - s)).
 * Pure host function; returns -1 for negative arguments. */
int64_t kvp_keep_count(int64_t seq_len, int64_t window, int64_t n_sink, int64_t top_k);

/* Stage 3 — per-KV-head keep-set.
 *   keep[b, h, :] = ascending( [0, min(s, S))                       sinks
 *                            U [max(0, S - w), S)                  window
 *                            U top-k of { mass[b,h,j] : s <= j < S - w } )
 * [KVpop] Fig. 1 (sinks and the protected window are always retained, the
 * remaining budget goes to the top-k long-range tokens), Eq. 1 (budget) and
 * Eq. 4 (eligible set at the last query: s <= t <= S-1-w); the StreamingLLM
 * sink rule of [Tut].  Order: score descending, equal scores by ascending
 * index (lower index wins).  The scores are masses (kvp_future_mass) or any
 * fp32 scores of either sign, e.g. kvp_target_scores; -0 equals +0, -inf is
 * allowed, NaN gives an unspecified keep-set.  Selection compares exactly,
 * through an order-preserving integer key of every fp32 value.
 *   mass      : device fp32 [B, Hkv, S] scores (the batch dimension may also
 *               stack layers: any number of independent [Hkv, S] rows).
 *   keep      : device int32 [B, Hkv, kvp_keep_count(S, window, n_sink, top_k)].
 *   workspace : device scratch of at least kvp_select_workspace_bytes(dims,
 *               top_k) bytes, 256-byte aligned, owned by the caller (NULL
 *               allowed when that is 0); contents on entry and exit are
 *               unspecified.  KVP_EWORKSPACE if workspace_bytes is smaller.
 *   dims      : only batch, n_kv_heads and seq_len are read.
 * Rows of up to 32768 scores run one workgroup per row with no workspace;
 * longer rows are split over many workgroups (chunks of >= 4096 scores)
 * whose histograms, candidate keys and per-chunk counts live in the
 * workspace.  Integer counts only, so the result is exact and reproducible. */
kvp_status_t kvp_select_topk(const float* mass, kvp_dims_t dims, int32_t window, int32_t n_sink,
                             int32_t top_k, int32_t* keep, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* kvp_select_topk for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and results without the workspace, which instead is a
 * fixed device array inside the library of KVP_SELECT_NOALLOC_MAX_WORKSPACE
 * bytes (32 MiB), one copy per GPU, held until the process ends.  The call
 * allocates nothing (no hipMalloc / hipFree, no allocating library routine);
 * its first call on a GPU looks up that GPU's copy once.
 *   KVP_EWORKSPACE if kvp_select_workspace_bytes(dims, top_k) exceeds
 *   KVP_SELECT_NOALLOC_MAX_WORKSPACE (e.g. more than about 8M scores in all
 *   in rows longer than 32768); nothing is launched then.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on the same GPU (different streams or host threads without ordering)
 * race and give undefined keep-sets.  Calls ordered on one stream are safe:
 * no part of the array needs to start at zero, every region is written before
 * it is read in each call. */
#define KVP_SELECT_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)
kvp_status_t kvp_select_topk_noalloc(const float* mass, kvp_dims_t dims, int32_t window,
                                     int32_t n_sink, int32_t top_k, int32_t* keep,
                                     hipStream_t stream);

/* Bytes of device workspace kvp_select_topk needs for `dims` (batch,
 * n_kv_heads and seq_len are read) and `top_k`: 0 for rows of at most 32768
 * scores; otherwise, with R = batch * n_kv_heads rows split into c chunks
 * each, about R * (8 KiB * c + 4 * seq_len) (histograms and candidate keys).
 * Pure host function; 0 for invalid arguments. */
size_t kvp_select_workspace_bytes(kvp_dims_t dims, int32_t top_k);

/* Number of query blocks [block_start + t * block_len, block_start + (t+1) *
 * block_len) that intersect [0, seq_len): ceil((S - block_start) / block_len),
 * 0 if S <= block_start.  Pure host function; -1 for invalid arguments. */
int64_t kvp_block_count(int64_t seq_len, int64_t block_start, int64_t block_len);

/* Golden-Eviction block and future scores ([FKV] §3.2 "Golden Eviction": the
 * attention matrix pooled over the rows of each query block of length L
 * after the first B tokens and over the query heads of each group; the
 * appendix's block-level surrogate takes the mean over a block's queries;
 * the future score at eviction step t is the largest block score of the
 * steps from t on, [FKV] §1).  With p_g(i->j) = exp(scale <q_i,k_j> - lse_i):
 *   block[b,u,t,j]  = (1 / (G_u * |Q_t|)) sum_{g in u} sum_{i in Q_t, i >= j + window} p_g(i->j)
 *   future[b,u,t,j] = max_{t' >= t} block[b,u,t',j]
 * where Q_t = [block_start + t L, block_start + (t+1) L) clipped to S (the
 * last block may be shorter), t < kvp_block_count(S, block_start, L), and the
 * unit u is a KV head with its G query heads (per_head = 0, the head pool is
 * the mean) or a single query head (per_head = 1, G_u = 1).  Rows below
 * block_start belong to no block.  Entries of keys that are not yet in the
 * cache at step t (j >= block_start + t L) follow the same formula.
 *   q, k, lse : as kvp_future_mass (lse from kvp_lse_fwd).
 *   window    : >= 0 (0 in [FKV]; a query counts for a key iff i >= j + window).
 *   block_start, block_len : >= 0 and >= 1; multiples of 32 (else
 *               KVP_EUNSUPPORTED).
 *   block_scores  : device fp32 [B, U, n_blocks, S] or NULL (not written).
 *   future_scores : device fp32 [B, U, n_blocks, S], written entirely;
 *                   U = Hkv (per_head = 0) or Hq (per_head = 1).
 * The same transposed pass as kvp_future_mass with the column sums flushed at
 * every block boundary: no S x S map, no atomics, bitwise reproducible. */
kvp_status_t kvp_block_future_scores(const void* q, const void* k, const float* lse,
                                     kvp_dtype_t dtype, kvp_dims_t dims, float scale,
                                     int32_t window, int32_t per_head, int32_t block_start,
                                     int32_t block_len, float* block_scores, float* future_scores,
                                     hipStream_t stream);

/* LKV Soft-TopK forward ([LKV] §3.2 "The Differentiable Soft-TopK Operator",
 * App. A.1).  Per row r of n scores x, with z = x / tau:
 *   y[r,i] = f(z_i - lam[r]),  f(u) = 1 - e^{-u}/2 for u >= 0, e^{u}/2 for u < 0
 * (the Laplace CDF), lam[r] the threshold with sum_i y[r,i] = k[r]: the root
 * of S1 e^{2 lam} + 2 (k - m) e^{lam} - S2 = 0 for the split m of elements
 * above it (S1 = sum over them of e^{-z_i}, S2 = sum over the rest of e^{z_i}).
 * Outputs lie in (0, 1), sum to k, keep the order of x and do not change
 * when a constant is added to x; tau -> 0 tends to the hard top-k.  Gumbel
 * noise ([LKV] §3.4), if wanted, is added to x by the caller.
 *   x   : device fp32 [rows, n];  k : device fp32 [rows], budgets in (0, n)
 *         (k <= 0 gives y = 0, lam = +inf; k >= n gives y = 1, lam = -inf).
 *   tau : temperature > 0.
 *   y   : device fp32 [rows, n];  lam : device fp32 [rows] (units of z) or NULL.
 * No sort: rows of n <= 32768 bracket the split with an fp32 Newton search
 * and confirm it, and form the sums and y, in fp64; longer rows find it by
 * bisection on the scores' bit patterns (at most 32 fp64 reductions).  x
 * must be finite. */
kvp_status_t kvp_soft_topk_fwd(const float* x, int64_t rows, int32_t n, const float* k, float tau,
                               float* y, float* lam, hipStream_t stream);

/* Soft-TopK backward ([LKV] App. A.2): with f'(u) = e^{-|u|}/2, u_i = z_i - lam,
 * A = sum_i dy_i f'(u_i), B = sum_i f'(u_i):
 *   dx[r,j] = f'(u_j) (dy[r,j] - A / B) / tau,   dk[r] = A / B.
 *   x, lam : as passed to / returned by kvp_soft_topk_fwd;  dy : device fp32
 *   [rows, n];  dx : device fp32 [rows, n];  dk : device fp32 [rows] or NULL. */
kvp_status_t kvp_soft_topk_bwd(const float* x, const float* lam, const float* dy, int64_t rows,
                               int32_t n, float tau, float* dx, float* dk, hipStream_t stream);

/* Bytes of device workspace kvp_running_cutoff needs for `dims` (batch,
 * n_kv_heads and seq_len are read) and `n_sink`: 20 * B * Hkv * (S - min(s, S)).
 * Pure host function; 0 for invalid arguments. */
size_t kvp_running_cutoff_workspace_bytes(kvp_dims_t dims, int32_t n_sink);

/* Running top-k cutoff ([KVpop] §3.2 "Efficient Target Implementation", the
 * paragraphs on running top-k sparse attention and on its kernel; Appendix I).
 * Per (b, h) row of static priorities score[b, h, 0..S):
 *   rank[b, h, t]   = position of t in the order of { s <= t' < S } by
 *                     score descending, equal scores by ascending index
 *                     (0 = best); -1 for the sinks t < s;
 *   cutoff[b, h, q] = rank of the k-th best token of the eligible set
 *                     E(q) = { s <= t <= q - window } (Eq. 4), or
 *                     S  while |E(q)| < k (every eligible token is kept),
 *                     -1 if top_k = 0 (none is).
 * At query q the sparse attention mask keeps the sinks, the window
 * (q - window < t <= q) and the eligible tokens t with
 * rank[b, h, t] <= cutoff[b, h, q]; at q = S - 1 this is exactly the
 * keep-set of kvp_select_topk.  Scores, their comparison and the signed-zero
 * / -inf / NaN rules are those of kvp_select_topk.
 *   score     : device fp32 [B, Hkv, S] (batch may stack layers).
 *   rank      : device int32 [B, Hkv, S], written entirely.
 *   cutoff    : device int32 [B, Hkv, S], written entirely.
 *   workspace : device scratch of at least
 *               kvp_running_cutoff_workspace_bytes(dims, n_sink) bytes, 4-byte
 *               aligned, owned by the caller (NULL allowed when that is 0);
 *               its contents on entry and exit are unspecified.
 *               KVP_EWORKSPACE if workspace_bytes is smaller.
 *   dims      : only batch, n_kv_heads and seq_len are read.
 * Results are exact (integer ranks); two kernels: a per-row stable radix
 * sort, then a per-row sweep over q whose cutoff only moves down. */
kvp_status_t kvp_running_cutoff(const float* score, kvp_dims_t dims, int32_t window, int32_t n_sink,
                                int32_t top_k, int32_t* rank, int32_t* cutoff, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* Static string for a status code. */
const char* kvp_status_string(kvp_status_t status);

/* Library ABI version (incremented on any signature change). */
int32_t kvp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVP_H_ */
