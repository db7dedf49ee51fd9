/*
 * entmaxkv.h - C ABI of the EntmaxKV support-aware paged decode library
 * (HIP, AMD CDNA4 / gfx950).
 *
 * The method is the one described by the web pages "Technical Summary:
 * EntmaxKV - Support-Aware Decoding for Entmax Attention" (gist.science) and
 * the arXiv abstract "EntmaxKV: Support-Aware Decoding for Entmax Attention"
 * (mlsanity.com index).  One decode step for a query reads lightweight
 * per-page key summaries, scores every page against the query, selects
 * candidate pages, gathers only those pages' keys and values through the page
 * table and runs alpha-entmax attention over them (Technical Summary, §2 A-C).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every array argument is a DEVICE pointer unless stated otherwise; the
 *    two structs below are HOST structs, read during the call only.
 *  - The caller allocates and owns every buffer.  The library never
 *    allocates or frees device memory, never synchronises and never copies
 *    device to host.  (ekv_entmax_decode_noalloc alone works in a static
 *    device array of the library instead of a caller's workspace.)  Work is enqueued on `stream` (a hipStream_t passed as
 *    void*; NULL is the default stream).  Results are valid once the caller
 *    has synchronised with that stream.
 *  - Unit: one (sequence b, KV head h) pair.  Query heads of KV head h are
 *    h*G .. h*G+G-1 (grouped-query attention with group size G); one page
 *    selection is made per unit and shared by its G query heads.
 *  - Scores: s_i = scale * <q, k_i>.  Entmax argument z_i = (alpha-1) s_i,
 *    threshold tau, exponent r = 1/(alpha-1): p_i = max(z_i - tau, 0)^r with
 *    sum_i p_i = 1 (alpha > 1; alpha = 2 is sparsemax).
 *  - Validation happens on the host before anything is launched; a failed
 *    validation returns EKV_ERR_INVALID_ARG or EKV_ERR_UNSUPPORTED and
 *    launches nothing.  A failed launch returns EKV_ERR_HIP.
 *    ekv_last_error() gives a message for the calling thread's last failure.
 *  - Device-resident contract (not checked): page_table entries for logical
 *    pages < ceil(seq_lens[b]/P) are in [0, num_slots); 1 <= seq_lens[b] <=
 *    max_pages * P; selection lists hold ascending, distinct logical pages
 *    below ceil(seq_lens[b]/P) with 1 <= count <= that page count.
 *  - Determinism: identical inputs give bit-identical outputs (no floating
 *    point atomics; every reduction has a fixed order).
 *  - Concurrency: no global mutable state besides the per-thread error text
 *    and the per-device scratch of ekv_entmax_decode_noalloc; calls on
 *    different streams with disjoint outputs and workspaces may run
 *    concurrently.
 */
#ifndef ENTMAXKV_H
#define ENTMAXKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EKV_VERSION 10000 /* 1.0.0 */

typedef enum ekv_status {
  EKV_OK = 0,
  EKV_ERR_INVALID_ARG = 1, /* null pointer, bad size, alpha <= 1, ...      */
  EKV_ERR_UNSUPPORTED = 2, /* valid but not built: D, P, G or dtype        */
  EKV_ERR_WORKSPACE = 3,   /* workspace missing, short or misaligned       */
  EKV_ERR_HIP = 4          /* a HIP launch reported an error               */
} ekv_status;

typedef enum ekv_dtype {
  EKV_F32 = 0,
  EKV_BF16 = 1
} ekv_dtype;

/* Scoring modes (bit flags, may be combined). */
#define EKV_SCORE_BBOX 1
#define EKV_SCORE_GAUSS 2

/* Operations for ekv_workspace_size. */
#define EKV_OP_SELECT_TOPK 1
#define EKV_OP_SELECT_GAUSS 2
#define EKV_OP_ENTMAX_DECODE 3
#define EKV_OP_SOFTMAX_DECODE 4
#define EKV_OP_ENTMAX_DECODE_SMALL 5

/*
 * Paged KV cache (Technical Summary, §2 and §2.A: the cache is cut into
 * fixed-size pages).  Physical pages ("slots") live in one pool; each
 * sequence maps its logical pages to slots through its page-table row.
 *   k, v        [num_slots][num_kv_heads][page_size][head_dim], kv_dtype
 *   page_table  [batch][max_pages] int32 logical page -> slot
 *   seq_lens    [batch] int32 valid tokens of each sequence
 * Supported: head_dim in {64, 128}; page_size in {16, 32, 64};
 * group in {1, 2, 4, 8}; kv_dtype EKV_F32 or EKV_BF16; batch *
 * num_kv_heads <= 4096; group * max_pages * page_size * 4 bytes (one unit's
 * scores) below 2 GiB - 64 KiB.  k, v and the metadata arrays must be
 * 16-byte aligned.
 */
typedef struct ekv_paged_kv {
  int32_t batch;
  int32_t num_kv_heads;
  int32_t group;
  int32_t head_dim;
  int32_t page_size;
  int32_t num_slots;
  int32_t max_pages;
  int32_t kv_dtype; /* ekv_dtype */
  const void *k;
  const void *v;
  const int32_t *page_table;
  const int32_t *seq_lens;
} ekv_paged_kv;

/*
 * Per-page key metadata (Technical Summary, §2.A: coordinate-wise minimum
 * and maximum keys for the box bound; first and second moments for the
 * Gaussian statistics).
 *   bbox   [num_slots][num_kv_heads][2][head_dim] in kv_dtype: [0] = kmin,
 *          [1] = kmax over the page's valid tokens (exact).  May be NULL.
 *   gauss  [num_slots][num_kv_heads][2][head_dim] float32: [0] = mean,
 *          [1] = population variance (divide by the valid token count)
 *          taken about the mean.  May be NULL.
 */
typedef struct ekv_meta {
  void *bbox;
  float *gauss;
} ekv_meta;

/*
 * ekv_build_meta - (re)build page metadata (Technical Summary, §2.A).
 * Rebuilds logical pages [first_page[b], ceil(seq_lens[b]/P)) of every
 * sequence b and every KV head; first_page == NULL rebuilds every page.
 * After appending tokens, passing first_page[b] = (seq_lens[b]-1)/P (the
 * page that received the token) refreshes only that page; the result is
 * bit-identical to a full rebuild.  span_hint is an upper bound on the
 * number of pages per sequence to rebuild, used only to size the launch
 * (<= 0: max_pages); the result never depends on it.  Null bbox or gauss
 * in *meta skips that part.
 */
ekv_status ekv_build_meta(const ekv_paged_kv *kv, const int32_t *first_page,
                          int32_t span_hint, const ekv_meta *meta,
                          void *stream);

/*
 * ekv_score_pages - query-aware page scoring (Technical Summary, §2.A).
 *   q      [batch][H_q][head_dim] float32, H_q = num_kv_heads * group.
 *   mode   EKV_SCORE_BBOX and/or EKV_SCORE_GAUSS.
 *   ub     (BBOX) ekv_score_size(kv, EKV_SCORE_BBOX) floats:
 *          [batch][H_q][max_pages] the box upper bound
 *          scale * sum_d max(q_d kmin_d, q_d kmax_d) of every page's scores,
 *          followed by [batch][num_kv_heads][T] the largest bound over each
 *          tile of 64 logical pages and the group's query heads
 *          (T = ceil(max_pages / 64)).
 *   gstat  (GAUSS) ekv_score_size(kv, EKV_SCORE_GAUSS) floats:
 *          [batch][H_q][max_pages][2] the mean scale * <q, mean> and the
 *          variance scale^2 * sum_d q_d^2 var_d of a page key's score under
 *          the page's diagonal Gaussian, followed (from the next multiple of
 *          4 floats) by [batch][H_q][T][4] per 64-page tile: max mu,
 *          max (mu + 8.5 sigma), max (mu + sqrt(2 ln P) sigma), 0.
 * The tile summaries let the selectors skip tiles that cannot matter.
 * Columns >= ceil(seq_lens[b]/P), and tiles past the last page, are left
 * untouched.  gstat must be 16-byte aligned.
 */
ekv_status ekv_score_pages(const ekv_paged_kv *kv, const ekv_meta *meta,
                           const float *q, float scale, int32_t mode,
                           float *ub, float *gstat, void *stream);

/*
 * ekv_refresh_score_pages - the metadata refresh and the scoring of one
 * decode step in one call (Technical Summary, §2.A: metadata kept up to date
 * as tokens arrive, then query-aware scoring).  For every sequence b with
 * seq_lens[b] > 0, the metadata of its last logical page (the page the
 * newest token went to) is rebuilt for every KV head, bit-identical to
 * ekv_build_meta; then the pages are scored exactly as by ekv_score_pages.
 * It replaces ekv_build_meta(first_page[b] = (seq_lens[b]-1)/P, span 1)
 * followed by ekv_score_pages, for steps that append at most one page's
 * worth of tokens per sequence, all of them to its last page.  Both parts
 * of *meta that are non-NULL are refreshed; k must be non-NULL and 16-byte
 * aligned.  Arguments as for ekv_score_pages.  Usually one kernel on the
 * stream (each sequence's last tile is scored by the wave that rebuilt it);
 * two when batch * num_kv_heads exceeds the waves the device holds.
 */
ekv_status ekv_refresh_score_pages(const ekv_paged_kv *kv, const ekv_meta *meta,
                                   const float *q, float scale, int32_t mode,
                                   float *ub, float *gstat, void *stream);

/*
 * ekv_select_topk - fixed-budget selection (Technical Summary, §2.B.1).
 * For each unit, ranks pages by the largest bound over its G query heads
 * and keeps the min(k, n_pages) highest; equal bounds favour the lower page
 * index.  sel [batch][H_kv][max_pages] int32 receives the kept logical
 * pages in ascending order, count [batch][H_kv] int32 their number.
 * Workspace: ekv_workspace_size(EKV_OP_SELECT_TOPK, kv, k) bytes.
 */
ekv_status ekv_select_topk(const ekv_paged_kv *kv, const float *ub, int32_t k,
                           int32_t *sel, int32_t *count, void *ws,
                           size_t ws_bytes, void *stream);

/*
 * ekv_select_gauss - Gaussian-aware entmax selection (Technical Summary,
 * §2.B.2).  Per query head, tau_hat solves
 *   sum_p n_p E[max(Z_p - tau_hat, 0)^r] = 1,
 *   Z_p ~ N((alpha-1) mu_p, (alpha-1)^2 sigma_p^2)   (mu, sigma^2 = gstat),
 * i.e. the entmax normalisation with every token of page p drawn from the
 * page's score Gaussian.  A page is kept for the unit when, for some query
 * head h of the group, (alpha-1)(mu_hp + sigma_hp sqrt(2 ln n_p)) >
 * tau_hat_h - delta (the page's estimated largest score exceeds the
 * threshold minus the margin).  If no page passes, the single page with the
 * largest margin max_h[(alpha-1) mhat_hp - tau_hat_h] is kept (lower index on
 * ties).  Outputs: sel/count as for top-k (ascending, count >= 1) and
 * tau_hat [batch][H_q] float32.  1.1 <= alpha <= 2 (r = 1/(alpha-1) in
 * [1, 10], where x -> max(x - tau, 0)^r is convex): the expectation has a
 * closed form in the normal CDF and density for alpha = 1.5 and 2 and is a
 * 24-node Gauss-Jacobi sum (16-node Gauss-Hermite far below the page mean)
 * otherwise, the rules built on the host at each call (see
 * ekv_quadrature_rule); other alpha return EKV_ERR_UNSUPPORTED.
 * delta >= 0.  Workspace: ekv_workspace_size(EKV_OP_SELECT_GAUSS, kv, 0)
 * bytes (one 64-bit page mask per query head and 64-page tile), 256-byte
 * aligned; its contents on entry do not matter.  tau_hat is found by
 * Newton iterations in float32 that climb to the root from a proven lower
 * bound (two kernels on the stream).
 */
ekv_status ekv_select_gauss(const ekv_paged_kv *kv, const float *gstat,
                            float alpha, float delta, int32_t *sel,
                            int32_t *count, float *tau_hat, void *ws,
                            size_t ws_bytes, void *stream);

/*
 * ekv_entmax_decode - sparse alpha-entmax attention over the selected pages
 * (Technical Summary, §2.C), gathered through the page table.  For each
 * query head: z_i = (alpha-1) scale <q, k_i> over the tokens of the
 * selected pages; tau solves sum_i max(z_i - tau, 0)^r = 1 (exact to
 * floating-point rounding for alpha in {1.5, 2}, by bisection otherwise);
 * out = sum_i p_i v_i / sum_i p_i with p_i = max(z_i - tau, 0)^r.
 *   sel, count   as produced by the selectors; sel == NULL means every page
 *                of every sequence (the full-cache entmax baseline), and
 *                count is then ignored.
 *   tau_hint     [batch][H_q] float32 or NULL: an estimate of each head's
 *                threshold, typically tau_hat from ekv_select_gauss.  The
 *                result does not depend on it (up to the floating-point
 *                order of the support sums); it only lets the key pass keep
 *                the scores above hint - 1/32 instead of all of them.  The
 *                threshold step checks that the kept scores alone reach the
 *                normalisation at that floor, which proves every support
 *                score was kept; when they do not (a hint too high, or more
 *                than 8192 kept scores or 2048 pages with kept scores per
 *                head) it recomputes that head's scores from the keys and
 *                solves as without a hint, which is slower.  Used for
 *                bfloat16 keys only, and ignored when probs is not NULL.
 *   out          [batch][H_q][head_dim] float32.
 *   tau          [batch][H_q] float32 or NULL.
 *   probs        [batch][H_q][max_pages*P] float32 or NULL (debug): p of
 *                every logical token, zero outside the selection, over
 *                [0, seq_lens[b]).
 * Workspace: ekv_workspace_size(EKV_OP_ENTMAX_DECODE, kv, 0).
 * Runs ekv_entmax_scores, ekv_entmax_threshold, ekv_entmax_apply in order.
 */
ekv_status ekv_entmax_decode(const ekv_paged_kv *kv, const float *q,
                             float scale, float alpha, const int32_t *sel,
                             const int32_t *count, const float *tau_hint,
                             float *out, float *tau, float *probs, void *ws,
                             size_t ws_bytes, void *stream);

/*
 * ekv_entmax_decode_noalloc - ekv_entmax_decode without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * workspace is a static device array of EKV_NOALLOC_SCRATCH_BYTES in the
 * library, one per GPU, held until the process ends; the call allocates
 * nothing (its first call on a GPU looks up that GPU's copy of the array).
 * Arguments, results and errors as for ekv_entmax_decode; a cache whose
 * workspace, ekv_workspace_size(EKV_OP_ENTMAX_DECODE, kv, 0), exceeds
 * EKV_NOALLOC_SCRATCH_BYTES returns EKV_ERR_WORKSPACE and launches nothing.
 * Every call on one GPU uses the same array: calls that overlap on one GPU
 * (different streams, or threads) race and must be serialised by the
 * caller.  No part of the array needs clearing between calls.
 */
#define EKV_NOALLOC_SCRATCH_BYTES (64u << 20) /* 64 MiB */
ekv_status ekv_entmax_decode_noalloc(const ekv_paged_kv *kv, const float *q,
                                     float scale, float alpha,
                                     const int32_t *sel, const int32_t *count,
                                     const float *tau_hint, float *out,
                                     float *tau, float *probs, void *stream);

/*
 * ekv_entmax_decode_small - ekv_entmax_decode in a single launch for small
 * selections (Technical Summary, §2.B.1 and §2.C: a fixed budget of k pages
 * per unit).  Blocks share each unit's selection: they gather its keys
 * through the page table and compute z for the unit's G query heads; the
 * last block to finish solves each head's tau exactly (alpha in {1.5, 2};
 * bisection otherwise) and sums the value rows of the support.  Scores stay
 * on chip when one block takes a unit (many units); otherwise they pass
 * through the workspace once.
 *   sel, count   as for ekv_entmax_decode (sel == NULL: every page).
 *   max_count    an upper bound on every unit's page count (for top-k
 *                selections: min(k, max_pages)), 1 <= max_count and
 *                max_count * page_size <= 2048 (EKV_ERR_INVALID_ARG below
 *                1, EKV_ERR_UNSUPPORTED above 2048 tokens).  A unit whose
 *                count exceeds max_count or max_pages gets NaN in its rows
 *                of out and tau, and nothing past the bound is read.
 *   out, tau     as for ekv_entmax_decode (tau nullable).
 * bfloat16 keys only (EKV_ERR_UNSUPPORTED otherwise).
 * Workspace: ekv_workspace_size(EKV_OP_ENTMAX_DECODE_SMALL, kv, max_count)
 * bytes, 256-byte aligned.  Unlike the other workspaces it holds state: it
 * must be zero-filled before its first use, and every call leaves it ready
 * for the next (its arrival counters back at zero).  Calls that overlap in
 * time must not share one.
 */
ekv_status ekv_entmax_decode_small(const ekv_paged_kv *kv, const float *q,
                                   float scale, float alpha,
                                   const int32_t *sel, const int32_t *count,
                                   int32_t max_count, float *out, float *tau,
                                   void *ws, size_t ws_bytes, void *stream);

/*
 * The three steps of ekv_entmax_decode, for callers that time or interleave
 * them.  They must be called in this order with the same kv, sel, count,
 * alpha and workspace.
 *   ekv_entmax_scores     gathers the selected keys and writes z to the
 *                         workspace with per-page maxima (with tau_hint,
 *                         only the scores above hint - 1/32, see
 *                         ekv_entmax_decode).
 *   ekv_entmax_threshold  solves tau per query head (tau may be NULL: it is
 *                         then kept in the workspace only) and gathers the
 *                         values of the support: with a selection (sel not
 *                         NULL) it writes every row of out; over the full
 *                         cache, the rows of the heads whose candidate
 *                         scores fit on chip (the usual case).
 *   ekv_entmax_apply      writes the remaining rows of out (all rows, and
 *                         probs, when probs is not NULL), reading values
 *                         only for tokens with p_i > 0.  With a selection
 *                         and probs NULL nothing remains: it returns
 *                         EKV_OK without launching any work.
 */
ekv_status ekv_entmax_scores(const ekv_paged_kv *kv, const float *q,
                             float scale, float alpha, const int32_t *sel,
                             const int32_t *count, const float *tau_hint,
                             void *ws, size_t ws_bytes, void *stream);
ekv_status ekv_entmax_threshold(const ekv_paged_kv *kv, float alpha,
                                const int32_t *sel, const int32_t *count,
                                float *tau, float *out, void *ws,
                                size_t ws_bytes, void *stream);
ekv_status ekv_entmax_apply(const ekv_paged_kv *kv, float alpha,
                            const int32_t *sel, const int32_t *count,
                            float *out, float *probs, void *ws,
                            size_t ws_bytes, void *stream);

/*
 * ekv_softmax_decode - split-K softmax attention (the full-cache baseline
 * the Technical Summary, §4, compares against).  Each piece of the pages
 * (bfloat16 K/V: a wave's run of pages within one unit; float32: a chunk of
 * pages) yields (running max, sum of exponentials, weighted value sum); a
 * second kernel merges the pieces in log-sum-exp form.  sel/count as above (NULL sel =
 * full cache).  out [batch][H_q][head_dim] float32; lse [batch][H_q]
 * float32 (natural log of sum_i exp(s_i)) or NULL.
 * Workspace: ekv_workspace_size(EKV_OP_SOFTMAX_DECODE, kv, 0).
 */
ekv_status ekv_softmax_decode(const ekv_paged_kv *kv, const float *q,
                              float scale, const int32_t *sel,
                              const int32_t *count, float *out, float *lse,
                              void *ws, size_t ws_bytes, void *stream);

/*
 * ekv_read_probe - measurement aid (not part of the method): streams `bytes`
 * (a multiple of 16, buf 16-byte aligned) from the device buffer `buf` with
 * 16-byte loads over the whole device and writes one 32-bit checksum per
 * wave to sink[0 .. EKV_READ_PROBE_SINK).  Timing it gives the HBM read
 * bandwidth the decode kernels' load pattern can reach.
 */
#define EKV_READ_PROBE_SINK 8192
ekv_status ekv_read_probe(const void *buf, size_t bytes, uint32_t *sink,
                          void *stream);

/*
 * ekv_quadrature_rule - the Gauss rules behind ekv_select_gauss at alpha
 * other than 1.5 and 2 (host only; no device work).  kind 0: Gauss-Jacobi
 * nodes and weights for the weight (1 + x)^param on [-1, 1], param > -1;
 * kind 1: Gauss-Hermite for the standard normal density (param ignored).
 * Writes n (1..64) nodes, ascending, and their weights to the host arrays
 * nodes[n] and weights[n]; EKV_ERR_INVALID_ARG otherwise.
 */
#define EKV_RULE_JACOBI 0
#define EKV_RULE_HERMITE 1
ekv_status ekv_quadrature_rule(int32_t kind, double param, int32_t n,
                               double *nodes, double *weights);

/* Floats of the ub (EKV_SCORE_BBOX) or gstat (EKV_SCORE_GAUSS) buffer,
 * page values plus tile summaries (host only; 0 on invalid input). */
size_t ekv_score_size(const ekv_paged_kv *kv, int32_t mode);

/* Bytes of workspace an operation needs (host only; 0 on invalid input). */
size_t ekv_workspace_size(int32_t op, const ekv_paged_kv *kv, int32_t k_or_0);

/* Static description of a status code (host only). */
const char *ekv_status_string(ekv_status s);

/* Message describing the calling thread's most recent failure (host only). */
const char *ekv_last_error(void);

/* EKV_VERSION of the built library (host only). */
int32_t ekv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ENTMAXKV_H */
