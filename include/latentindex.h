/*
 * latentindex.h -- C ABI of the LatentIndex decode indexer for AMD Instinct
 * MI355X (gfx950).
 *
 * The method (LatentIndex paper summary on picx.dev, "Methodology"): a group
 * of consecutive layers shares one latent cache c_t built from the anchor
 * layer's hidden state (eqs. 1-2); each layer l owns a decoder D^(l) that
 * defines its indexer keys k_t = D^(l) c_t (+ b^(l) on the NoPE part, eq. 3);
 * decoders are absorbed into the queries, q~ = D^T q and beta = q^N . b
 * (eq. 6), so that q . k_t = q~ . c_t + beta (eq. 7); every layer scores the
 * shared cache with u_t = sum_h w_h ReLU(q~_h . c_t + beta_h) (eq. 8) and
 * keeps its own top-k (the TopK definition after eq. 8).  Hierarchical
 * selection ("Hierarchical Selection" paragraph): the anchor's top-B
 * positions form a candidate set that each follower rescores and refines.
 *
 * Conventions shared by every call:
 *  - Ownership: the caller allocates every buffer (inputs, outputs and the
 *    workspace); the library never allocates, frees or synchronises.
 *  - Pointers named "device" must be device memory of the current HIP device;
 *    all other arguments are host values.  Arrays are dense row-major.
 *  - Execution: each call only enqueues kernels on `stream` (a hipStream_t;
 *    NULL = the null stream) and returns.  Results are ready when the stream
 *    reaches that point.
 *  - Errors: every shape/dtype/pointer check runs on the host before any
 *    launch; a non-OK status means nothing was enqueued (LI_ERR_HIP: a launch
 *    failed).  li_last_error() returns a thread-local message.  Device data
 *    is trusted: out-of-range block-table entries, token ids or lengths are
 *    undefined behaviour.
 *  - Only gfx950 devices are supported (LI_ERR_UNSUPPORTED otherwise).
 *  - Calls are reentrant.  Besides the thread-local error string the library
 *    keeps, per device and behind locks or atomics: the result of the
 *    architecture check, the compute-unit count, and whether a kernel's
 *    dynamic-LDS limit has been raised.  None of it changes results.
 *  - Scores are never NaN for finite inputs.  Ordering of scores treats
 *    -0.0 and +0.0 as equal.  "Top-k" always means: the first min(k, n)
 *    positions under (score descending, token id ascending), returned as
 *    ascending token ids and padded with -1.
 */
#ifndef LATENTINDEX_H
#define LATENTINDEX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum li_status {
  LI_OK = 0,
  LI_ERR_INVALID = 1,      /* bad pointer, size or combination of arguments */
  LI_ERR_UNSUPPORTED = 2,  /* valid request outside what the library implements */
  LI_ERR_HIP = 3           /* a HIP runtime call or kernel launch failed */
} li_status;

typedef enum li_dtype {
  LI_FP32 = 0,
  LI_BF16 = 1,
  LI_FP8_E4M3 = 2          /* OCP E4M3FN: bias 7, no inf, max 448 */
} li_dtype;

/*
 * One layer group's paged latent cache (the shared cache of "Methodology",
 * eq. 2).  Token t of sequence s lives in physical block
 * block_table[s * max_blocks + t / block_size], row t % block_size.
 *   data        device [n_blocks, block_size, r] of `dtype` (FP32, BF16 or
 *               FP8_E4M3).  Row-major: one token's r values are contiguous.
 *   scale       device fp32 [n_blocks, block_size, n_scales]: per-token
 *               dequantisation scales, FP8 only (NULL otherwise).  Value of
 *               element j = code * scale[j / scale_block] (one scale per
 *               token when scale_block == 0).
 *   block_table device int32 [n_seq, max_blocks] physical block ids.
 *   block_size  must be 64.
 *   r           latent width d_C; a multiple of 16, at most 1024.
 *   scale_block FP8: 0 (one scale per token, n_scales = 1) or 128 (one scale
 *               per 128-value block, n_scales = ceil(r / 128): with r = 192,
 *               a 200-byte token record of 192 codes and two fp32 scales: the
 *               200-byte per-token latent, scales included, that the
 *               LatentIndex explainer's storage paragraph counts).  Must be 0
 *               for other types.
 */
typedef struct li_cache {
  void *data;
  float *scale;
  const int32_t *block_table;
  int32_t n_seq;
  int32_t max_blocks;
  int32_t n_blocks;
  int32_t block_size;
  int32_t r;
  li_dtype dtype;
  int32_t scale_block;
} li_cache;

/* Thread-local message describing the last non-OK status of this thread. */
const char *li_last_error(void);

/* LI_OK if the current HIP device is a gfx950, LI_ERR_UNSUPPORTED if not. */
li_status li_check_device(void);

/*
 * li_append_latent -- write new tokens' shared latents into the cache
 * ("Methodology", eqs. 1-2: c_t = [Q_t P_R^T x_t ; P_N^T x_t], built once per
 * token from the anchor layer's hidden state x_t).
 *   x          device [n_tok, d_model] of x_dt (FP32 or BF16).
 *   P          device [d_model, r] of x_dt; columns 0..r_R-1 are P_R, the
 *              rest P_N.  NULL: x already is the latent (d_model must be r).
 *   rope_theta device fp32 [r_R / 2] rotary frequencies, or NULL when
 *              r_R == 0.  Pair (2j, 2j+1) of the R branch is rotated by the
 *              angle pos * theta_j (as the complex number z_2j + i z_2j+1
 *              times exp(i * angle)); the angle is formed in double.
 *   seq_idx, pos device int32 [n_tok]: destination sequence and position.
 *   cache      destination; BF16: round to nearest even; FP8: per token
 *              (per 128-value block when scale_block == 128) amax = max|c|,
 *              scale = amax / 448, codes = RNE(c * (448 / amax)) saturated
 *              to +-448 (amax == 0: scale 1, codes 0); FP32: stored as is.
 *              The projection accumulates in fp32.
 *   ws         device workspace of li_append_workspace_bytes() bytes
 *              (may be NULL when that is 0, i.e. when P is NULL).
 * Tokens with equal (seq_idx, pos) race.  n_tok == 0 is a no-op.
 */
size_t li_append_workspace_bytes(int32_t n_tok, int32_t d_model, int32_t r, int32_t has_P);
li_status li_append_latent(const void *x, li_dtype x_dt, int32_t n_tok, int32_t d_model,
                           const void *P, const float *rope_theta, int32_t r_R,
                           const int32_t *seq_idx, const int32_t *pos, const li_cache *cache,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * li_absorb_queries -- query-side decoder absorption ("Methodology", eq. 6):
 * q~_{s,h} = D^T q_{s,h} and beta_{s,h} = q_{s,h}[nope_off:] . b, for
 * n_layers layers in one call (each with its own decoder; every operand is
 * stacked layer-major).
 *   q        device [n_layers, n_q, H, d_I] of q_dt (FP32 or BF16).
 *   Dt       device fp32 D transposed, per layer [r, d_I] row-major; head h
 *            uses the layer's Dt + h * Dt_head_stride (elements; 0 = one
 *            decoder for all heads, the per-layer decoder of eq. 3, else a
 *            layer holds H * Dt_head_stride elements).
 *   b        device fp32 [n_layers, d_I - nope_off] key bias on the NoPE
 *            coordinates, or NULL for b = 0.  0 <= nope_off <= d_I.
 *   q_tilde  device fp32 [n_layers, n_q, H, r] (out).
 *   beta     device fp32 [n_layers, n_q, H] (out); may be NULL.
 * Accumulates in fp32.  1 <= n_layers <= 64, H <= 1024, d_I <= 1024,
 * r <= 1024; d_I and Dt_head_stride multiples of 4, q and Dt 16-byte
 * aligned.
 */
li_status li_absorb_queries(const void *q, li_dtype q_dt, int32_t n_layers, int32_t n_q,
                            int32_t H, int32_t d_I, const float *Dt, int64_t Dt_head_stride,
                            const float *b, int32_t nope_off, int32_t r, float *q_tilde,
                            float *beta, void *stream);

/*
 * li_append_absorb -- li_append_latent without a projection (P = NULL,
 * d_model = cache->r) and li_absorb_queries with r = cache->r, in one
 * launch: the decode step's two independent preludes (the new tokens' latents
 * c_t of "Methodology", eqs. 1-2, stored into the cache, and the queries'
 * absorption of eq. 6).  Arguments, layouts, limits and results are those of
 * the two calls; the results are identical to theirs, bit for bit.  The
 * queries' absorption reads nothing the append writes, so the two halves may
 * run in any order.  Either n_tok or n_q may be 0.  Errors as for the two
 * calls; on an error nothing is launched.
 */
li_status li_append_absorb(const void *x, li_dtype x_dt, int32_t n_tok, const float *rope_theta,
                           int32_t r_R, const int32_t *seq_idx, const int32_t *pos,
                           const li_cache *cache, const void *q, li_dtype q_dt, int32_t n_layers,
                           int32_t n_q, int32_t H, int32_t d_I, const float *Dt,
                           int64_t Dt_head_stride, const float *b, int32_t nope_off,
                           float *q_tilde, float *beta, void *stream);

/*
 * li_score -- score the shared cache for n_q queries ("Methodology", eq. 8):
 * scores[i * ld + t] = sum_h w[i,h] ReLU(q~[i,h,:] . c_t + beta[i,h]) for
 * 0 <= t < q_len[i], c_t read from sequence q_seq[i].  Entries at
 * t >= q_len[i] are left untouched.
 *   q_tilde  device [n_q, H, r] of qt_dt: FP32 (decode; absorbed queries as
 *            li_absorb_queries returns them) or BF16 (stored absorbed queries).
 *   w        device fp32 [n_q, H] head weights.
 *   beta     device fp32 [n_q, H] or NULL (= 0).
 *   q_seq    device int32 [n_q] sequence of each query.
 *   q_len    device int32 [n_q] causal prefix length (1 <= q_len[i], and
 *            q_len[i] <= max_len, and the sequence holds that many tokens).
 *   max_len  host bound on every q_len (used to size the launch), <= ld.
 *   scores   device fp32 [n_q, ld] (out).
 * Arithmetic, by cache:
 *  - FP32 cache (any H, r), and BF16 / FP8 caches of other shapes: vector
 *    ALU; cache values and q~ decoded exactly to fp32, products and sums in
 *    fp32.
 *  - BF16 cache, H = 64, r = 256 (or r = 192 with at most 64 queries): bf16
 *    matrix cores.  An FP32 q~ is carried
 *    as a pair of bf16 values (hi = RNE(q~), lo = RNE(q~ - hi)) whose sum is
 *    within 2^-16 relative of q~; a BF16 q~ is used as is.  Products are
 *    exact, sums in fp32.
 *  - FP8 cache, H = 64, r = 128, 192 or 256 (and at most 64 queries, or
 *    r = 256 with one scale per token): fp8 matrix cores.  Each head's q~ is
 *    scaled by a power of two (largest element into (224, 448]) and split
 *    into E4M3 terms, each the rounding of what the earlier terms left: two
 *    terms with at most 64 queries (about 2^-8 relative, a bf16 q~'s
 *    precision), three above that (about 2^-12; two for a BF16 q~); the
 *    matrix core accumulates each 128-long group of exact fp8 products in
 *    fp32 to about 2^-11 of the group's largest product.
 *  The FP8 scales (and the head's power of two) multiply the dot products
 *  of their blocks before beta and ReLU.
 */
li_status li_score(const void *q_tilde, li_dtype qt_dt, const float *w, const float *beta,
                   int32_t n_q, int32_t H, const int32_t *q_seq, const int32_t *q_len,
                   int32_t max_len, const li_cache *cache, float *scores, int64_t ld,
                   void *stream);

/*
 * li_topk -- each layer's own selection (the TopK definition after eq. 8:
 * S = TopK_{t in V}(u_t, min(k, |V|))), per row of a score matrix.
 *   scores    device fp32 [n_rows, ld]; row i is valid on [0, valid_len[i]).
 *   valid_len device int32 [n_rows], each in [0, max_len].
 *   max_len   host bound on valid_len, <= ld.
 *   k         1 <= k <= 65536.
 *   out_idx   device int32 [n_rows, k] (out): ascending token ids of the
 *             first min(k, valid_len) positions by (score desc, id asc),
 *             then -1.
 *   out_val   device fp32 [n_rows, k] (out, may be NULL): the score of each
 *             selected id; -inf in padding slots.
 *   ws        device workspace of li_topk_workspace_bytes() bytes.
 * Integer decisions are made on the fp32 bit patterns (no rounding).
 */
size_t li_topk_workspace_bytes(int32_t n_rows, int32_t max_len, int32_t k);
li_status li_topk(const float *scores, int64_t ld, int32_t n_rows, const int32_t *valid_len,
                  int32_t max_len, int32_t k, int32_t *out_idx, float *out_val, void *ws,
                  size_t ws_bytes, void *stream);

/*
 * li_hs_anchor_select -- the anchor layer's part of hierarchical selection
 * ("Hierarchical Selection" paragraph): from the anchor's full score rows,
 * the candidate set C = top-min(B, |V|) positions and the anchor's own
 * selection S = top-min(k, |V|) (S is inside C because B >= k), both in one
 * pass over the scores (rows of at most 8192 positions: one single-workgroup
 * selection per output instead, which is faster there).
 *   scores, ld, n_rows, valid_len, max_len: as for li_topk.
 *   max_len    at most 2,097,152 (LI_ERR_UNSUPPORTED beyond).
 *   B, cand    1 <= B <= 65536; cand device int32 [n_rows, B] (out):
 *              ascending token ids, -1 padded (the input of li_hs_select).
 *   k, sel     1 <= k <= B; sel device int32 [n_rows, k] (out), ascending,
 *              -1 padded.  sel may be NULL when only C is wanted.
 *   ws         device workspace of li_hs_anchor_workspace_bytes() bytes,
 *              zeroed once before its first use (e.g. one hipMemsetAsync);
 *              none (0 bytes, ws may be NULL) for max_len <= 8192.
 *              Each call leaves the counters it relies on zeroed again, so
 *              the workspace serves later calls of any n_rows <= 64 and
 *              max_len it is large enough for without another clear (with
 *              n_rows > 64 every call clears them itself).  Calls sharing
 *              a workspace must not overlap in time.
 * Results equal two li_topk calls with k = B and with k.
 */
size_t li_hs_anchor_workspace_bytes(int32_t n_rows, int32_t max_len);
li_status li_hs_anchor_select(const float *scores, int64_t ld, int32_t n_rows,
                              const int32_t *valid_len, int32_t max_len, int32_t B, int32_t *cand,
                              int32_t k, int32_t *sel, void *ws, size_t ws_bytes, void *stream);

/*
 * li_hs_anchor -- the anchor layer's whole part of hierarchical selection in
 * one call ("Hierarchical Selection" paragraph, eq. 8): its scores of every
 * position (as li_score) and, from them, C and S (as li_hs_anchor_select).
 * For the caches the issuer/compute scorer serves (bf16 with r = 192 or
 * 256, fp8 with r = 128, 192 or 256), H = 64, at most 64 queries (and no
 * more than the cache has sequences) and max_len above 8192, the scorer
 * builds the rows' key histograms as it writes the scores, so the selection
 * does not read them an extra time; otherwise it is the two calls in turn.
 *   q_tilde .. ld: as for li_score; q_len[i] is also row i's valid length;
 *               max_len at most 2,097,152 (LI_ERR_UNSUPPORTED beyond).
 *   B, cand, k, sel: as for li_hs_anchor_select.
 *   ws          device workspace of li_hs_anchor_workspace_bytes(n_q,
 *               max_len) bytes, zeroed once before its first use and shared
 *               with li_hs_anchor_select on the same terms.
 *   scan_events NULL, or two hipEvent_t recorded on the stream just before
 *               and just after the scoring launch (to time the scorer alone).
 * Results equal li_score followed by li_hs_anchor_select.
 */
li_status li_hs_anchor(const void *q_tilde, li_dtype qt_dt, const float *w, const float *beta,
                       int32_t n_q, int32_t H, const int32_t *q_seq, const int32_t *q_len,
                       int32_t max_len, const li_cache *cache, float *scores, int64_t ld,
                       int32_t B, int32_t *cand, int32_t k, int32_t *sel, void *ws, size_t ws_bytes,
                       void *const *scan_events, void *stream);

/*
 * li_score_topk -- one layer's full-scan selection in one call ("Methodology",
 * eq. 8 and the TopK definition after it): the scores of every position (as
 * li_score) and each query's top-min(k, q_len[i]) positions (as li_topk with
 * valid_len = q_len).  On the caches and shapes li_hs_anchor names, the
 * scorer builds the rows' key histograms as it writes the scores, so the
 * selection reads them once fewer.
 *   q_tilde .. ld: as for li_score; max_len at most 2,097,152.
 *   k, out_idx   1 <= k <= 65536; out_idx device int32 [n_q, k] (out):
 *                ascending token ids, -1 padded.
 *   ws           device workspace of li_hs_anchor_workspace_bytes(n_q,
 *                max_len) bytes, zeroed once before its first use and kept
 *                valid by every call (shared with li_hs_anchor and
 *                li_hs_anchor_select on the same terms).
 *   scan_events  NULL, or two hipEvent_t recorded just before and just after
 *                the scoring launch.
 * Results equal li_score followed by li_topk.
 */
li_status li_score_topk(const void *q_tilde, li_dtype qt_dt, const float *w, const float *beta,
                        int32_t n_q, int32_t H, const int32_t *q_seq, const int32_t *q_len,
                        int32_t max_len, const li_cache *cache, float *scores, int64_t ld,
                        int32_t k, int32_t *out_idx, void *ws, size_t ws_bytes,
                        void *const *scan_events, void *stream);

/*
 * li_hs_select -- the follower layers' hierarchical selection ("Hierarchical
 * Selection" paragraph): rescore only the anchor's candidate set with each
 * follower's own absorbed queries, then keep each follower's top-k within
 * the set.  The n_f followers of a group share the candidate set, so one
 * call serves them all (operands stacked follower-major).
 *   cand        device int32 [n_q, B]: ascending token ids of query i's
 *               candidates (e.g. li_topk with k = B on the anchor's scores),
 *               padded at the end with -1.
 *   n_f         followers, 1 <= n_f <= 64.
 *   q_tilde     device [n_f, n_q, H, r] of qt_dt (FP32 or BF16).
 *   w, beta     device fp32 [n_f, n_q, H]; beta may be NULL.
 *   q_seq, H, cache: as for li_score.
 *   k           1 <= k <= B.
 *   out_idx     device int32 [n_f, n_q, k] (out): ascending token ids, -1
 *               padded.
 *   cand_scores device fp32 [n_f, n_q, B] (out, may be NULL): each
 *               follower's score of each candidate slot; -inf in padding.
 *   ws          device workspace of li_hs_workspace_bytes() bytes.
 * Ties are broken by token id (equivalently by candidate slot).
 */
size_t li_hs_workspace_bytes(int32_t n_f, int32_t n_q, int32_t B, int32_t k);
li_status li_hs_select(const int32_t *cand, int32_t B, int32_t n_f, const void *q_tilde,
                       li_dtype qt_dt, const float *w, const float *beta, int32_t n_q, int32_t H,
                       const int32_t *q_seq, const li_cache *cache, int32_t k, int32_t *out_idx,
                       float *cand_scores, void *ws, size_t ws_bytes, void *stream);

/*
 * li_calib_gram -- the normal equations of the training-free calibration
 * ("Methodology", Training-free Calibration: ridge reduced-rank regression
 * jointly fitting the group's shared projection and every layer's decoder
 * to the layers' indexer keys): over n calibration tokens,
 *   G_xx = X^T X, G_xy = X^T Y, x_sum = X^T 1, y_sum = Y^T 1,
 * written (accumulate == 0) or added to what the outputs hold (so that the
 * tokens can come in batches).  The closed-form solves that follow work on
 * these small matrices.
 *   X      device [n, d] of x_dt (FP32 or BF16): the anchor hidden states.
 *   Y      device [n, e] of y_dt (FP32 or BF16), or NULL: the layers' keys,
 *          stacked along columns.
 *   G_xx   device fp32 [d, d] (out); G_xy device fp32 [d, e] (out, may be
 *          NULL); x_sum device fp32 [d], y_sum device fp32 [e] (out, each
 *          may be NULL).
 * Products exact in fp32 on the matrix cores, sums in fp32 in a fixed order
 * (deterministic).  1 <= d, e <= 65536; n >= 0 (n == 0 with accumulate == 0
 * writes zeros).
 */
li_status li_calib_gram(const void *X, li_dtype x_dt, int64_t n, int32_t d, const void *Y,
                        li_dtype y_dt, int32_t e, float *G_xx, float *G_xy, float *x_sum,
                        float *y_sum, int32_t accumulate, void *stream);

/*
 * li_hs_select_noalloc -- li_hs_select for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Arguments, checks and results are li_hs_select's
 * without the ws / ws_bytes pair: the workspace is a fixed array of
 * LI_HS_NOALLOC_SCRATCH_BYTES bytes of the library's own device memory, one
 * per device, held until the process ends.  The call allocates and frees
 * nothing.  A call whose li_hs_workspace_bytes(n_f, n_q, B, k) exceeds that
 * size returns LI_ERR_UNSUPPORTED with nothing enqueued.  Every call on a
 * device uses that device's one array: calls that overlap in time on one
 * device (two streams, two threads without ordering) race and must be
 * serialised by the caller.  The array keeps nothing between calls: each call
 * writes or clears everything it reads there.
 */
#define LI_HS_NOALLOC_SCRATCH_BYTES (8u << 20)
li_status li_hs_select_noalloc(const int32_t *cand, int32_t B, int32_t n_f, const void *q_tilde,
                               li_dtype qt_dt, const float *w, const float *beta, int32_t n_q,
                               int32_t H, const int32_t *q_seq, const li_cache *cache, int32_t k,
                               int32_t *out_idx, float *cand_scores, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LATENTINDEX_H */
