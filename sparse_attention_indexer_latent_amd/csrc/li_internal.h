// Host-side launcher interface between the C ABI layer (latentindex_api.cpp)
// and the kernel translation units.  Every launcher enqueues on `st`, assumes
// its arguments were validated by the ABI layer, and returns the status of
// the launch (hipGetLastError after enqueue).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/latentindex.h"

namespace li {

// Plain-value view of a validated li_cache, passed to kernels by value.
struct CacheView {
  const void *data;
  const float *scale;
  const int32_t *block_table;
  int32_t max_blocks;
  int32_t r;
  int32_t dtype;  // li_dtype
  int32_t n_seq;
  int32_t n_blocks;
  int32_t scale_block;  // fp8: 0 (one scale per token) or 128
};

inline CacheView view_of(const li_cache &c) {
  return CacheView{c.data, c.scale, c.block_table, c.max_blocks, c.r, (int32_t)c.dtype, c.n_seq,
                   c.n_blocks, c.scale_block};
}

// Scales per token of a cache (0 for caches without scales).
__host__ __device__ inline int n_scales(const CacheView &cv) {
  if (cv.dtype != LI_FP8_E4M3) return 0;
  return cv.scale_block ? (cv.r + cv.scale_block - 1) / cv.scale_block : 1;
}

// Per-device state of the library (latentindex_api.cpp), thread-safe.
// Raises `fn`'s dynamic-LDS limit to `bytes` once per device (the attribute
// is a property of the kernel on the current device).
struct DeviceOnce;
DeviceOnce *device_once_new();
hipError_t raise_lds_limit(DeviceOnce *once, const void *fn, int bytes);
// Compute units of the current device (read once per device).
int device_cu_count();

// append.hip
size_t append_ws_bytes(int n_tok, int d_model, int r, bool has_P);
hipError_t launch_append(const void *x, int x_dt, int n_tok, int d_model, const void *P,
                         const float *theta, int r_R, const int32_t *seq_idx,
                         const int32_t *pos, const li_cache &cache, void *ws, hipStream_t st);
// Append without projection (x has cache.r columns) and absorption with
// r = cache.r, in one launch.
hipError_t launch_append_absorb(const void *x, int x_dt, int n_tok, const float *theta, int r_R,
                                const int32_t *seq_idx, const int32_t *pos, const li_cache &cache,
                                const void *q, int q_dt, int n_layers, int n_q, int H, int d_I,
                                const float *Dt, int64_t Dt_head_stride, const float *b,
                                int nope_off, float *q_tilde, float *beta, hipStream_t st);

// absorb.hip
hipError_t launch_absorb(const void *q, int q_dt, int n_layers, int n_q, int H, int d_I,
                         const float *Dt,
                         int64_t Dt_head_stride, const float *b, int nope_off, int r,
                         float *q_tilde, float *beta, hipStream_t st);

// Scorers.  Page mode (cand == nullptr): token t < q_len[i] of sequence
// q_seq[i] goes to out[i*ld + t].  Candidate mode: with c = i % cand_rows,
// slot j < B of query i scores token cand[c*B + j] of sequence q_seq[c] (or
// writes -inf where it is -1) into out[i*ld + j]; q_len is unused.  Several
// layers' queries (i = layer * cand_rows + c) thus share one candidate list.
// score_valu.hip: generic vector-ALU scorer, any supported dtype.
hipError_t launch_score_valu(const void *q_tilde, int qt_dt, const float *w, const float *beta,
                             int n_q, int H, const int32_t *q_seq, const int32_t *q_len,
                             int max_len, const CacheView &cv, const int32_t *cand, int B,
                             int cand_rows, float *out, int64_t ld, hipStream_t st);

// score_mfma.hip: matrix-core scorer for H == 64 and bf16/fp8 caches.
bool score_mfma_supported(int qt_dt, int H, const CacheView &cv);
hipError_t launch_score_mfma(const void *q_tilde, int qt_dt, const float *w, const float *beta,
                             int n_q, int H, const int32_t *q_seq, const int32_t *q_len,
                             int max_len, const CacheView &cv, const int32_t *cand, int B,
                             int cand_rows, float *out, int64_t ld, hipStream_t st);

// score_scan.hip: full-scan decode scorer for a bf16 cache, H == 64,
// r == 256 and at most 64 queries (page mode), one workgroup per CU.
bool score_scan_supported(int qt_dt, int H, int n_q, int max_len, const CacheView &cv);
// hist (may be null): [n_q][4096] row histograms of the order-preserving
// score keys (bin = key >> 20), added to; zbuf[0 .. zwords) is zeroed.
hipError_t launch_score_scan(const void *q_tilde, int qt_dt, const float *w, const float *beta,
                             int n_q, const int32_t *q_seq, const int32_t *q_len, int max_len,
                             const CacheView &cv, float *out, int64_t ld, hipStream_t st,
                             uint32_t *hist = nullptr, uint32_t *zbuf = nullptr, int zwords = 0);
// The same kernel in candidate mode (HS followers): query i scores the B
// slots of candidate list i % cand_rows into out[i*ld + j], -inf on padding.
bool score_scan_cand_supported(int qt_dt, int H, int n_q, int B, int cand_rows,
                               const CacheView &cv);
hipError_t launch_score_scan_cand(const void *q_tilde, int qt_dt, const float *w,
                                  const float *beta, int n_q, const int32_t *q_seq,
                                  const CacheView &cv, const int32_t *cand, int B, int cand_rows,
                                  float *out, int64_t ld, hipStream_t st);

// score_prefill.hip: matrix-core scorer for many bf16 queries per sequence
// (a prefill chunk), page mode only.
bool score_prefill_supported(int qt_dt, int H, int n_q, const CacheView &cv);
hipError_t launch_score_prefill(const void *q_tilde, const float *w, const float *beta, int n_q,
                                const int32_t *q_seq, const int32_t *q_len, int max_len,
                                const CacheView &cv, float *out, int64_t ld, hipStream_t st);

// topk.hip.  `ids` (may be null) maps a row position j to the id reported
// for it (row i uses ids + (i % ids_rows)*ids_ld); positions are ordered by id exactly as
// by j (ids ascending), so ties break by position.  valid_len may be null
// when every row is valid on [0, max_len) and max_len <= 16384.
size_t topk_ws_bytes(int n_rows, int max_len, int k);
hipError_t launch_topk(const float *scores, int64_t ld, int n_rows, const int32_t *valid_len,
                       const int32_t *ids, int64_t ids_ld, int ids_rows, int max_len, int k,
                       int32_t *out_idx,
                       float *out_val, void *ws, hipStream_t st);
// Rows of at most this many positions are selected by one workgroup per row
// in a single launch (no workspace), which beats the two launches of the
// nested multi-workgroup pass there.
int topk_single_max();
// The single-workgroup selection of rows of at most topk_single_max()
// positions (max_len), writing besides the top-k of each row the list of all
// its positions, -1 padded to all_k >= max_len (a selection whose size
// covers the row).
hipError_t launch_topk_with_all(const float *scores, int64_t ld, int n_rows,
                                const int32_t *valid_len, int max_len, int k, int32_t *out_idx,
                                int all_k, int32_t *all_idx, hipStream_t st);

// Two nested selections (k_outer >= k_inner) in one pass; ws of
// topk2_ws_bytes(n_rows, max_len) bytes; rows of at most topk2_max_len()
// positions.
size_t topk2_ws_bytes(int n_rows, int max_len);
int64_t topk2_max_len();
hipError_t launch_topk2(const float *scores, int64_t ld, int n_rows, const int32_t *valid_len,
                        int max_len, int k_outer, int32_t *out_outer, int k_inner,
                        int32_t *out_inner, void *ws, hipStream_t st);
// The anchor path whose scorer builds the row histograms itself (n_rows <= 64
// and a workspace kept zeroed as li_hs_anchor_select requires): where the row
// histograms go in ws (zero on entry), and the second-level histograms the
// scorer must zero; then the selection without its histogram step.
void topk2_count_arrays(void *ws, int n_rows, int max_len, uint32_t **hist, uint32_t **h10,
                        int *h10_words);
int topk2_counted_max_rows();
hipError_t launch_topk2_counted(const float *scores, int64_t ld, int n_rows, const int32_t *valid_len,
                                int max_len, int k_outer, int32_t *out_outer, int k_inner,
                                int32_t *out_inner, void *ws, hipStream_t st);

// calib.hip: normal equations of the calibration (G_xx = X^T X, G_xy = X^T Y,
// column sums), written or added to.
hipError_t launch_calib_gram(const void *X, int x_bf16, int64_t n, int d, const void *Y,
                             int y_bf16, int e, float *G_xx, float *G_xy, float *x_sum,
                             float *y_sum, int accumulate, hipStream_t st);

// Fill n int32 values with v (device).
hipError_t launch_fill_i32(int32_t *dst, int n, int32_t v, hipStream_t st);

}  // namespace li
