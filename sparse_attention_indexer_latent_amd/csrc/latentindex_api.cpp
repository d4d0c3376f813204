// C ABI of the LatentIndex indexer: argument validation on the host, device
// architecture check, and dispatch to the kernel launchers.  Nothing here
// allocates, frees or synchronises device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/latentindex.h"
#include "li_internal.h"

namespace {

thread_local std::string g_err;

li_status fail(li_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

li_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return LI_OK;
  return fail(LI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxDev = 64;
std::mutex g_dev_mu;
int g_dev_state[kMaxDev];  // 0 unknown, 1 gfx950, 2 other

li_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDev) return fail(LI_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDeviceProperties");
    g_dev_state[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
  }
  if (g_dev_state[dev] != 1) return fail(LI_ERR_UNSUPPORTED, "device %d is not a gfx950", dev);
  return LI_OK;
}

bool dtype_ok(int d) { return d == LI_FP32 || d == LI_BF16 || d == LI_FP8_E4M3; }

li_status check_cache(const li_cache *c, bool writable) {
  if (!c) return fail(LI_ERR_INVALID, "cache is NULL");
  if (!c->data || !c->block_table) return fail(LI_ERR_INVALID, "cache data/block_table is NULL");
  if (!dtype_ok(c->dtype)) return fail(LI_ERR_INVALID, "cache dtype %d unknown", (int)c->dtype);
  if (c->block_size != 64) return fail(LI_ERR_UNSUPPORTED, "block_size %d (only 64)", c->block_size);
  if (c->r <= 0 || c->r > 1024) return fail(LI_ERR_INVALID, "r = %d out of range", c->r);
  if (c->r % 16) return fail(LI_ERR_UNSUPPORTED, "r = %d not a multiple of 16", c->r);
  if (c->n_seq <= 0 || c->max_blocks <= 0 || c->n_blocks <= 0)
    return fail(LI_ERR_INVALID, "cache n_seq/max_blocks/n_blocks must be positive");
  if ((c->dtype == LI_FP8_E4M3) != (c->scale != nullptr))
    return fail(LI_ERR_INVALID, "scale must be given exactly for an FP8 cache");
  if (c->scale_block != 0 && !(c->dtype == LI_FP8_E4M3 && c->scale_block == 128))
    return fail(LI_ERR_INVALID, "scale_block %d: 0, or 128 for an FP8 cache", c->scale_block);
  (void)writable;
  return LI_OK;
}

}  // namespace

namespace li {

struct DeviceOnce {
  std::mutex mu;
  bool done[kMaxDev] = {};
};

DeviceOnce *device_once_new() { return new DeviceOnce(); }  // one per kernel, kept for the process

hipError_t raise_lds_limit(DeviceOnce *once, const void *fn, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(once->mu);
  if (!once->done[dev]) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    once->done[dev] = true;
  }
  return hipSuccess;
}

namespace {
std::atomic<int> g_cu[kMaxDev];
}

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 256;
  int n = g_cu[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    g_cu[dev].store(n, std::memory_order_relaxed);  // every thread stores the same value
  }
  return n;
}

}  // namespace li

extern "C" {

const char *li_last_error(void) { return g_err.c_str(); }

li_status li_check_device(void) { return check_device(); }

size_t li_append_workspace_bytes(int32_t n_tok, int32_t d_model, int32_t r, int32_t has_P) {
  if (n_tok <= 0 || d_model <= 0 || r <= 0) return 0;
  return li::append_ws_bytes(n_tok, d_model, r, has_P != 0);
}

}  // extern "C"

// Argument checks shared by li_append_latent and li_append_absorb (pointers
// only when n_tok > 0).
static li_status check_append_args(const void *x, li_dtype x_dt, int32_t n_tok, int32_t d_model,
                                   const void *P, const float *rope_theta, int32_t r_R,
                                   const int32_t *seq_idx, const int32_t *pos,
                                   const li_cache *cache) {
  li_status s = check_cache(cache, true);
  if (s != LI_OK) return s;
  if (n_tok < 0) return fail(LI_ERR_INVALID, "n_tok < 0");
  if (x_dt != LI_FP32 && x_dt != LI_BF16) return fail(LI_ERR_INVALID, "x dtype must be FP32 or BF16");
  if (d_model <= 0 || d_model > (1 << 20)) return fail(LI_ERR_INVALID, "d_model = %d out of range", d_model);
  if (!P && d_model != cache->r) return fail(LI_ERR_INVALID, "P is NULL but d_model (%d) != r (%d)", d_model, cache->r);
  if (r_R < 0 || r_R > cache->r || (r_R & 1)) return fail(LI_ERR_INVALID, "r_R = %d must be even and in [0, r]", r_R);
  if ((r_R > 0) != (rope_theta != nullptr)) return fail(LI_ERR_INVALID, "rope_theta must be given exactly when r_R > 0");
  if (n_tok > 0 && (!x || !seq_idx || !pos)) return fail(LI_ERR_INVALID, "x/seq_idx/pos is NULL");
  return LI_OK;
}

// Argument checks shared by li_absorb_queries and li_append_absorb.
static li_status check_absorb_args(const void *q, li_dtype q_dt, int32_t n_layers, int32_t n_q,
                                   int32_t H, int32_t d_I, const float *Dt,
                                   int64_t Dt_head_stride, int32_t nope_off, int32_t r,
                                   const float *q_tilde) {
  if (q_dt != LI_FP32 && q_dt != LI_BF16) return fail(LI_ERR_INVALID, "q dtype must be FP32 or BF16");
  if (n_layers < 1 || n_layers > 64) return fail(LI_ERR_INVALID, "n_layers = %d out of [1, 64]", n_layers);
  if (n_q < 0) return fail(LI_ERR_INVALID, "n_q < 0");
  if (H <= 0 || H > 1024 || d_I <= 0 || d_I > 1024 || r <= 0 || r > 1024)
    return fail(LI_ERR_INVALID, "H/d_I/r out of range (1..1024)");
  if (nope_off < 0 || nope_off > d_I) return fail(LI_ERR_INVALID, "nope_off out of [0, d_I]");
  if (Dt_head_stride < 0) return fail(LI_ERR_INVALID, "Dt_head_stride < 0");
  if (d_I % 4 || Dt_head_stride % 4) return fail(LI_ERR_UNSUPPORTED, "d_I and Dt_head_stride must be multiples of 4");
  if (n_q > 0 && (!q || !Dt || !q_tilde)) return fail(LI_ERR_INVALID, "q/Dt/q_tilde is NULL");
  return LI_OK;
}

extern "C" {

li_status li_append_latent(const void *x, li_dtype x_dt, int32_t n_tok, int32_t d_model,
                           const void *P, const float *rope_theta, int32_t r_R,
                           const int32_t *seq_idx, const int32_t *pos, const li_cache *cache,
                           void *ws, size_t ws_bytes, void *stream) {
  li_status s = check_append_args(x, x_dt, n_tok, d_model, P, rope_theta, r_R, seq_idx, pos, cache);
  if (s != LI_OK) return s;
  if (n_tok == 0) return LI_OK;
  size_t need = li::append_ws_bytes(n_tok, d_model, cache->r, P != nullptr);
  if (need && (!ws || ws_bytes < need)) return fail(LI_ERR_INVALID, "workspace needs %zu bytes", need);
  if ((s = check_device()) != LI_OK) return s;
  return hip_status(li::launch_append(x, x_dt, n_tok, d_model, P, rope_theta, r_R, seq_idx, pos,
                                      *cache, ws, (hipStream_t)stream),
                    "li_append_latent launch");
}

li_status li_absorb_queries(const void *q, li_dtype q_dt, int32_t n_layers, int32_t n_q,
                            int32_t H, int32_t d_I, const float *Dt, int64_t Dt_head_stride,
                            const float *b, int32_t nope_off, int32_t r, float *q_tilde,
                            float *beta, void *stream) {
  li_status s = check_absorb_args(q, q_dt, n_layers, n_q, H, d_I, Dt, Dt_head_stride, nope_off, r,
                                  q_tilde);
  if (s != LI_OK || n_q == 0) return s;
  if ((s = check_device()) != LI_OK) return s;
  return hip_status(li::launch_absorb(q, q_dt, n_layers, n_q, H, d_I, Dt, Dt_head_stride, b, nope_off, r,
                                      q_tilde, beta, (hipStream_t)stream),
                    "li_absorb_queries launch");
}

li_status li_append_absorb(const void *x, li_dtype x_dt, int32_t n_tok, const float *rope_theta,
                           int32_t r_R, const int32_t *seq_idx, const int32_t *pos,
                           const li_cache *cache, const void *q, li_dtype q_dt, int32_t n_layers,
                           int32_t n_q, int32_t H, int32_t d_I, const float *Dt,
                           int64_t Dt_head_stride, const float *b, int32_t nope_off,
                           float *q_tilde, float *beta, void *stream) {
  li_status s = check_append_args(x, x_dt, n_tok, cache ? cache->r : 1, nullptr, rope_theta, r_R,
                                   seq_idx, pos, cache);
  if (s != LI_OK) return s;
  if ((s = check_absorb_args(q, q_dt, n_layers, n_q, H, d_I, Dt, Dt_head_stride, nope_off,
                             cache->r, q_tilde)) != LI_OK)
    return s;
  if (n_tok == 0 && n_q == 0) return LI_OK;
  if ((s = check_device()) != LI_OK) return s;
  return hip_status(li::launch_append_absorb(x, x_dt, n_tok, rope_theta, r_R, seq_idx, pos, *cache,
                                             q, q_dt, n_layers, n_q, H, d_I, Dt, Dt_head_stride,
                                             b, nope_off, q_tilde, beta, (hipStream_t)stream),
                    "li_append_absorb launch");
}

static li_status check_score_args(const void *q_tilde, li_dtype qt_dt, const float *w, int32_t n_q,
                                  int32_t H, const int32_t *q_seq, const li_cache *cache) {
  li_status s = check_cache(cache, false);
  if (s != LI_OK) return s;
  if (qt_dt != LI_FP32 && qt_dt != LI_BF16) return fail(LI_ERR_INVALID, "q_tilde dtype must be FP32 or BF16");
  if (n_q < 0) return fail(LI_ERR_INVALID, "n_q < 0");
  if (H <= 0 || H > 1024) return fail(LI_ERR_INVALID, "H = %d out of range", H);
  if ((int64_t)H * cache->r > 16384) return fail(LI_ERR_UNSUPPORTED, "H * r = %d exceeds 16384", H * cache->r);
  if (n_q > 0 && (!q_tilde || !w || !q_seq)) return fail(LI_ERR_INVALID, "q_tilde/w/q_seq is NULL");
  return LI_OK;
}

li_status li_score(const void *q_tilde, li_dtype qt_dt, const float *w, const float *beta,
                   int32_t n_q, int32_t H, const int32_t *q_seq, const int32_t *q_len,
                   int32_t max_len, const li_cache *cache, float *scores, int64_t ld,
                   void *stream) {
  li_status s = check_score_args(q_tilde, qt_dt, w, n_q, H, q_seq, cache);
  if (s != LI_OK) return s;
  if (max_len < 0 || (int64_t)max_len > ld) return fail(LI_ERR_INVALID, "need 0 <= max_len <= ld");
  if ((int64_t)max_len > (int64_t)cache->max_blocks * 64)
    return fail(LI_ERR_INVALID, "max_len %d exceeds the block table (%d blocks)", max_len, cache->max_blocks);
  if (n_q == 0 || max_len == 0) return LI_OK;
  if (!q_len || !scores) return fail(LI_ERR_INVALID, "q_len/scores is NULL");
  if ((s = check_device()) != LI_OK) return s;
  li::CacheView cv = li::view_of(*cache);
  hipError_t e;
  if (li::score_prefill_supported(qt_dt, H, n_q, cv))
    e = li::launch_score_prefill(q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, scores, ld,
                                 (hipStream_t)stream);
  else if (li::score_scan_supported(qt_dt, H, n_q, max_len, cv))
    e = li::launch_score_scan(q_tilde, qt_dt, w, beta, n_q, q_seq, q_len, max_len, cv, scores, ld,
                              (hipStream_t)stream);
  else if (li::score_mfma_supported(qt_dt, H, cv))
    e = li::launch_score_mfma(q_tilde, qt_dt, w, beta, n_q, H, q_seq, q_len, max_len, cv, nullptr,
                              0, 1, scores, ld, (hipStream_t)stream);
  else
    e = li::launch_score_valu(q_tilde, qt_dt, w, beta, n_q, H, q_seq, q_len, max_len, cv, nullptr,
                              0, 1, scores, ld, (hipStream_t)stream);
  return hip_status(e, "li_score launch");
}

size_t li_topk_workspace_bytes(int32_t n_rows, int32_t max_len, int32_t k) {
  if (n_rows <= 0 || max_len <= 0 || k <= 0) return 0;
  return li::topk_ws_bytes(n_rows, max_len, k);
}

li_status li_topk(const float *scores, int64_t ld, int32_t n_rows, const int32_t *valid_len,
                  int32_t max_len, int32_t k, int32_t *out_idx, float *out_val, void *ws,
                  size_t ws_bytes, void *stream) {
  if (n_rows < 0) return fail(LI_ERR_INVALID, "n_rows < 0");
  if (k <= 0 || k > 65536) return fail(LI_ERR_INVALID, "k = %d out of [1, 65536]", k);
  if (max_len < 0 || (int64_t)max_len > ld) return fail(LI_ERR_INVALID, "need 0 <= max_len <= ld");
  if (n_rows == 0) return LI_OK;
  if (!scores || !valid_len || !out_idx) return fail(LI_ERR_INVALID, "scores/valid_len/out_idx is NULL");
  size_t need = li::topk_ws_bytes(n_rows, max_len, k);
  if (need && (!ws || ws_bytes < need)) return fail(LI_ERR_INVALID, "workspace needs %zu bytes", need);
  li_status s = check_device();
  if (s != LI_OK) return s;
  return hip_status(li::launch_topk(scores, ld, n_rows, valid_len, nullptr, 0, 1, max_len, k, out_idx,
                                    out_val, ws, (hipStream_t)stream),
                    "li_topk launch");
}

size_t li_hs_anchor_workspace_bytes(int32_t n_rows, int32_t max_len) {
  // rows of at most topk_single_max() positions select without a workspace
  if (n_rows <= 0 || max_len <= li::topk_single_max()) return 0;
  return li::topk2_ws_bytes(n_rows, max_len);
}

li_status li_hs_anchor_select(const float *scores, int64_t ld, int32_t n_rows,
                              const int32_t *valid_len, int32_t max_len, int32_t B, int32_t *cand,
                              int32_t k, int32_t *sel, void *ws, size_t ws_bytes, void *stream) {
  if (n_rows < 0) return fail(LI_ERR_INVALID, "n_rows < 0");
  if (B <= 0 || B > 65536) return fail(LI_ERR_INVALID, "B = %d out of [1, 65536]", B);
  if (k <= 0) return fail(LI_ERR_INVALID, "k = %d must be positive", k);
  if (B < k) return fail(LI_ERR_INVALID, "B (%d) < k (%d): the candidate set must hold k", B, k);
  if (max_len < 0 || (int64_t)max_len > ld) return fail(LI_ERR_INVALID, "need 0 <= max_len <= ld");
  if ((int64_t)max_len > li::topk2_max_len())
    return fail(LI_ERR_UNSUPPORTED, "max_len %d exceeds %lld positions per row", max_len,
                (long long)li::topk2_max_len());
  if (n_rows == 0) return LI_OK;
  if (!scores || !valid_len || !cand) return fail(LI_ERR_INVALID, "scores/valid_len/cand is NULL");
  size_t need = li_hs_anchor_workspace_bytes(n_rows, max_len);
  if (need && (!ws || ws_bytes < need)) return fail(LI_ERR_INVALID, "workspace needs %zu bytes", need);
  li_status s = check_device();
  if (s != LI_OK) return s;
  if (max_len <= li::topk_single_max()) {
    // short rows: one single-workgroup launch per selection; where B covers
    // the row, C is the row's positions in order and comes with S's launch
    if (sel && B >= max_len)
      return hip_status(li::launch_topk_with_all(scores, ld, n_rows, valid_len, max_len, k, sel, B,
                                                 cand, (hipStream_t)stream),
                        "li_hs_anchor_select launch");
    hipError_t e = li::launch_topk(scores, ld, n_rows, valid_len, nullptr, 0, 1, max_len, B, cand,
                                   nullptr, nullptr, (hipStream_t)stream);
    if (e == hipSuccess && sel)
      e = li::launch_topk(scores, ld, n_rows, valid_len, nullptr, 0, 1, max_len, k, sel, nullptr,
                          nullptr, (hipStream_t)stream);
    return hip_status(e, "li_hs_anchor_select launch");
  }
  hipError_t e = sel ? li::launch_topk2(scores, ld, n_rows, valid_len, max_len > 0 ? max_len : 1, B,
                                        cand, k, sel, ws, (hipStream_t)stream)
                     : li::launch_topk2(scores, ld, n_rows, valid_len, max_len > 0 ? max_len : 1, B,
                                        cand, B, cand, ws, (hipStream_t)stream);
  return hip_status(e, "li_hs_anchor_select launch");
}

li_status li_hs_anchor(const void *q_tilde, li_dtype qt_dt, const float *w, const float *beta,
                       int32_t n_q, int32_t H, const int32_t *q_seq, const int32_t *q_len,
                       int32_t max_len, const li_cache *cache, float *scores, int64_t ld,
                       int32_t B, int32_t *cand, int32_t k, int32_t *sel, void *ws, size_t ws_bytes,
                       void *const *scan_events, void *stream) {
  li_status s = check_score_args(q_tilde, qt_dt, w, n_q, H, q_seq, cache);
  if (s != LI_OK) return s;
  if (max_len < 0 || (int64_t)max_len > ld) return fail(LI_ERR_INVALID, "need 0 <= max_len <= ld");
  if ((int64_t)max_len > (int64_t)cache->max_blocks * 64)
    return fail(LI_ERR_INVALID, "max_len %d exceeds the block table (%d blocks)", max_len, cache->max_blocks);
  if (B <= 0 || B > 65536) return fail(LI_ERR_INVALID, "B = %d out of [1, 65536]", B);
  if (k <= 0) return fail(LI_ERR_INVALID, "k = %d must be positive", k);
  if (B < k) return fail(LI_ERR_INVALID, "B (%d) < k (%d): the candidate set must hold k", B, k);
  if ((int64_t)max_len > li::topk2_max_len())
    return fail(LI_ERR_UNSUPPORTED, "max_len %d exceeds %lld positions per row", max_len,
                (long long)li::topk2_max_len());
  if (n_q == 0) return LI_OK;
  if (!q_len || !scores || !cand) return fail(LI_ERR_INVALID, "q_len/scores/cand is NULL");
  size_t need = li_hs_anchor_workspace_bytes(n_q, max_len);
  if (need && (!ws || ws_bytes < need)) return fail(LI_ERR_INVALID, "workspace needs %zu bytes", need);
  if ((s = check_device()) != LI_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  li::CacheView cv = li::view_of(*cache);
  // (short rows take the single-workgroup selection, which needs no histograms)
  const bool fused = max_len > li::topk_single_max() &&
                     !li::score_prefill_supported(qt_dt, H, n_q, cv) &&
                     li::score_scan_supported(qt_dt, H, n_q, max_len, cv) &&
                     n_q <= li::topk2_counted_max_rows();
  auto record = [&](int i) {
    return scan_events ? hipEventRecord((hipEvent_t)scan_events[i], st) : hipSuccess;
  };
  if (!fused) {
    hipError_t e = record(0);
    if (e != hipSuccess) return hip_status(e, "li_hs_anchor event");
    if ((s = li_score(q_tilde, qt_dt, w, beta, n_q, H, q_seq, q_len, max_len, cache, scores, ld,
                      stream)) != LI_OK)
      return s;
    if ((e = record(1)) != hipSuccess) return hip_status(e, "li_hs_anchor event");
    return li_hs_anchor_select(scores, ld, n_q, q_len, max_len, B, cand, k, sel, ws, ws_bytes,
                               stream);
  }
  uint32_t *hist, *h10;
  int h10_words;
  li::topk2_count_arrays(ws, n_q, max_len, &hist, &h10, &h10_words);
  hipError_t e = record(0);
  if (e == hipSuccess)
    e = li::launch_score_scan(q_tilde, qt_dt, w, beta, n_q, q_seq, q_len, max_len, cv, scores, ld,
                              st, hist, h10, h10_words);
  if (e == hipSuccess) e = record(1);
  if (e == hipSuccess)
    e = sel ? li::launch_topk2_counted(scores, ld, n_q, q_len, max_len, B, cand, k, sel, ws, st)
            : li::launch_topk2_counted(scores, ld, n_q, q_len, max_len, B, cand, B, cand, ws, st);
  return hip_status(e, "li_hs_anchor launch");
}

li_status li_score_topk(const void *q_tilde, li_dtype qt_dt, const float *w, const float *beta,
                        int32_t n_q, int32_t H, const int32_t *q_seq, const int32_t *q_len,
                        int32_t max_len, const li_cache *cache, float *scores, int64_t ld,
                        int32_t k, int32_t *out_idx, void *ws, size_t ws_bytes,
                        void *const *scan_events, void *stream) {
  if (k <= 0 || k > 65536) return fail(LI_ERR_INVALID, "k = %d out of [1, 65536]", k);
  // The anchor's nested selection with one level: its candidate set with
  // B = k is the layer's top-k.
  return li_hs_anchor(q_tilde, qt_dt, w, beta, n_q, H, q_seq, q_len, max_len, cache, scores, ld,
                      k, out_idx, k, nullptr, ws, ws_bytes, scan_events, stream);
}

li_status li_calib_gram(const void *X, li_dtype x_dt, int64_t n, int32_t d, const void *Y,
                        li_dtype y_dt, int32_t e, float *G_xx, float *G_xy, float *x_sum,
                        float *y_sum, int32_t accumulate, void *stream) {
  if (x_dt != LI_FP32 && x_dt != LI_BF16) return fail(LI_ERR_INVALID, "X dtype must be FP32 or BF16");
  if (n < 0) return fail(LI_ERR_INVALID, "n < 0");
  if (d < 1 || d > 65536) return fail(LI_ERR_INVALID, "d = %d out of [1, 65536]", d);
  if (!X && n > 0) return fail(LI_ERR_INVALID, "X is NULL");
  if (!G_xx) return fail(LI_ERR_INVALID, "G_xx is NULL");
  if (Y) {
    if (y_dt != LI_FP32 && y_dt != LI_BF16) return fail(LI_ERR_INVALID, "Y dtype must be FP32 or BF16");
    if (e < 1 || e > 65536) return fail(LI_ERR_INVALID, "e = %d out of [1, 65536]", e);
  } else if (G_xy || y_sum) {
    return fail(LI_ERR_INVALID, "G_xy / y_sum need Y");
  }
  li_status s = check_device();
  if (s != LI_OK) return s;
  return hip_status(li::launch_calib_gram(X, x_dt == LI_BF16, n, d, Y, y_dt == LI_BF16, e, G_xx,
                                          G_xy, x_sum, y_sum, accumulate, (hipStream_t)stream),
                    "li_calib_gram launch");
}

size_t li_hs_workspace_bytes(int32_t n_f, int32_t n_q, int32_t B, int32_t k) {
  if (n_f <= 0 || n_q <= 0 || B <= 0 || k <= 0) return 0;
  const int64_t rows = (int64_t)n_f * n_q;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al((size_t)rows * B * sizeof(float)) + al((size_t)rows * sizeof(int32_t)) +
         li::topk_ws_bytes((int)rows, B, k);
}

}  // extern "C"

// li_hs_select's argument checks (all but the workspace).
static li_status check_hs_select_args(const int32_t *cand, int32_t B, int32_t n_f,
                                      const void *q_tilde, li_dtype qt_dt, const float *w,
                                      int32_t n_q, int32_t H, const int32_t *q_seq,
                                      const li_cache *cache, int32_t k, const int32_t *out_idx) {
  li_status s = check_score_args(q_tilde, qt_dt, w, n_q, H, q_seq, cache);
  if (s != LI_OK) return s;
  if (B <= 0 || B > 65536) return fail(LI_ERR_INVALID, "B = %d out of [1, 65536]", B);
  if (n_f < 1 || n_f > 64) return fail(LI_ERR_INVALID, "n_f = %d out of [1, 64]", n_f);
  if (k <= 0) return fail(LI_ERR_INVALID, "k = %d must be positive", k);
  if (B < k) return fail(LI_ERR_INVALID, "B (%d) < k (%d): the candidate set must hold k", B, k);
  if ((int64_t)n_f * n_q > (1 << 20)) return fail(LI_ERR_INVALID, "n_f * n_q too large");
  if (n_q > 0 && (!cand || !out_idx)) return fail(LI_ERR_INVALID, "cand/out_idx is NULL");
  return LI_OK;
}

// li_hs_select's launches on a workspace of li_hs_workspace_bytes() bytes.
static li_status hs_select_on(const int32_t *cand, int32_t B, int32_t n_f, const void *q_tilde,
                              li_dtype qt_dt, const float *w, const float *beta, int32_t n_q,
                              int32_t H, const int32_t *q_seq, const li_cache *cache, int32_t k,
                              int32_t *out_idx, float *cand_scores, void *ws, void *stream) {
  const int rows = n_f * n_q;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char *p = (char *)ws;
  float *sc = (float *)p;
  p += al((size_t)rows * B * sizeof(float));
  int32_t *lens = (int32_t *)p;
  p += al((size_t)rows * sizeof(int32_t));
  void *tws = p;
  float *dst = cand_scores ? cand_scores : sc;
  hipStream_t st = (hipStream_t)stream;
  li::CacheView cv = li::view_of(*cache);
  // Rows are (follower, query) pairs, follower-major; row i reads query
  // i % n_q's candidate list.
  // 1. each follower's scores of every candidate slot (-inf on padding);
  // 2. each row's top-k over all B slots: padding ranks below every
  //    candidate and maps to id -1, so the output is the top-min(k, |C|)
  //    then -1 padding.
  hipError_t e;
  if (li::score_scan_cand_supported(qt_dt, H, rows, B, n_q, cv))
    e = li::launch_score_scan_cand(q_tilde, qt_dt, w, beta, rows, q_seq, cv, cand, B, n_q, dst, B,
                                   st);
  else if (li::score_mfma_supported(qt_dt, H, cv))
    e = li::launch_score_mfma(q_tilde, qt_dt, w, beta, rows, H, q_seq, nullptr, B, cv, cand, B,
                              n_q, dst, B, st);
  else
    e = li::launch_score_valu(q_tilde, qt_dt, w, beta, rows, H, q_seq, nullptr, B, cv, cand, B,
                              n_q, dst, B, st);
  const int32_t *vl = nullptr;
  if (e == hipSuccess && B > 16384) {  // the longer-row paths need per-row lengths
    e = li::launch_fill_i32(lens, rows, B, st);
    vl = lens;
  }
  if (e == hipSuccess)
    e = li::launch_topk(dst, B, rows, vl, cand, B, n_q, B, k, out_idx, nullptr, tws, st);
  return hip_status(e, "li_hs_select launch");
}

// li_hs_select_noalloc's workspace: a fixed array of device memory of this
// library, one per device, held until the process ends, for callers that
// cannot allocate.  Host code never takes the array's name as an address:
// each device's address comes from hipGetSymbolAddress, once, with that
// device current.  Every call on a device shares its array.
static __device__ __align__(256) char scratch[LI_HS_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDev];

li_status scratch_of_current_device(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDev) return fail(LI_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(LI_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LI_OK;
}
}  // namespace

extern "C" {

li_status li_hs_select(const int32_t *cand, int32_t B, int32_t n_f, const void *q_tilde,
                       li_dtype qt_dt, const float *w, const float *beta, int32_t n_q, int32_t H,
                       const int32_t *q_seq, const li_cache *cache, int32_t k, int32_t *out_idx,
                       float *cand_scores, void *ws, size_t ws_bytes, void *stream) {
  li_status s = check_hs_select_args(cand, B, n_f, q_tilde, qt_dt, w, n_q, H, q_seq, cache, k,
                                     out_idx);
  if (s != LI_OK || n_q == 0) return s;
  size_t need = li_hs_workspace_bytes(n_f, n_q, B, k);
  if (!ws || ws_bytes < need) return fail(LI_ERR_INVALID, "workspace needs %zu bytes", need);
  if ((s = check_device()) != LI_OK) return s;
  return hs_select_on(cand, B, n_f, q_tilde, qt_dt, w, beta, n_q, H, q_seq, cache, k, out_idx,
                      cand_scores, ws, stream);
}

li_status li_hs_select_noalloc(const int32_t *cand, int32_t B, int32_t n_f, const void *q_tilde,
                               li_dtype qt_dt, const float *w, const float *beta, int32_t n_q,
                               int32_t H, const int32_t *q_seq, const li_cache *cache, int32_t k,
                               int32_t *out_idx, float *cand_scores, void *stream) {
  li_status s = check_hs_select_args(cand, B, n_f, q_tilde, qt_dt, w, n_q, H, q_seq, cache, k,
                                     out_idx);
  if (s != LI_OK || n_q == 0) return s;
  const size_t need = li_hs_workspace_bytes(n_f, n_q, B, k);
  if (need > (size_t)LI_HS_NOALLOC_SCRATCH_BYTES)
    return fail(LI_ERR_UNSUPPORTED,
                "li_hs_select_noalloc: n_f = %d, n_q = %d, B = %d, k = %d need %zu bytes of "
                "scratch, more than its %zu",
                n_f, n_q, B, k, need, (size_t)LI_HS_NOALLOC_SCRATCH_BYTES);
  if ((s = check_device()) != LI_OK) return s;
  void *ws = nullptr;
  if ((s = scratch_of_current_device(&ws)) != LI_OK) return s;
  return hs_select_on(cand, B, n_f, q_tilde, qt_dt, w, beta, n_q, H, q_seq, cache, k, out_idx,
                      cand_scores, ws, stream);
}

}  // extern "C"
