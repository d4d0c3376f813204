// Per-row top-k selection (LatentIndex summary, "Methodology": each layer's
// S = TopK_{t in V}(u_t, min(k, |V|))), with the order (score desc, position
// asc) and ascending output.
//
// Radix select on order-preserving 32-bit keys, one workgroup of 1024
// threads per row:
//   1. histogram of the top 12 key bits over the row (LDS atomics); the bin
//      b1 holding the k-th largest key is found with a block suffix scan;
//   2. the row's keys in bin b1 are gathered into an LDS candidate list
//      (or, if more than kCap fall there, the next passes re-stream the row);
//   3. two 10-bit digits refine the exact k-th key theta, and the number of
//      keys equal to theta that must be taken (lowest positions first);
//   4. one ordered pass emits positions with key > theta, plus the first
//      `need_eq` positions with key == theta, via ballot/prefix compaction,
//      so ids come out ascending without a sort.
#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = 4096;
constexpr int kCap = 6144;
constexpr int kPer = 8;  // consecutive positions per thread in the emit pass

struct TopkShared {
  uint32_t hist[kBins];
  uint32_t ckey[kCap];
  int32_t cpos[kCap];
  uint32_t wtot[kWaves];
  uint32_t n_cand;
  uint32_t sel_bin;
  uint32_t sel_above;
  uint32_t sel_count;
};

// Inclusive block-wide prefix sum of one uint32 per thread.  Returns the
// exclusive prefix; *total gets the block sum.  Contains two barriers.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *wtot,
                                                         uint32_t *total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const uint32_t x = wave_incl_scan(v);
  if (lane == kWave - 1) wtot[wave] = x;
  lds_sync();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w2 = 0; w2 < kWaves; ++w2) {
    const uint32_t t = wtot[w2];
    before += (w2 < wave) ? t : 0u;
    all += t;
  }
  lds_sync();
  *total = all;
  return before + x - v;
}

// Given a histogram of `nb` bins (counts of keys per digit), find the digit
// holding the `need`-th largest key: the bin b with
// sum_{b' > b} hist[b'] < need <= sum_{b' >= b} hist[b'].
// Writes sel_bin, sel_above (the count above b) and sel_count (hist[b]).
__device__ void find_bin(TopkShared &sh, int nb, uint32_t need) {
  const int per = nb / kThreads;  // bins per thread, highest bins to thread 0
  const int top = nb - 1 - threadIdx.x * per;
  uint32_t s = 0;
  for (int e = 0; e < per; ++e) s += sh.hist[top - e];
  uint32_t total;
  uint32_t run = block_exclusive_scan(s, sh.wtot, &total);
  for (int e = 0; e < per; ++e) {
    const uint32_t c = sh.hist[top - e];
    if (run < need && need <= run + c) {
      sh.sel_bin = top - e;
      sh.sel_above = run;
      sh.sel_count = c;
    }
    run += c;
  }
  lds_sync();
}

__global__ void __launch_bounds__(kThreads)
topk_row_kernel(const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ valid_len,
                const int32_t *__restrict__ ids, int64_t ids_ld, int ids_rows, int k,
                int32_t *__restrict__ out_idx, float *__restrict__ out_val) {
  extern __shared__ __align__(16) unsigned char smem[];
  TopkShared &sh = *reinterpret_cast<TopkShared *>(smem);
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = valid_len[row];
  const float *u = scores + (int64_t)row * ld;
  const int32_t *idm = ids ? ids + (int64_t)(row % ids_rows) * ids_ld : nullptr;
  int32_t *oi = out_idx + (int64_t)row * k;
  float *ov = out_val ? out_val + (int64_t)row * k : nullptr;
  const int m = min(k, n);

  // padding
  for (int j = m + tid; j < k; j += kThreads) {
    oi[j] = -1;
    if (ov) ov[j] = -INFINITY;
  }
  if (n <= k) {
    for (int p = tid; p < n; p += kThreads) {
      oi[p] = idm ? idm[p] : p;
      if (ov) ov[p] = u[p];
    }
    return;
  }

  // 1. top-12-bit histogram
  for (int b = tid; b < kBins; b += kThreads) sh.hist[b] = 0;
  lds_sync();
  for (int p = tid; p < n; p += kThreads) atomicAdd(&sh.hist[score_key(u[p]) >> 20], 1u);
  lds_sync();
  find_bin(sh, kBins, (uint32_t)k);
  const uint32_t b1 = sh.sel_bin;
  uint32_t need = (uint32_t)k - sh.sel_above;  // keys to take from bin b1 (>= 1)
  const uint32_t n_b1 = sh.sel_count;
  const bool in_lds = n_b1 <= (uint32_t)kCap;

  // 2. gather bin b1 into the candidate list
  if (tid == 0) sh.n_cand = 0;
  lds_sync();
  if (in_lds) {
    for (int p = tid; p < n; p += kThreads) {
      const uint32_t key = score_key(u[p]);
      if ((key >> 20) == b1) {
        const uint32_t s = atomicAdd(&sh.n_cand, 1u);
        if (s < (uint32_t)kCap) {
          sh.ckey[s] = key;
          sh.cpos[s] = p;
        }
      }
    }
  }
  lds_sync();

  // 3. refine the low 20 bits: digit 2 = bits 19..10, digit 3 = bits 9..0
  uint32_t prefix = b1;  // key bits known so far, right-aligned
  int known = 12;        // number of known leading bits
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = 20 - 10 * (pass + 1);
    for (int b = tid; b < 1024; b += kThreads) sh.hist[b] = 0;
    lds_sync();
    if (in_lds) {
      const uint32_t nc = min(sh.n_cand, (uint32_t)kCap);
      for (uint32_t c = tid; c < nc; c += kThreads) {
        const uint32_t key = sh.ckey[c];
        if ((key >> (32 - known)) == prefix) atomicAdd(&sh.hist[(key >> shift) & 1023u], 1u);
      }
    } else {
      for (int p = tid; p < n; p += kThreads) {
        const uint32_t key = score_key(u[p]);
        if ((key >> (32 - known)) == prefix) atomicAdd(&sh.hist[(key >> shift) & 1023u], 1u);
      }
    }
    lds_sync();
    find_bin(sh, 1024, need);
    need -= sh.sel_above;
    prefix = (prefix << 10) | sh.sel_bin;
    known += 10;
  }
  const uint32_t theta = prefix;
  const uint32_t n_eq = sh.sel_count;  // keys equal to theta in the row
  const bool take_all_eq = need == n_eq;

  // 4. ordered emit
  uint32_t eq_carry = 0, sel_carry = 0;
  for (int base = 0; base < n && sel_carry < (uint32_t)m; base += kThreads * kPer) {
    const int p0 = base + tid * kPer;
    uint32_t key[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) key[e] = (p0 + e < n) ? score_key(u[p0 + e]) : 0u;
    uint32_t eq_before = 0;
    if (!take_all_eq) {
      uint32_t c_eq = 0;
#pragma unroll
      for (int e = 0; e < kPer; ++e) c_eq += (p0 + e < n && key[e] == theta) ? 1u : 0u;
      uint32_t tot;
      eq_before = eq_carry + block_exclusive_scan(c_eq, sh.wtot, &tot);
      eq_carry += tot;
    }
    bool sel[kPer];
    uint32_t c_sel = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const bool valid = p0 + e < n;
      const bool eq = valid && key[e] == theta;
      sel[e] = valid && (key[e] > theta || (eq && (take_all_eq || eq_before < need)));
      eq_before += eq ? 1u : 0u;
      c_sel += sel[e] ? 1u : 0u;
    }
    uint32_t tot;
    uint32_t pos = sel_carry + block_exclusive_scan(c_sel, sh.wtot, &tot);
    sel_carry += tot;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (sel[e] && pos < (uint32_t)m) {
        const int p = p0 + e;
        oi[pos] = idm ? idm[p] : p;
        if (ov) ov[pos] = u[p];
        ++pos;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Multi-workgroup path for few, long rows (decode: one row per query).
//   clear:    zero the per-row 4096-bin histogram in the workspace
//   hist:     one workgroup per 2048-element segment: LDS histogram of the
//             top 12 key bits, merged into the row histogram with atomics
//             (integer counts: the result does not depend on their order)
//   extract:  one workgroup per segment finds the bucket b1 of the largest
//             requested k from the row histogram and writes, in position
//             order, every (key, position) with top-12 bits >= b1
//   finalize: one workgroup per row gathers the extracted lists (about
//             k + one bucket entries) into LDS, refines the exact k-th key
//             for each requested k and emits ascending positions.
// ---------------------------------------------------------------------------

constexpr int kSeg = 2048;
constexpr int kSegThreads = 256;
constexpr int kSegPer = kSeg / kSegThreads;  // 8 consecutive positions per thread
constexpr int kFinCap = 12288;               // LDS list capacity of the finalize step
constexpr int kMaxSegs = 1024;

struct MultiWs {
  uint32_t *hist;     // [n_rows][kBins]
  uint32_t *seg_cnt;  // [n_rows][S]
  uint2 *list;        // [n_rows][S][kSeg]  (key, position)
  int S;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

MultiWs carve(void *ws, int n_rows, int max_len) {
  MultiWs m;
  m.S = (max_len + kSeg - 1) / kSeg;
  char *p = (char *)ws;
  m.hist = (uint32_t *)p;
  p += align256((size_t)n_rows * kBins * 4);
  m.seg_cnt = (uint32_t *)p;
  p += align256((size_t)n_rows * m.S * 4);
  m.list = (uint2 *)p;
  return m;
}

size_t multi_ws_bytes(int n_rows, int max_len) {
  const size_t S = (max_len + kSeg - 1) / kSeg;
  return align256((size_t)n_rows * kBins * 4) + align256((size_t)n_rows * S * 4) +
         (size_t)n_rows * S * kSeg * sizeof(uint2);
}

bool use_multi(int n_rows, int max_len) {
  return n_rows <= 64 && max_len >= 4096 && (max_len + kSeg - 1) / kSeg <= kMaxSegs;
}

__global__ void __launch_bounds__(256) topk_clear_kernel(uint32_t *__restrict__ hist, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) hist[i] = 0;
}

__global__ void __launch_bounds__(kSegThreads)
topk_hist_kernel(const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ valid_len,
                 uint32_t *__restrict__ hist) {
  __shared__ uint32_t h[kBins];
  const int row = blockIdx.y, seg = blockIdx.x, tid = threadIdx.x;
  const int n = valid_len[row];
  const int p0 = seg * kSeg;
  if (p0 >= n) return;
  const int p1 = min(n, p0 + kSeg);
  for (int b = tid; b < kBins; b += kSegThreads) h[b] = 0;
  lds_sync();
  const float *u = scores + (int64_t)row * ld;
  float v[kSegPer];
#pragma unroll
  for (int j = 0; j < kSegPer; ++j) {
    const int p = p0 + tid + j * kSegThreads;
    v[j] = p < p1 ? u[p] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kSegPer; ++j)
    if (p0 + tid + j * kSegThreads < p1) atomicAdd(&h[score_key(v[j]) >> 20], 1u);
  lds_sync();
  uint32_t *g = hist + (int64_t)row * kBins;
  for (int b = tid; b < kBins; b += kSegThreads)
    if (h[b]) atomicAdd(&g[b], h[b]);
}

// Block-wide exclusive scan for kSegThreads threads.
__device__ __forceinline__ uint32_t seg_scan(uint32_t v, uint32_t *wt, uint32_t *total) {
  constexpr int W = kSegThreads / kWave;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const uint32_t x = wave_incl_scan(v);
  if (lane == kWave - 1) wt[wave] = x;
  lds_sync();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w2 = 0; w2 < W; ++w2) {
    before += (w2 < wave) ? wt[w2] : 0u;
    all += wt[w2];
  }
  lds_sync();
  *total = all;
  return before + x - v;
}

__global__ void __launch_bounds__(kSegThreads)
topk_extract_kernel(const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ valid_len,
                    int kmax, MultiWs m) {
  __shared__ uint32_t wt[kSegThreads / kWave];
  __shared__ uint32_t s_b1;
  const int row = blockIdx.y, seg = blockIdx.x, tid = threadIdx.x;
  const int n = valid_len[row];
  const int p0 = seg * kSeg;
  if (p0 >= n) {
    if (tid == 0) m.seg_cnt[(int64_t)row * m.S + seg] = 0;
    return;
  }
  uint32_t b1 = 0;
  if (n > kmax) {
    // bucket of the kmax-th largest key: suffix scan of the row histogram,
    // highest bins first (16 per thread)
    const uint32_t *g = m.hist + (int64_t)row * kBins;
    constexpr int per = kBins / kSegThreads;
    const int top = kBins - 1 - tid * per;
    uint32_t c[per], sum = 0;
#pragma unroll
    for (int e = 0; e < per; ++e) {
      c[e] = g[top - e];
      sum += c[e];
    }
    uint32_t tot;
    uint32_t run = seg_scan(sum, wt, &tot);
#pragma unroll
    for (int e = 0; e < per; ++e) {
      if (run < (uint32_t)kmax && (uint32_t)kmax <= run + c[e]) s_b1 = top - e;
      run += c[e];
    }
    lds_sync();
    b1 = s_b1;
  }
  const float *u = scores + (int64_t)row * ld;
  const int pb = p0 + tid * kSegPer;
  uint32_t key[kSegPer];
  uint32_t cnt = 0;
#pragma unroll
  for (int e = 0; e < kSegPer; ++e) {
    const int p = pb + e;
    key[e] = p < n ? score_key(u[p]) : 0u;
    cnt += (p < n && (key[e] >> 20) >= b1) ? 1u : 0u;
  }
  uint32_t tot;
  uint32_t pos = seg_scan(cnt, wt, &tot);
  uint2 *out = m.list + ((int64_t)row * m.S + seg) * kSeg;
#pragma unroll
  for (int e = 0; e < kSegPer; ++e) {
    const int p = pb + e;
    if (p < n && (key[e] >> 20) >= b1) out[pos++] = make_uint2(key[e], (uint32_t)p);
  }
  if (tid == 0) m.seg_cnt[(int64_t)row * m.S + seg] = tot;
}

struct FinShared {
  uint32_t lkey[kFinCap];
  int32_t lpos[kFinCap];
  uint32_t hist[kBins];
  uint32_t hist12[kBins];  // the row's top-12-bit histogram, kept for every output
  uint32_t small[4096];
  uint32_t seg_off[kMaxSegs + 1];
  uint32_t wtot[kWaves];
  uint32_t sel_bin, sel_above, sel_count, n_small;
};

// Radix refinement of the `need`-th largest key among the entries given by
// `get(i)` for i < M.  Returns theta; *need_eq receives how many entries equal
// to theta are taken (lowest positions first), *all_eq whether that is all of
// them.
// Radix refinement of the `need`-th largest key among the entries get(i),
// i < M.  Pass 1 uses the 12-bit histogram in sh.hist when have_hist (it must
// agree with the entries' own on every bin from the need-th largest key up,
// e.g. the whole row's histogram when the entries are all keys at or above a
// bucket chosen for a larger k); otherwise it builds it.  The keys of the
// selected 12-bit bucket are then compacted into sh.small (when they fit) so
// the two 10-bit passes touch only that bucket.  Returns theta; *need_eq
// receives how many entries equal to theta are taken (lowest positions
// first), *all_eq whether that is all of them.  sh.hist is clobbered.
constexpr int kSmall = 4096;

template <typename SHT, typename Get>
__device__ uint32_t refine(SHT &sh, uint32_t M, uint32_t need, Get get, uint32_t *need_eq,
                           bool *all_eq, bool have_hist) {
  const int tid = threadIdx.x;
  auto find = [&](int nb, uint32_t nd) {  // bin of the nd-th largest (highest bins to thread 0)
    const int per = nb / kThreads;
    const int top = nb - 1 - tid * per;
    uint32_t sum = 0;
    for (int e = 0; e < per; ++e) sum += sh.hist[top - e];
    uint32_t total;
    uint32_t run = block_exclusive_scan(sum, sh.wtot, &total);
    for (int e = 0; e < per; ++e) {
      const uint32_t c = sh.hist[top - e];
      if (run < nd && nd <= run + c) {
        sh.sel_bin = top - e;
        sh.sel_above = run;
        sh.sel_count = c;
      }
      run += c;
    }
    lds_sync();
  };
  // pass 1: top 12 bits
  constexpr int RB = 8;  // entries per thread per batch: reads issued before the atomics
  if (!have_hist) {
    for (int b = tid; b < kBins; b += kThreads) sh.hist[b] = 0;
    lds_sync();
    for (uint32_t base = 0; base < M; base += kThreads * RB) {
      uint32_t key[RB];
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const uint32_t i = base + j * kThreads + tid;
        key[j] = i < M ? get(i).x : 0u;
      }
#pragma unroll
      for (int j = 0; j < RB; ++j)
        if (base + j * kThreads + tid < M) atomicAdd(&sh.hist[key[j] >> 20], 1u);
    }
    lds_sync();
  }
  find(kBins, need);
  need -= sh.sel_above;
  uint32_t prefix = sh.sel_bin;
  const uint32_t n_bucket = sh.sel_count;
  lds_sync();
  // compact the bucket's keys (any order: only counts are taken from them)
  const bool small = n_bucket <= (uint32_t)kSmall;
  if (small) {
    if (tid == 0) sh.n_small = 0;
    lds_sync();
    for (uint32_t base = 0; base < M; base += kThreads * RB) {
      uint32_t key[RB];
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const uint32_t i = base + j * kThreads + tid;
        key[j] = i < M ? get(i).x : 0u;
      }
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        if (base + j * kThreads + tid < M && (key[j] >> 20) == prefix) {
          const uint32_t slot = atomicAdd(&sh.n_small, 1u);
          if (slot < (uint32_t)kSmall) sh.small[slot] = key[j];
        }
      }
    }
    lds_sync();
  }
  const uint32_t ns = small ? n_bucket : M;
  int known = 12;
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = 32 - known - 10;
    for (int b = tid; b < 1024; b += kThreads) sh.hist[b] = 0;
    lds_sync();
    for (uint32_t base = 0; base < ns; base += kThreads * RB) {
      uint32_t key[RB];
#pragma unroll
      for (int j = 0; j < RB; ++j) {
        const uint32_t i = base + j * kThreads + tid;
        key[j] = i < ns ? (small ? sh.small[i] : get(i).x) : 0u;
      }
#pragma unroll
      for (int j = 0; j < RB; ++j)
        if (base + j * kThreads + tid < ns && (key[j] >> (32 - known)) == prefix)
          atomicAdd(&sh.hist[(key[j] >> shift) & 1023u], 1u);
    }
    lds_sync();
    find(1024, need);
    need -= sh.sel_above;
    prefix = (prefix << 10) | sh.sel_bin;
    known += 10;
    lds_sync();
  }
  *need_eq = need;
  *all_eq = need == sh.sel_count;
  return prefix;
}

// Ordered emit over entries get(i), i < M (ascending positions): entries with
// key > theta, then the first need_eq entries equal to theta.  Each thread
// takes kPer consecutive entries per round, so one round covers 8192 entries.
template <typename SHT, typename Get>
__device__ void emit(SHT &sh, uint32_t M, uint32_t theta, uint32_t need_eq, bool all_eq,
                     bool take_all, Get get, const int32_t *idm, const float *u, int32_t *oi,
                     float *ov, int m) {
  const int tid = threadIdx.x;
  uint32_t eq_carry = 0, sel_carry = 0;
  for (uint32_t base = 0; base < M && sel_carry < (uint32_t)m; base += kThreads * kPer) {
    const uint32_t i0 = base + tid * kPer;
    uint2 e[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) e[j] = (i0 + j < M) ? get(i0 + j) : make_uint2(0u, 0u);
    uint32_t eq_before = 0;
    if (!take_all && !all_eq) {
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) c += (i0 + j < M && e[j].x == theta) ? 1u : 0u;
      uint32_t tot;
      eq_before = eq_carry + block_exclusive_scan(c, sh.wtot, &tot);
      eq_carry += tot;
    }
    bool sel[kPer];
    uint32_t c_sel = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const bool valid = i0 + j < M;
      const bool eq = valid && e[j].x == theta;
      sel[j] = valid && (take_all || e[j].x > theta || (eq && (all_eq || eq_before < need_eq)));
      eq_before += eq ? 1u : 0u;
      c_sel += sel[j] ? 1u : 0u;
    }
    // ids and values of the selected entries, fetched before the scan so the
    // loads overlap it
    int32_t idv[kPer];
    float vv[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int p = (int)e[j].y;
      idv[j] = (sel[j] && idm) ? idm[p] : p;
      vv[j] = (sel[j] && ov) ? u[p] : 0.f;
    }
    uint32_t tot;
    uint32_t pos = sel_carry + block_exclusive_scan(c_sel, sh.wtot, &tot);
    sel_carry += tot;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (sel[j] && pos < (uint32_t)m) {
        oi[pos] = idv[j];
        if (ov) ov[pos] = vv[j];
        ++pos;
      }
    }
  }
}

struct FinOut {
  int k;
  int32_t *idx;
  float *val;
};

__global__ void __launch_bounds__(kThreads)
topk_finalize_kernel(const float *__restrict__ scores, int64_t ld,
                     const int32_t *__restrict__ valid_len, const int32_t *__restrict__ ids,
                     int64_t ids_ld, int ids_rows, FinOut o0, FinOut o1, int n_out, MultiWs m) {
  extern __shared__ __align__(16) unsigned char smem[];
  FinShared &sh = *reinterpret_cast<FinShared *>(smem);
  const int row = blockIdx.x, tid = threadIdx.x;
  const int n = valid_len[row];
  const int32_t *idm = ids ? ids + (int64_t)(row % ids_rows) * ids_ld : nullptr;
  const float *u = scores + (int64_t)row * ld;
  // padding of both outputs
  for (int j = 0; j < n_out; ++j) {
    const FinOut &o = j ? o1 : o0;
    const int mm = min(o.k, n);
    for (int t = mm + tid; t < o.k; t += kThreads) {
      o.idx[(int64_t)row * o.k + t] = -1;
      if (o.val) o.val[(int64_t)row * o.k + t] = -INFINITY;
    }
  }
  if (n <= 0) return;
  const int S = (n + kSeg - 1) / kSeg;
  const uint32_t *cnt = m.seg_cnt + (int64_t)row * m.S;
  // exclusive prefix of the segment counts (S <= kMaxSegs)
  uint32_t carry = 0;
  for (int b = 0; b < S; b += kThreads) {
    const uint32_t c = (b + tid < S) ? cnt[b + tid] : 0u;
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan(c, sh.wtot, &tot);
    if (b + tid < S) sh.seg_off[b + tid] = carry + ex;
    carry += tot;
  }
  if (tid == 0) sh.seg_off[S] = carry;
  lds_sync();
  const uint32_t M = carry;
  const uint2 *glist = m.list + (int64_t)row * m.S * kSeg;
  const bool in_lds = M <= (uint32_t)kFinCap;
  const uint32_t *g12 = m.hist + (int64_t)row * kBins;
  for (int b = tid; b < kBins; b += kThreads) sh.hist12[b] = g12[b];
  if (in_lds) {
    // flat copy in batches of 16 independent loads per thread, all in flight
    // at once (one round trip per batch instead of one per segment)
    constexpr int CP = 16;
    for (uint32_t base = 0; base < M; base += kThreads * CP) {
      uint2 v[CP];
#pragma unroll
      for (int j = 0; j < CP; ++j) {
        const uint32_t i = base + j * kThreads + tid;
        if (i < M) {
          int lo = 0;  // segment holding flat index i: fixed-step search (unrollable)
#pragma unroll
          for (int step = kMaxSegs / 2; step > 0; step >>= 1)
            if (lo + step < S && sh.seg_off[lo + step] <= i) lo += step;
          v[j] = glist[(int64_t)lo * kSeg + (i - sh.seg_off[lo])];
        }
      }
#pragma unroll
      for (int j = 0; j < CP; ++j) {
        const uint32_t i = base + j * kThreads + tid;
        if (i < M) {
          sh.lkey[i] = v[j].x;
          sh.lpos[i] = (int32_t)v[j].y;
        }
      }
    }
  }
  lds_sync();
  auto get_lds = [&](uint32_t i) { return make_uint2(sh.lkey[i], (uint32_t)sh.lpos[i]); };
  auto get_glb = [&](uint32_t i) {
    int lo = 0, hi = S - 1;  // segment holding flat index i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sh.seg_off[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return glist[(int64_t)lo * kSeg + (i - sh.seg_off[lo])];
  };
  for (int j = 0; j < n_out; ++j) {
    const FinOut &o = j ? o1 : o0;
    const int mm = min(o.k, n);
    int32_t *oi = o.idx + (int64_t)row * o.k;
    float *ov = o.val ? o.val + (int64_t)row * o.k : nullptr;
    const bool take_all = o.k >= n;  // then every element was extracted
    uint32_t theta = 0, need_eq = 0;
    bool all_eq = true;
    if (!take_all) {
      // pass 1 from the whole row's histogram (exact for every k <= kmax)
      for (int b = tid; b < kBins; b += kThreads) sh.hist[b] = sh.hist12[b];
      lds_sync();
      if (in_lds) theta = refine(sh, M, (uint32_t)o.k, get_lds, &need_eq, &all_eq, true);
      else theta = refine(sh, M, (uint32_t)o.k, get_glb, &need_eq, &all_eq, true);
    }
    if (in_lds) emit(sh, M, theta, need_eq, all_eq, take_all, get_lds, idm, u, oi, ov, mm);
    else emit(sh, M, theta, need_eq, all_eq, take_all, get_glb, idm, u, oi, ov, mm);
    lds_sync();
  }
}

// ---------------------------------------------------------------------------
// Rows of at most kLdsRow elements (e.g. a follower's candidate scores): one
// workgroup per row keeps the whole row's keys in LDS, so the three radix
// passes and the ordered emit touch global memory once.
// ---------------------------------------------------------------------------
constexpr int kLdsRow = 16384;

struct LdsRowShared {
  uint32_t key[kLdsRow];
  uint32_t hist[kBins];
  uint32_t small[4096];
  uint32_t wtot[kWaves];
  uint32_t sel_bin, sel_above, sel_count, n_small;
};

__global__ void __launch_bounds__(kThreads)
topk_lds_kernel(const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ valid_len,
                int const_len, const int32_t *__restrict__ ids, int64_t ids_ld, int ids_rows, int k,
                int32_t *__restrict__ out_idx, float *__restrict__ out_val) {
  extern __shared__ __align__(16) unsigned char smem[];
  LdsRowShared &sh = *reinterpret_cast<LdsRowShared *>(smem);
  const int row = blockIdx.x, tid = threadIdx.x;
  const int n = min(valid_len ? valid_len[row] : const_len, kLdsRow);
  const float *u = scores + (int64_t)row * ld;
  const int32_t *idm = ids ? ids + (int64_t)(row % ids_rows) * ids_ld : nullptr;
  int32_t *oi = out_idx + (int64_t)row * k;
  float *ov = out_val ? out_val + (int64_t)row * k : nullptr;
  const int m = min(k, n);
  for (int j = m + tid; j < k; j += kThreads) {
    oi[j] = -1;
    if (ov) ov[j] = -INFINITY;
  }
  if (n <= k) {
    for (int p = tid; p < n; p += kThreads) {
      oi[p] = idm ? idm[p] : p;
      if (ov) ov[p] = u[p];
    }
    return;
  }
  {
    constexpr int LB = kLdsRow / kThreads;  // all of a thread's loads in flight at once
    float v[LB];
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int p = tid + j * kThreads;
      v[j] = p < n ? u[p] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int p = tid + j * kThreads;
      if (p < n) sh.key[p] = score_key(v[j]);
    }
  }
  lds_sync();
  auto get = [&](uint32_t i) { return make_uint2(sh.key[i], i); };
  uint32_t need_eq = 0;
  bool all_eq = true;
  const uint32_t theta = refine(sh, (uint32_t)n, (uint32_t)k, get, &need_eq, &all_eq, false);
  emit(sh, (uint32_t)n, theta, need_eq, all_eq, false, get, idm, u, oi, ov, m);
}

hipError_t launch_multi(const float *scores, int64_t ld, int n_rows, const int32_t *valid_len,
                        const int32_t *ids, int64_t ids_ld, int ids_rows, int max_len, FinOut o0, FinOut o1,
                        int n_out, void *ws, hipStream_t st) {
  MultiWs m = carve(ws, n_rows, max_len);
  const int kmax = n_out == 2 ? max(o0.k, o1.k) : o0.k;
  const int nh = n_rows * kBins;
  topk_clear_kernel<<<(nh + 255) / 256, 256, 0, st>>>(m.hist, nh);
  dim3 g(m.S, n_rows);
  topk_hist_kernel<<<g, kSegThreads, 0, st>>>(scores, ld, valid_len, m.hist);
  topk_extract_kernel<<<g, kSegThreads, 0, st>>>(scores, ld, valid_len, kmax, m);
  const size_t lds = sizeof(FinShared);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void *)topk_finalize_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr_set = true;
  }
  topk_finalize_kernel<<<n_rows, kThreads, lds, st>>>(scores, ld, valid_len, ids, ids_ld, ids_rows, o0, o1,
                                                      n_out, m);
  return hipGetLastError();
}

}  // namespace

size_t topk_ws_bytes(int n_rows, int max_len, int) {
  return (max_len > kLdsRow && use_multi(n_rows, max_len)) ? multi_ws_bytes(n_rows, max_len) : 0;
}

hipError_t launch_topk(const float *scores, int64_t ld, int n_rows, const int32_t *valid_len,
                       const int32_t *ids, int64_t ids_ld, int ids_rows, int max_len, int k, int32_t *out_idx,
                       float *out_val, void *ws, hipStream_t st) {
  if (max_len <= kLdsRow) {
    const size_t lds = sizeof(LdsRowShared);
    static bool attr_lds = false;
    if (!attr_lds) {
      (void)hipFuncSetAttribute((const void *)topk_lds_kernel,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      attr_lds = true;
    }
    topk_lds_kernel<<<n_rows, kThreads, lds, st>>>(scores, ld, valid_len, max_len, ids, ids_ld, ids_rows, k,
                                                   out_idx, out_val);
    return hipGetLastError();
  }
  if (use_multi(n_rows, max_len))
    return launch_multi(scores, ld, n_rows, valid_len, ids, ids_ld, ids_rows, max_len,
                        FinOut{k, out_idx, out_val}, FinOut{0, nullptr, nullptr}, 1, ws, st);
  const size_t lds = sizeof(TopkShared);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void *)topk_row_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr_set = true;
  }
  topk_row_kernel<<<n_rows, kThreads, lds, st>>>(scores, ld, valid_len, ids, ids_ld, ids_rows, k, out_idx,
                                                 out_val);
  return hipGetLastError();
}

size_t topk2_ws_bytes(int n_rows, int max_len) { return multi_ws_bytes(n_rows, max_len); }

namespace {
__global__ void fill_i32_kernel(int32_t *__restrict__ dst, int n, int32_t v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = v;
}
}  // namespace

hipError_t launch_fill_i32(int32_t *dst, int n, int32_t v, hipStream_t st) {
  fill_i32_kernel<<<(n + 255) / 256, 256, 0, st>>>(dst, n, v);
  return hipGetLastError();
}

hipError_t launch_topk2(const float *scores, int64_t ld, int n_rows, const int32_t *valid_len,
                        int max_len, int k_outer, int32_t *out_outer, int k_inner,
                        int32_t *out_inner, void *ws, hipStream_t st) {
  return launch_multi(scores, ld, n_rows, valid_len, nullptr, 0, 1, max_len,
                      FinOut{k_outer, out_outer, nullptr}, FinOut{k_inner, out_inner, nullptr}, 2,
                      ws, st);
}

}  // namespace li
