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
  __align__(16) uint32_t hist[kBins];
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
  const int n = max(valid_len[row], 0);
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
//   clear:   zero the per-row histograms in the workspace
//   hist:    one workgroup per 2048-element segment: LDS histogram of the
//            top 12 key bits, merged into the row histogram with atomics
//            (integer counts: the result does not depend on their order)
//   extract: one workgroup per segment finds, from the row histogram, the
//            12-bit bucket of each requested k; writes, in position order,
//            every (key, position) at or above the bucket of the largest k;
//            and counts the keys of each threshold bucket into a global
//            histogram of their next 10 bits
//   select:  one workgroup per segment derives the exact thresholds, its
//            output offset and emits its own selected positions (below).
// ---------------------------------------------------------------------------

constexpr int kSeg = 2048;
constexpr int kSegThreads = 256;
constexpr int kSegPer = kSeg / kSegThreads;  // 8 consecutive positions per thread
constexpr int kMaxSegs = 1024;

// Workspace of the many-row path.  The row histograms must be zero when a
// call starts; nothing reads them after the extract step, so the select step
// zeroes them again (each workgroup a slice of its row), and a workspace that
// starts zeroed needs no clearing launch.  For up to kHeadRows rows they sit
// at a fixed offset at the front (the same place whatever n_rows and
// max_len); beyond that they follow and every call clears them.  The
// second-level histograms are zeroed by the histogram step of the same call
// (the select step of the previous call has read them by then).
constexpr int kHeadRows = 64;

struct MultiWs {
  uint32_t *hist;     // [n_rows][kBins]
  uint32_t *h10;      // [n_rows][2][1024]: next 10 bits of each output's threshold bucket
  uint32_t *bsel;     // [n_rows][2][2]: each output's 12-bit bucket and the count above it
  uint32_t *seg_cnt;  // [n_rows][S]
  uint32_t *lkey;     // [n_rows][S][kSeg]
  int32_t *lpos;      // [n_rows][S][kSeg]
  int S;
  int max_len;        // allocated length of every score row (bounds speculative loads)
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline size_t hist_bytes(int n) { return (size_t)n * kBins * 4; }

MultiWs carve(void *ws, int n_rows, int max_len) {
  MultiWs m;
  m.S = (max_len + kSeg - 1) / kSeg;
  m.max_len = max_len;
  char *p = (char *)ws;
  m.hist = (uint32_t *)(n_rows <= kHeadRows ? p : p + hist_bytes(kHeadRows));
  p += hist_bytes(kHeadRows) + (n_rows <= kHeadRows ? 0 : hist_bytes(n_rows));
  m.h10 = (uint32_t *)p;
  p += align256((size_t)n_rows * 2 * 1024 * 4);
  m.bsel = (uint32_t *)p;
  p += align256((size_t)n_rows * 4 * 4);
  m.seg_cnt = (uint32_t *)p;
  p += align256((size_t)n_rows * m.S * 4);
  m.lkey = (uint32_t *)p;
  p += align256((size_t)n_rows * m.S * kSeg * 4);
  m.lpos = (int32_t *)p;
  return m;
}

size_t multi_ws_bytes(int n_rows, int max_len) {
  const size_t S = (max_len + kSeg - 1) / kSeg;
  return hist_bytes(kHeadRows) + (n_rows <= kHeadRows ? 0 : hist_bytes(n_rows)) +
         align256((size_t)n_rows * 2 * 1024 * 4) + align256((size_t)n_rows * 4 * 4) +
         align256((size_t)n_rows * S * 4) + 2 * align256((size_t)n_rows * S * kSeg * 4);
}

bool use_multi(int n_rows, int max_len) {
  return n_rows <= 64 && max_len >= 4096 && (max_len + kSeg - 1) / kSeg <= kMaxSegs;
}

__global__ void __launch_bounds__(256) topk_clear_kernel(uint32_t *__restrict__ hist, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) hist[i] = 0;
}

// Workgroup seg of a row's nw zeroes its share of n words at p.
template <int NT>
__device__ __forceinline__ void zero_share(uint32_t *p, int n, int seg, int nw) {
  const int per = (n + nw - 1) / nw;
  const int e = min(n, (seg + 1) * per);
  for (int i = seg * per + (int)threadIdx.x; i < e; i += NT) p[i] = 0;
}

__global__ void __launch_bounds__(kSegThreads)
topk_hist_kernel(const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ valid_len,
                 MultiWs m) {
  __shared__ uint32_t h[kBins];
  uint32_t *hist = m.hist;
  const int row = blockIdx.y, seg = blockIdx.x, tid = threadIdx.x;
  const int p0 = seg * kSeg;
  // the segment's scores are loaded before the row's valid length arrives
  // (buffer loads bounded by the allocated row length)
  const float *u = scores + (int64_t)row * ld;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(u), 0, m.max_len * 4, 0x00020000);
  float v[kSegPer];
#pragma unroll
  for (int j = 0; j < kSegPer; ++j)
    v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (p0 + tid + j * kSegThreads) * 4, 0, 0));
  const int n = min(max(valid_len[row], 0), m.max_len);
  zero_share<kSegThreads>(m.h10 + (int64_t)row * 2 * 1024, 2 * 1024, seg, gridDim.x);
  if (p0 >= n) return;
  const int p1 = min(n, p0 + kSeg);
  for (int b = tid; b < kBins; b += kSegThreads) h[b] = 0;
  lds_sync();
#pragma unroll
  for (int j = 0; j < kSegPer; ++j)
    if (p0 + tid + j * kSegThreads < p1) atomicAdd(&h[score_key(v[j]) >> 20], 1u);
  lds_sync();
  uint32_t *g = hist + (int64_t)row * kBins;
  for (int b = tid; b < kBins; b += kSegThreads)
    if (h[b]) atomicAdd(&g[b], h[b]);
}

// Block-wide exclusive scan for NT threads.
template <int NT>
__device__ __forceinline__ uint32_t nt_scan(uint32_t v, uint32_t *wt, uint32_t *total) {
  constexpr int W = NT / kWave;
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

// Bin of the nd-th largest entry of hist[0 .. nb) (nb a multiple of NT,
// highest bins to thread 0).  Returns the bin; *above gets the count in
// higher bins, *count the bin's own count.
template <int NT>
__device__ uint32_t nt_find(const uint32_t *hist, int nb, uint32_t nd, uint32_t *wt, uint32_t *res,
                            uint32_t *above, uint32_t *count) {
  const int tid = threadIdx.x;
  const int per = nb / NT;
  const int top = nb - 1 - tid * per;
  uint32_t sum = 0;
  for (int e = 0; e < per; ++e) sum += hist[top - e];
  uint32_t tot;
  uint32_t run = nt_scan<NT>(sum, wt, &tot);
  for (int e = 0; e < per; ++e) {
    const uint32_t c = hist[top - e];
    if (run < nd && nd <= run + c) {
      res[0] = top - e;
      res[1] = run;
      res[2] = c;
    }
    run += c;
  }
  lds_sync();
  const uint32_t b = res[0];
  *above = res[1];
  *count = res[2];
  lds_sync();
  return b;
}

// The same search by one wavefront, without barriers (nb a multiple of 256,
// at most 4096, hist 16-byte aligned): lane l owns bins top - l*per ...
// top - l*per - per + 1
// (highest bins to lane 0) and sums them, reading them rotated by l so the
// wavefront's reads spread over the LDS banks; a wavefront prefix sum picks
// the lane holding the nd-th largest key, then every lane takes one of that
// lane's bins and a second prefix sum picks the bin.  nd must be at least 1
// and at most the histogram total.
template <int NB>
__device__ __forceinline__ uint32_t wave_find_nb(const uint32_t *hist, int nb_rt, uint32_t nd,
                                                 uint32_t *above, uint32_t *count) {
  const int nb = NB ? NB : nb_rt;
  const int lane = threadIdx.x % kWave;
  const int per = nb / kWave;
  const int top = nb - 1 - lane * per;
  uint32_t sum = 0;
  {
    // 16 bytes at a time, chunk order rotated by lane (bank spread); with a
    // compile-time size every read is issued before the first is summed
    const uint4 *h4 = (const uint4 *)(hist + top - per + 1);
    const int nc = per / 4;
    if constexpr (NB != 0) {
      constexpr int NC = NB / kWave / 4;
      uint4 v[NC];
#pragma unroll
      for (int e = 0; e < NC; ++e) v[e] = h4[(e + lane) & (NC - 1)];
#pragma unroll
      for (int e = 0; e < NC; ++e) sum += (v[e].x + v[e].y) + (v[e].z + v[e].w);
    } else {
      for (int e = 0; e < nc; ++e) {
        const uint4 v = h4[(e + lane) & (nc - 1)];
        sum += (v.x + v.y) + (v.z + v.w);
      }
    }
  }
  const uint32_t incl = wave_incl_scan(sum), excl = incl - sum;
  const uint64_t hit = __ballot(excl < nd && nd <= incl);
  const int L = hit ? __ffsll((unsigned long long)hit) - 1 : kWave - 1;
  const uint32_t base = __shfl(excl, L, kWave);
  const int topL = nb - 1 - L * per;
  const uint32_t v = lane < per ? hist[topL - lane] : 0u;
  const uint32_t inc2 = base + wave_incl_scan(v), ex2 = inc2 - v;
  const uint64_t hit2 = __ballot(lane < per && ex2 < nd && nd <= inc2);
  const int t = hit2 ? __ffsll((unsigned long long)hit2) - 1 : 0;
  *above = __shfl(ex2, t, kWave);
  *count = __shfl(v, t, kWave);
  return (uint32_t)(topL - t);
}

__device__ uint32_t wave_find(const uint32_t *hist, int nb, uint32_t nd, uint32_t *above,
                              uint32_t *count) {
  if (nb == 4096) return wave_find_nb<4096>(hist, nb, nd, above, count);
  if (nb == 1024) return wave_find_nb<1024>(hist, nb, nd, above, count);
  return wave_find_nb<0>(hist, nb, nd, above, count);
}

// Sum over the wavefront, in every lane (DPP scan, then lane 63's total).
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(v), kWave - 1);
}

__global__ void __launch_bounds__(kSegThreads)
topk_extract_kernel(const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ valid_len,
                    int k0, int k1, MultiWs m) {
  __shared__ uint32_t wt[kSegThreads / kWave];
  __shared__ uint32_t res[4];
  __shared__ __align__(16) uint32_t h12[kBins];
  const int row = blockIdx.y, seg = blockIdx.x, tid = threadIdx.x;
  const int p0 = seg * kSeg;
  // One round trip: this segment's scores (buffer loads bounded by the
  // allocated row length, issued before the row's valid length arrives) and
  // the row histogram (into LDS).
  const float *u = scores + (int64_t)row * ld;
  const int pb = p0 + tid * kSegPer;
  float sv[kSegPer];
  {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(u), 0, m.max_len * 4, 0x00020000);
    if ((reinterpret_cast<uintptr_t>(u) & 15) == 0) {
#pragma unroll
      for (int h = 0; h < kSegPer / 4; ++h) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, (pb + 4 * h) * 4, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[4 * h + e] = __uint_as_float(x[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < kSegPer; ++e)
        sv[e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (pb + e) * 4, 0, 0));
    }
  }
  uint32_t a[kBins / kSegThreads];
  {
    const uint32_t *g = m.hist + (int64_t)row * kBins;
#pragma unroll
    for (int e = 0; e < kBins / kSegThreads; ++e) a[e] = g[e * kSegThreads + tid];
  }
  const int n = min(max(valid_len[row], 0), m.max_len);
  if (p0 >= n) {
    if (tid == 0) m.seg_cnt[(int64_t)row * m.S + seg] = 0;
    return;
  }
#pragma unroll
  for (int e = 0; e < kBins / kSegThreads; ++e) h12[e * kSegThreads + tid] = a[e];
  uint32_t key[kSegPer];
#pragma unroll
  for (int e = 0; e < kSegPer; ++e) key[e] = pb + e < n ? score_key(sv[e]) : 0u;
  lds_sync();
  // threshold buckets of both outputs (all ones: the output takes every key),
  // output j's by wavefront j
  {
    const int wave = tid / kWave;
    if (wave < 2) {
      const int kj = wave ? k1 : k0;
      const bool on = wave ? (k1 > 0 && k1 < n) : (k0 < n);
      uint32_t b = 0xFFFFFFFFu, above = 0, c;
      if (on) b = wave_find(h12, kBins, (uint32_t)kj, &above, &c);
      if (tid % kWave == 0) {
        res[wave] = b;
        if (seg == 0) {  // for the select step, which no longer reads the row histogram
          m.bsel[(int64_t)row * 4 + 2 * wave] = b;
          m.bsel[(int64_t)row * 4 + 2 * wave + 1] = above;
        }
      }
    }
    lds_sync();
  }
  const uint32_t bk[2] = {res[0], res[1]};
  const int kmax = max(k0, k1);
  const uint32_t b1 = kmax < n ? (k1 > k0 ? bk[1] : bk[0]) : 0u;  // extraction bucket
  uint32_t cnt = 0;
#pragma unroll
  for (int e = 0; e < kSegPer; ++e) {
    const int p = pb + e;
    cnt += (p < n && (key[e] >> 20) >= b1) ? 1u : 0u;
  }
  uint32_t tot;
  uint32_t pos = nt_scan<kSegThreads>(cnt, wt, &tot);
  const int64_t off = ((int64_t)row * m.S + seg) * kSeg;
  uint32_t *h10 = m.h10 + (int64_t)row * 2 * 1024;
#pragma unroll
  for (int e = 0; e < kSegPer; ++e) {
    const int p = pb + e;
    if (p < n && (key[e] >> 20) >= b1) {
      m.lkey[off + pos] = key[e];
      m.lpos[off + pos] = p;
      ++pos;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (p < n && (key[e] >> 20) == bk[j]) atomicAdd(&h10[j * 1024 + ((key[e] >> 10) & 1023u)], 1u);
  }
  // zeros up to the next multiple of 256 slots, so the select step reads the
  // list in whole 16-byte-per-lane rows without masks (key 0 is no score's)
  for (uint32_t e = tot + tid; e < ((tot + 255u) & ~255u); e += kSegThreads) m.lkey[off + e] = 0u;
  if (tid == 0) m.seg_cnt[(int64_t)row * m.S + seg] = tot;
}

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
  auto find = [&](int nb, uint32_t nd) {  // bin of the nd-th largest, by wavefront 0
    if (tid < kWave) {
      uint32_t above, c;
      const uint32_t b = wave_find(sh.hist, nb, nd, &above, &c);
      if (tid == 0) {
        sh.sel_bin = b;
        sh.sel_above = above;
        sh.sel_count = c;
      }
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

// ---------------------------------------------------------------------------
// Select step of the multi-workgroup path, one workgroup per (row, segment).
// Every workgroup derives the exact thresholds itself: the 12-bit bucket (and
// the count above it) as the extract step found it, the next 10 bits from the
// bucket's histogram built by the extract step (one wavefront per output, a
// single-wavefront search), the last 10 bits from the row's extracted keys
// that share those 22 bits.  The same
// pass over the extracted keys (one wavefront per segment) counts, in the
// segments before its own, the keys above each threshold and those equal to
// it, which fixes the output offset of the segment's first selected key; the
// segment then emits its own selected keys in ascending positions.  Two
// outputs share every pass (their per-thread counts ride in the two halves
// of a 32-bit word where they are bounded by 2048).
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;

struct SelShared {
  __align__(16) uint32_t h10[2][1024];
  uint32_t seg_off[kMaxSegs + 1];
  __align__(16) uint32_t hlow[2][1024];  // low 10 bits of the keys sharing the 22-bit prefix: whole row
  __align__(16) uint32_t hbef[2][1024];  // ... in segments before this one
  uint32_t wt[kSelThreads / kWave];
  uint32_t pre22[2], need[2], gtb[2], theta[2], need_eq[2], all_eq[2], sel_before[2], eq_before[2];
};

__global__ void __launch_bounds__(kSelThreads)
topk_select_kernel(const float *__restrict__ scores, int64_t ld,
                   const int32_t *__restrict__ valid_len, const int32_t *__restrict__ ids,
                   int64_t ids_ld, int ids_rows, FinOut o0, FinOut o1, int n_out, MultiWs m) {
  __shared__ SelShared sh;
  const int row = blockIdx.y, seg = blockIdx.x, tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  constexpr int NW = kSelThreads / kWave;
  constexpr int kOwn = kSeg / kSelThreads;  // own entries per thread
  // Every load whose address depends on no other load is issued here, before
  // any result is used: the row's valid length, buckets and second-level
  // histograms, the segments' key counts, this segment's extracted keys and positions, and the first
  // 256 extracted keys of the 8 segments this wavefront scans first.  Each
  // segment owns kSeg slots, so these are in bounds whatever the counts.
  const int n = min(max(valid_len[row], 0), m.max_len);
  uint32_t b[2 * 1024 / kSelThreads];
  {
    const uint32_t *g10 = m.h10 + (int64_t)row * 2 * 1024;
#pragma unroll
    for (int e = 0; e < 2 * 1024 / kSelThreads; ++e) b[e] = g10[e * kSelThreads + tid];
  }
  const uint4 bs = *reinterpret_cast<const uint4 *>(m.bsel + (int64_t)row * 4);  // bucket, above x2
  const uint32_t *cnt = m.seg_cnt + (int64_t)row * m.S;
  // (unconditional loads from clamped, in-bounds addresses: a load under a
  // branch makes the compiler wait for every load before it at the join;
  // values past the row's segments are never used)
  const uint32_t c_first = cnt[min(tid, m.S - 1)];
  const int64_t own = ((int64_t)row * m.S + seg) * kSeg;
  const uint32_t i0 = tid * kOwn;
  static_assert(kOwn == 2, "own entries load as one 8-byte vector");
  const uint2 ek2 = *reinterpret_cast<const uint2 *>(m.lkey + own + i0);
  const int2 ep2 = *reinterpret_cast<const int2 *>(m.lpos + own + i0);
  const uint32_t *lkey = m.lkey + (int64_t)row * m.S * kSeg;
  constexpr int kPF = 4;  // segments wave + NW u, u < kPF: their first 256 keys, 4 per lane
  uint4 pk[kPF];
#pragma unroll
  for (int v = 0; v < kPF; ++v) {
    const int sg = min(wave + NW * v, m.S - 1);
    pk[v] = *reinterpret_cast<const uint4 *>(lkey + (int64_t)sg * kSeg + 4 * lane);
  }
  const FinOut out[2] = {o0, o1};
  if (seg == 0) {  // padding of the outputs
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j >= n_out) continue;
      for (int t = min(out[j].k, n) + tid; t < out[j].k; t += kSelThreads) {
        out[j].idx[(int64_t)row * out[j].k + t] = -1;
        if (out[j].val) out[j].val[(int64_t)row * out[j].k + t] = -INFINITY;
      }
    }
  }
  const int S = (n + kSeg - 1) / kSeg;
  // the row histogram is read by no later step: zero it for the next call
  zero_share<kSelThreads>(m.hist + (int64_t)row * kBins, kBins, seg, gridDim.x);
  if (n <= 0 || seg >= S) return;  // uniform per workgroup
  const int32_t *idm = ids ? ids + (int64_t)(row % ids_rows) * ids_ld : nullptr;
  const float *u = scores + (int64_t)row * ld;
#pragma unroll
  for (int e = 0; e < 2 * 1024 / kSelThreads; ++e) (&sh.h10[0][0])[e * kSelThreads + tid] = b[e];
  // offsets of the segments' lists in the row's flattened extracted keys
  // (rows of up to 64 segments: one wavefront's prefix sum, no barrier; the
  // barrier below publishes it)
  if (S <= kWave) {
    if (wave == 0) {
      const uint32_t c = lane < S ? c_first : 0u;
      const uint32_t incl = wave_incl_scan(c);
      if (lane < S) sh.seg_off[lane] = incl - c;
      if (lane == S - 1) sh.seg_off[S] = incl;
    }
  } else {
    uint32_t carry = 0;
    for (int b0 = 0; b0 < S; b0 += kSelThreads) {
      const uint32_t c = (b0 + tid < S) ? (b0 == 0 ? c_first : cnt[b0 + tid]) : 0u;
      uint32_t tot;
      const uint32_t ex = nt_scan<kSelThreads>(c, sh.wt, &tot);
      if (b0 + tid < S) sh.seg_off[b0 + tid] = carry + ex;
      carry += tot;
    }
    if (tid == 0) sh.seg_off[S] = carry;
  }
  for (int b0 = tid; b0 < 2 * 1024; b0 += kSelThreads) {
    (&sh.hlow[0][0])[b0] = 0;
    (&sh.hbef[0][0])[b0] = 0;
  }
  lds_sync();
  if (tid < 2) sh.gtb[tid] = 0;
  // thresholds: top 12 bits, then the next 10; output j's by wavefront j
  bool act[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) act[j] = j < n_out && out[j].k < n;  // else every key is taken
  // (selects instead of indexing by the wavefront: a runtime index would put
  // the arrays in scratch memory)
  const bool act_w = wave == 0 ? act[0] : act[1];
  const uint32_t k_w = (uint32_t)(wave == 0 ? o0.k : o1.k);
  if (wave < 2 && act_w) {
    const int j = wave;
    uint32_t above, c;
    const uint32_t b12 = j == 0 ? bs.x : bs.z;
    const uint32_t nd = k_w - (j == 0 ? bs.y : bs.w);
    const uint32_t d10 = wave_find(sh.h10[j], 1024, nd, &above, &c);
    if (lane == 0) {
      sh.pre22[j] = (b12 << 10) | d10;
      sh.need[j] = nd - above;
    }
  }
  lds_sync();
  uint32_t pre22[2] = {0, 0}, need[2] = {0, 0};
#pragma unroll
  for (int j = 0; j < 2; ++j)
    if (act[j]) {
      pre22[j] = sh.pre22[j];
      need[j] = sh.need[j];
    }
  // One pass over the row's extracted keys, one wavefront per segment, four
  // keys per lane per 16-byte load (the lists are zero-padded to whole
  // 256-key rows; key 0 matches no prefix): the low 10 bits of the keys
  // sharing each 22-bit prefix, over the row and over the segments before
  // this one, and the keys above it before this one (per-lane counts, summed
  // once at the end).
  const uint32_t my0 = sh.seg_off[seg];
  uint32_t gtc[2] = {0, 0};
  auto visit4 = [&](const uint4 kv, bool before) __attribute__((always_inline)) {
    const uint32_t ks[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (!act[j]) continue;  // uniform
      const uint32_t P = pre22[j];
      bool hit = false;
#pragma unroll
      for (int t = 0; t < 4; ++t) hit |= (ks[t] >> 10) == P;
      if (before) {  // uniform
#pragma unroll
        for (int t = 0; t < 4; ++t) gtc[j] += (ks[t] >> 10) > P ? 1u : 0u;
      }
      if (hit) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if ((ks[t] >> 10) == P) {
            atomicAdd(&sh.hlow[j][ks[t] & 1023u], 1u);
            if (before) atomicAdd(&sh.hbef[j][ks[t] & 1023u], 1u);
          }
      }
    }
  };
  auto seg_pass = [&](int sg, const uint4 first, uint32_t cn) __attribute__((always_inline)) {
    if (sg >= S) return;  // uniform
    const bool before = sg < seg;
    if (cn == 0) return;
    visit4(first, before);
    for (uint32_t e0 = 256; e0 < cn; e0 += 256)  // lists longer than 256 keys
      visit4(*reinterpret_cast<const uint4 *>(lkey + (int64_t)sg * kSeg + e0 + 4 * lane), before);
  };
  if (act[0] || act[1]) {
    uint32_t cns[kPF];  // the segments' key counts, read before any is used
#pragma unroll
    for (int v = 0; v < kPF; ++v) {
      const int sg = min(wave + NW * v, S - 1);
      cns[v] = sh.seg_off[sg + 1] - sh.seg_off[sg];
    }
#pragma unroll
    for (int v = 0; v < kPF; ++v) seg_pass(wave + NW * v, pk[v], cns[v]);
    for (int sg = wave + NW * kPF; sg < S; sg += NW)
      seg_pass(sg, *reinterpret_cast<const uint4 *>(lkey + (int64_t)sg * kSeg + 4 * lane),
               sh.seg_off[sg + 1] - sh.seg_off[sg]);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t g = act[j] ? wave_sum_u32(gtc[j]) : 0u;
    if (lane == 0 && g) atomicAdd(&sh.gtb[j], g);
  }
  lds_sync();
  // exact thresholds and this segment's offsets, output j's by wavefront j
  if (wave < 2 && act_w) {
    const int j = wave;
    const uint32_t need_w = j == 0 ? need[0] : need[1], pre_w = j == 0 ? pre22[0] : pre22[1];
    uint32_t above, c;
    const uint32_t d = wave_find(sh.hlow[j], 1024, need_w, &above, &c);
    uint32_t gl = 0;  // keys of the 22-bit prefix above theta, before this segment
    {
      uint32_t hb[1024 / kWave];  // every read issued before the first is used
#pragma unroll
      for (int i = 0; i < 1024 / kWave; ++i) hb[i] = sh.hbef[j][lane + i * kWave];
#pragma unroll
      for (int i = 0; i < 1024 / kWave; ++i) gl += (uint32_t)(lane + i * kWave) > d ? hb[i] : 0u;
    }
    gl = wave_sum_u32(gl);
    if (lane == 0) {
      const uint32_t ne = need_w - above, eb = sh.hbef[j][d];
      sh.theta[j] = (pre_w << 10) | d;
      sh.need_eq[j] = ne;
      sh.all_eq[j] = ne == c ? 1u : 0u;
      sh.eq_before[j] = eb;
      sh.sel_before[j] = sh.gtb[j] + gl + min(eb, ne);
    }
  }
  lds_sync();
  uint32_t theta[2] = {0, 0}, need_eq[2] = {0, 0}, sel_before[2] = {my0, my0},
           eq_before[2] = {0, 0};
  bool all_eq[2] = {true, true};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (!act[j]) continue;  // every key is taken: offset = extracted keys before
    theta[j] = sh.theta[j];
    need_eq[j] = sh.need_eq[j];
    all_eq[j] = sh.all_eq[j] != 0;
    eq_before[j] = sh.eq_before[j];
    sel_before[j] = sh.sel_before[j];
  }
  // emit this segment's selected keys in ascending positions
  const uint32_t mc = sh.seg_off[seg + 1] - my0;
  const uint32_t ek[kOwn] = {ek2.x, ek2.y};
  const int32_t ep[kOwn] = {ep2.x, ep2.y};
  uint32_t eqb[2] = {eq_before[0], eq_before[1]};
  if ((act[0] && !all_eq[0]) || (act[1] && !all_eq[1])) {
    uint32_t c = 0;
#pragma unroll
    for (int t = 0; t < kOwn; ++t) {
      const bool valid = i0 + t < mc;
      c += (valid && act[0] && ek[t] == theta[0]) ? 1u : 0u;
      c += (valid && act[1] && ek[t] == theta[1]) ? 0x10000u : 0u;
    }
    uint32_t tot;
    const uint32_t ex = nt_scan<kSelThreads>(c, sh.wt, &tot);
    eqb[0] += ex & 0xFFFFu;
    eqb[1] += ex >> 16;
  }
  uint32_t selm[2] = {0, 0}, c_sel = 0;
#pragma unroll
  for (int t = 0; t < kOwn; ++t) {
    const bool valid = i0 + t < mc;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j >= n_out) continue;
      const bool eq = valid && act[j] && ek[t] == theta[j];
      const bool s = valid && (!act[j] || ek[t] > theta[j] ||
                               (eq && (all_eq[j] || eqb[j] < need_eq[j])));
      eqb[j] += eq ? 1u : 0u;
      selm[j] |= s ? (1u << t) : 0u;
      c_sel += s ? (j ? 0x10000u : 1u) : 0u;
    }
  }
  uint32_t tot;
  const uint32_t ex = nt_scan<kSelThreads>(c_sel, sh.wt, &tot);
  uint32_t pos[2] = {sel_before[0] + (ex & 0xFFFFu), sel_before[1] + (ex >> 16)};
#pragma unroll
  for (int t = 0; t < kOwn; ++t) {
    const int p = ep[t];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j >= n_out || !((selm[j] >> t) & 1u)) continue;
      const uint32_t mm = (uint32_t)min(out[j].k, n);
      if (pos[j] < mm) {
        out[j].idx[(int64_t)row * out[j].k + pos[j]] = idm ? idm[p] : p;
        if (out[j].val) out[j].val[(int64_t)row * out[j].k + pos[j]] = u[p];
      }
      ++pos[j];
    }
  }
}

// ---------------------------------------------------------------------------
// Rows of 8193 .. kLdsRow elements (longer candidate lists): one
// workgroup per row keeps the whole row's keys in LDS, so the three radix
// passes and the ordered emit touch global memory once.
// ---------------------------------------------------------------------------
constexpr int kLdsRow = 16384;

struct LdsRowShared {
  __align__(16) uint32_t key[kLdsRow];
  __align__(16) uint32_t hist[kBins];
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
  const int n = max(min(valid_len ? valid_len[row] : const_len, min(const_len, kLdsRow)), 0);
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

// ---------------------------------------------------------------------------
// Rows of at most 8192 scores (a follower layer's rescored candidates): one
// workgroup of 1024 threads per row, eight consecutive positions per thread
// held in registers together with their ids (both loaded up front), so LDS
// holds only histograms and every pass re-reads registers:
//   A. histogram of key bits 31..21 in 8 interleaved copies (lane % 8 picks
//      one: a candidate set's scores crowd into few bins, and lanes of one
//      atomic that hit the same bin then mostly hit different words); each
//      thread merges two bins and a block scan finds the bin b1 of the k-th
//      largest key (likewise in B and C);
//   B. among keys in b1, histogram of bits 20..10; C. among keys matching
//      both, of bits 9..0: theta, and how many keys equal to it are taken;
//   D. the equal keys taken are the lowest positions, so one block scan of
//      the per-thread counts of keys above theta and equal to it (two 16-bit
//      halves of one word) gives every thread its output offset.
// ---------------------------------------------------------------------------
constexpr int kR8Per = 8;
constexpr int kR8Max = kThreads * kR8Per;  // 8192
constexpr int kR8Bins = 2048;
constexpr int kR8Copies = 8;

struct R8Shared {
  __align__(16) uint32_t hA[kR8Bins * kR8Copies];  // [bin][copy]
  __align__(16) uint32_t hB[kR8Bins];
  __align__(16) uint32_t hC[1024];
  uint32_t wtot[kWaves];
  uint32_t sel[3];  // bin, count above it, its own count
};

// Block-wide search for the bin of the nd-th largest key: thread t holds the
// counts c[e] of bins top - e, top = nb - 1 - PER t (highest bins to thread
// 0); one block scan of the per-thread sums, then the thread whose bins hold
// the nd-th key publishes (bin, count above it, its count) in sel.  nd must
// be at least 1 and at most the histogram total.
template <int PER>
__device__ __forceinline__ void r8_find(const uint32_t (&c)[PER], int nb, uint32_t nd, uint32_t *wtot,
                                        uint32_t *sel) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  uint32_t s = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) s += c[e];
  const uint32_t incl = wave_incl_scan(s);
  if (lane == kWave - 1) wtot[wave] = incl;
  lds_sync();
  uint32_t run = incl - s;
#pragma unroll
  for (int w2 = 0; w2 < kWaves; ++w2) run += w2 < wave ? wtot[w2] : 0u;
  const int top = nb - 1 - PER * tid;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (run < nd && nd <= run + c[e]) {
      sel[0] = (uint32_t)(top - e);
      sel[1] = run;
      sel[2] = c[e];
    }
    run += c[e];
  }
  lds_sync();
}

__global__ void __launch_bounds__(kThreads)
topk_r8_kernel(const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ valid_len,
               int const_len, const int32_t *__restrict__ ids, int64_t ids_ld, int ids_rows, int k,
               int32_t *__restrict__ out_idx, float *__restrict__ out_val,
               int32_t *__restrict__ all_idx, int all_k) {
  __shared__ R8Shared sh;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const float *u = scores + (int64_t)row * ld;
  const int32_t *idm = ids ? ids + (int64_t)(row % ids_rows) * ids_ld : nullptr;
  const int cap = min(const_len, kR8Max);  // the row's allocated length bounds the loads
  // Scores and ids are loaded before the row's valid length is known (buffer
  // loads bounded by the allocated length), so their latency overlaps its.
  const int p0 = kR8Per * tid;
  float v[kR8Per];
  int32_t id[kR8Per];
  {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(u), 0, cap * 4, 0x00020000);
    if ((reinterpret_cast<uintptr_t>(u) & 15) == 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, (p0 + 4 * h) * 4, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[4 * h + j] = __uint_as_float(x[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kR8Per; ++j)
        v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (p0 + j) * 4, 0, 0));
    }
    if (idm) {
      const __amdgpu_buffer_rsrc_t ri =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(idm), 0, cap * 4, 0x00020000);
      if ((reinterpret_cast<uintptr_t>(idm) & 15) == 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const auto x = __builtin_amdgcn_raw_buffer_load_b128(ri, (p0 + 4 * h) * 4, 0, 0);
#pragma unroll
          for (int j = 0; j < 4; ++j) id[4 * h + j] = (int32_t)x[j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < kR8Per; ++j)
          id[j] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ri, (p0 + j) * 4, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kR8Per; ++j) id[j] = p0 + j;
    }
  }
  const int n = max(valid_len ? min(valid_len[row], cap) : cap, 0);
  int32_t *oi = out_idx + (int64_t)row * k;
  float *ov = out_val ? out_val + (int64_t)row * k : nullptr;
  const int m = min(k, n);
  for (int j = m + tid; j < k; j += kThreads) {
    oi[j] = -1;
    if (ov) ov[j] = -INFINITY;
  }
  if (all_idx) {  // a second output that takes every position (all_k >= n)
    int32_t *oa = all_idx + (int64_t)row * all_k;
    for (int j = tid; j < all_k; j += kThreads) oa[j] = j < n ? (idm ? idm[j] : j) : -1;
  }
  if (n <= k) {
    for (int p = tid; p < n; p += kThreads) {
      oi[p] = idm ? idm[p] : p;
      if (ov) ov[p] = u[p];
    }
    return;
  }
  const int nv = min(kR8Per, max(0, n - p0));  // this thread's valid entries (a prefix)
  // clear the histograms while the loads are in flight
  {
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < kR8Bins * kR8Copies / 4 / kThreads; ++i)
      reinterpret_cast<uint4 *>(sh.hA)[tid + i * kThreads] = z;
    if (tid < kR8Bins / 4) reinterpret_cast<uint4 *>(sh.hB)[tid] = z;
    if (tid < 1024 / 4) reinterpret_cast<uint4 *>(sh.hC)[tid] = z;
  }
  uint32_t key[kR8Per];
#pragma unroll
  for (int j = 0; j < kR8Per; ++j) key[j] = score_key(v[j]);
  lds_sync();
  // A: thread t then merges the copies of bins 2047 - 2t and 2046 - 2t
  {
    uint32_t *h = sh.hA + (lane & (kR8Copies - 1));
#pragma unroll
    for (int j = 0; j < kR8Per; ++j)
      if (j < nv) atomicAdd(&h[(key[j] >> 21) * kR8Copies], 1u);
  }
  lds_sync();
  uint32_t cA[2];
  {
    const uint4 *c = reinterpret_cast<const uint4 *>(sh.hA) + 4 * (kR8Bins / 2 - 1 - tid);
    const uint4 a = c[0], b = c[1], d = c[2], e = c[3];  // bin 2046 - 2t, then 2047 - 2t
    cA[1] = (a.x + a.y) + (a.z + a.w) + (b.x + b.y) + (b.z + b.w);
    cA[0] = (d.x + d.y) + (d.z + d.w) + (e.x + e.y) + (e.z + e.w);
  }
  r8_find<2>(cA, kR8Bins, (uint32_t)k, sh.wtot, sh.sel);
  const uint32_t b1 = sh.sel[0];
  uint32_t need = (uint32_t)k - sh.sel[1];
  // B
#pragma unroll
  for (int j = 0; j < kR8Per; ++j)
    if (j < nv && (key[j] >> 21) == b1) atomicAdd(&sh.hB[(key[j] >> 10) & 2047u], 1u);
  lds_sync();
  uint32_t cB[2];
  {
    const uint2 x = reinterpret_cast<const uint2 *>(sh.hB)[kR8Bins / 2 - 1 - tid];
    cB[0] = x.y;
    cB[1] = x.x;
  }
  r8_find<2>(cB, kR8Bins, need, sh.wtot, sh.sel);
  const uint32_t p22 = (b1 << 11) | sh.sel[0];
  need -= sh.sel[1];
  // C
#pragma unroll
  for (int j = 0; j < kR8Per; ++j)
    if (j < nv && (key[j] >> 10) == p22) atomicAdd(&sh.hC[key[j] & 1023u], 1u);
  lds_sync();
  uint32_t cC[1] = {sh.hC[1023 - tid]};
  r8_find<1>(cC, 1024, need, sh.wtot, sh.sel);
  const uint32_t theta = (p22 << 10) | sh.sel[0];
  need -= sh.sel[1];  // keys equal to theta to take (lowest positions), >= 1
  // D
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < kR8Per; ++j) {
    gt += (j < nv && key[j] > theta) ? 1u : 0u;
    eq += (j < nv && key[j] == theta) ? 1u : 0u;
  }
  const uint32_t packed = gt | (eq << 16);  // each half bounded by 8192
  const uint32_t incl = wave_incl_scan(packed);
  if (lane == kWave - 1) sh.wtot[wave] = incl;
  lds_sync();
  uint32_t before = incl - packed;
#pragma unroll
  for (int w2 = 0; w2 < kWaves; ++w2) before += w2 < wave ? sh.wtot[w2] : 0u;
  uint32_t eq_b = before >> 16;
  uint32_t pos = (before & 0xFFFFu) + min(eq_b, need);
#pragma unroll
  for (int j = 0; j < kR8Per; ++j) {
    const bool is_eq = j < nv && key[j] == theta;
    const bool s = j < nv && (key[j] > theta || (is_eq && eq_b < need));
    if (s) {
      if (pos < (uint32_t)m) {
        oi[pos] = id[j];
        if (ov) ov[pos] = v[j];
      }
      ++pos;
    }
    eq_b += is_eq ? 1u : 0u;
  }
}

// ---------------------------------------------------------------------------
// Many rows of up to 64K scores (a prefill chunk: one row per query): one
// workgroup of 1024 threads per row holds the whole row's keys in registers
// (64 per thread), so the row is read from memory once.  Thread t holds
// positions it*4096 + 4t + j (it < NIT, j < 4): 16-byte coalesced loads, and
// every thread's positions ascend with (it, j).
//   A. histogram of key bits 31..21, the bin of the k-th largest key.  Score
//      rows crowd into few bins, so the histogram has 8 interleaved copies
//      (lane % 8 picks one): lanes of one atomic that hit the same bin mostly
//      hit different words;
//   the keys at or above that bin (the selection plus the bin's rest) are
//      gathered with their positions into an LDS list;
//   B. among keys in that bin, histogram of bits 20..10;
//   C. among keys matching both, histogram of bits 9..0: theta and how many
//      keys equal to theta are taken (lowest positions first);
//   D. two bitmaps over positions (key > theta, key == theta), then one
//      ordered pass over them: thread t owns positions 64t..64t+63, block
//      scans give the equal keys taken before it and its output offset.
//   B-D read the LDS list, or the row again from memory when more keys than
//   the list holds reach bin b1 (heavy ties).
// ---------------------------------------------------------------------------
constexpr int kRegMax = 65536;
constexpr int kRegBins = 2048;
constexpr int kRegCopies = 8;
constexpr int kRegCand = 6144;  // gathered (key, position) pairs, in pass A's space
static_assert(kRegBins + 1024 + 2 * (kRegCand + kWave) <= kRegBins * kRegCopies,
              "candidate list fits");

struct RegShared {
  __align__(16) uint32_t hA[kRegBins * kRegCopies];  // pass A copies [bin][copy]; then B and C
  uint32_t hM[kRegBins];               // pass A merged
  uint32_t gt[kRegMax / 32];
  uint32_t eq[kRegMax / 32];
  uint32_t wtot[kWaves];
  uint32_t sel_bin, sel_above, sel_count;
};

// Bin holding the need-th largest key of an nb-bin histogram h (nb a
// multiple of kThreads): sum_{b' > b} h[b'] < need <= sum_{b' >= b} h[b'].
__device__ void reg_find(RegShared &sh, const uint32_t *h, int nb, uint32_t need) {
  const int per = nb / kThreads;
  const int top = nb - 1 - threadIdx.x * per;
  uint32_t s = 0;
  for (int e = 0; e < per; ++e) s += h[top - e];
  uint32_t total;
  uint32_t run = block_exclusive_scan(s, sh.wtot, &total);
  for (int e = 0; e < per; ++e) {
    const uint32_t c = h[top - e];
    if (run < need && need <= run + c) {
      sh.sel_bin = top - e;
      sh.sel_above = run;
      sh.sel_count = c;
    }
    run += c;
  }
  lds_sync();
}

template <int NIT>
__global__ void __launch_bounds__(kThreads)
topk_reg_kernel(const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ valid_len,
                const int32_t *__restrict__ ids, int64_t ids_ld, int ids_rows, int k,
                int32_t *__restrict__ out_idx, float *__restrict__ out_val) {
  __shared__ RegShared sh;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid % kWave;
  const int n = max(min(valid_len[row], NIT * 4 * kThreads), 0);
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
  for (int b = tid; b < kRegCopies * kRegBins; b += kThreads) sh.hA[b] = 0;
  // this thread's valid elements form a prefix of its (it, j) order
  int nv = 0;
#pragma unroll
  for (int it = 0; it < NIT; ++it) nv += min(4, max(0, n - 4 * tid - it * 4096));
  // Buffer loads bounded by the row's valid length never read past the row.
  // Positions >= n get key 0: they land in bin 0 of pass A, whose count is
  // corrected below; a selection that reaches bin 0 takes the re-reading
  // path.
  uint32_t key[NIT * 4];
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(u), 0, n * 4, 0x00020000);
  if ((reinterpret_cast<uintptr_t>(u) & 15) == 0) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, (it * 4096 + 4 * tid) * 4, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) key[it * 4 + j] = score_key(__uint_as_float(x[j]));
    }
  } else {
#pragma unroll
    for (int it = 0; it < NIT; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        key[it * 4 + j] = score_key(__uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(rs, (it * 4096 + 4 * tid + j) * 4, 0, 0)));
  }
#pragma unroll
  for (int e = 0; e < NIT * 4; ++e) key[e] = e < nv ? key[e] : 0u;
  lds_sync();  // histogram cleared
  // A (consumes keys as their loads land)
  {
    uint32_t *h = sh.hA + (lane & (kRegCopies - 1));
#pragma unroll
    for (int e = 0; e < NIT * 4; ++e) atomicAdd(&h[(key[e] >> 21) * kRegCopies], 1u);
  }
  lds_sync();
  for (int b = tid; b < kRegBins; b += kThreads) {
    const uint4 *c = reinterpret_cast<const uint4 *>(sh.hA + b * kRegCopies);
    const uint4 x = c[0], y = c[1];
    sh.hM[b] = x.x + x.y + x.z + x.w + y.x + y.y + y.z + y.w -
               (b == 0 ? (uint32_t)(NIT * 4 * kThreads - n) : 0u);
  }
  lds_sync();
  uint32_t *hB = sh.hA, *hC = sh.hA + kRegBins;
  for (int b = tid; b < kRegBins + 1024; b += kThreads) sh.hA[b] = 0;
  reg_find(sh, sh.hM, kRegBins, (uint32_t)k);
  const uint32_t b1 = sh.sel_bin;
  uint32_t need = (uint32_t)k - sh.sel_above;
  // Gather every key at or above bin b1 (the selection plus bin b1's rest)
  // with its position into an LDS list: per-thread counts, one block scan
  // for the offsets, then writes of the listed keys only (a few percent of
  // the row), so the LDS sees only their traffic.
  uint32_t *ckey = sh.hA + kRegBins + 1024, *cpos = ckey + kRegCand + kWave;
  const uint32_t lo = b1 << 21;
  uint32_t cnt = 0;
#pragma unroll
  for (int e = 0; e < NIT * 4; ++e) cnt += key[e] >= lo ? 1u : 0u;
  uint32_t n_cand;
  uint32_t slot = block_exclusive_scan(cnt, sh.wtot, &n_cand);
  const bool listed = b1 > 0 && n_cand <= (uint32_t)kRegCand;  // else B-D re-read the row
  if (listed) {
#pragma unroll
    for (int e = 0; e < NIT * 4; ++e) {
      if (key[e] >= lo) {
        ckey[slot] = key[e];
        cpos[slot] = (e >> 2) * 4096 + 4 * tid + (e & 3);
        ++slot;
      }
    }
  }
  lds_sync();
  // B
  if (listed) {
    for (uint32_t c = tid; c < n_cand; c += kThreads)
      if ((ckey[c] >> 21) == b1) atomicAdd(&hB[(ckey[c] >> 10) & 2047u], 1u);
  } else {
    for (int p = tid; p < n; p += kThreads) {
      const uint32_t kp = score_key(u[p]);
      if ((kp >> 21) == b1) atomicAdd(&hB[(kp >> 10) & 2047u], 1u);
    }
  }
  lds_sync();
  reg_find(sh, hB, kRegBins, need);
  const uint32_t p22 = (b1 << 11) | sh.sel_bin;
  need -= sh.sel_above;
  // C
  if (listed) {
    for (uint32_t c = tid; c < n_cand; c += kThreads)
      if ((ckey[c] >> 10) == p22) atomicAdd(&hC[ckey[c] & 1023u], 1u);
  } else {
    for (int p = tid; p < n; p += kThreads) {
      const uint32_t kp = score_key(u[p]);
      if ((kp >> 10) == p22) atomicAdd(&hC[kp & 1023u], 1u);
    }
  }
  lds_sync();
  reg_find(sh, hC, 1024, need);
  const uint32_t theta = (p22 << 10) | sh.sel_bin;
  need -= sh.sel_above;  // keys equal to theta to take, 1 <= need <= n_eq
  const bool take_all_eq = need == sh.sel_count;
  // D: bitmaps of the positions with key > theta and key == theta
  if (listed) {
    for (int wd = tid; wd < kRegMax / 32; wd += kThreads) sh.gt[wd] = sh.eq[wd] = 0;
    lds_sync();
    for (uint32_t c = tid; c < n_cand; c += kThreads) {
      const uint32_t kc = ckey[c], pc = cpos[c];
      if (kc > theta) atomicOr(&sh.gt[pc >> 5], 1u << (pc & 31));
      else if (kc == theta) atomicOr(&sh.eq[pc >> 5], 1u << (pc & 31));
    }
  } else {
    // thread t builds the words of positions 64t..64t+63 from the row itself
    for (int h = 0; h < 2; ++h) {
      uint32_t g = 0, q = 0;
      for (int b = 0; b < 32; ++b) {
        const int p = 64 * tid + 32 * h + b;
        if (p < n) {
          const uint32_t kp = score_key(u[p]);
          g |= (kp > theta ? 1u : 0u) << b;
          q |= (kp == theta ? 1u : 0u) << b;
        }
      }
      sh.gt[2 * tid + h] = g;
      sh.eq[2 * tid + h] = q;
    }
  }
  lds_sync();
  uint64_t sel = (uint64_t)sh.gt[2 * tid] | (uint64_t)sh.gt[2 * tid + 1] << 32;
  uint64_t eqm = (uint64_t)sh.eq[2 * tid] | (uint64_t)sh.eq[2 * tid + 1] << 32;
  if (take_all_eq) {
    sel |= eqm;
  } else {
    uint32_t tot;
    const uint32_t before = block_exclusive_scan((uint32_t)__popcll(eqm), sh.wtot, &tot);
    const uint32_t take = need > before ? need - before : 0u;  // lowest `take` equal keys
    for (uint32_t c = 0; c < take && eqm; ++c) {
      const uint64_t low = eqm & (~eqm + 1);
      sel |= low;
      eqm ^= low;
    }
  }
  uint32_t tot;
  uint32_t pos = block_exclusive_scan((uint32_t)__popcll(sel), sh.wtot, &tot);
  while (sel) {
    const int b = __builtin_ctzll(sel);
    sel &= sel - 1;
    const int p = 64 * tid + b;
    if (pos < (uint32_t)m) {
      oi[pos] = idm ? idm[p] : p;
      if (ov) ov[pos] = u[p];
    }
    ++pos;
  }
}

hipError_t launch_multi(const float *scores, int64_t ld, int n_rows, const int32_t *valid_len,
                        const int32_t *ids, int64_t ids_ld, int ids_rows, int max_len, FinOut o0,
                        FinOut o1, int n_out, void *ws, bool ws_clean, hipStream_t st,
                        bool counted = false) {
  MultiWs m = carve(ws, n_rows, max_len);
  dim3 g(m.S, n_rows);
  if (!counted) {  // else the scorer built the row histograms and zeroed h10
    if (!(ws_clean && n_rows <= kHeadRows)) {
      const int nc = n_rows * kBins;
      topk_clear_kernel<<<(nc + 255) / 256, 256, 0, st>>>(m.hist, nc);
    }
    topk_hist_kernel<<<g, kSegThreads, 0, st>>>(scores, ld, valid_len, m);
  }
  topk_extract_kernel<<<g, kSegThreads, 0, st>>>(scores, ld, valid_len, o0.k,
                                                 n_out == 2 ? o1.k : 0, m);
  topk_select_kernel<<<g, kSelThreads, 0, st>>>(scores, ld, valid_len, ids, ids_ld, ids_rows, o0,
                                                o1, n_out, m);
  return hipGetLastError();
}

}  // namespace

size_t topk_ws_bytes(int n_rows, int max_len, int) {
  return (max_len > kLdsRow && use_multi(n_rows, max_len)) ? multi_ws_bytes(n_rows, max_len) : 0;
}

hipError_t launch_topk_with_all(const float *scores, int64_t ld, int n_rows,
                                const int32_t *valid_len, int max_len, int k, int32_t *out_idx,
                                int all_k, int32_t *all_idx, hipStream_t st) {
  if (max_len > kR8Max || all_k < max_len) return hipErrorInvalidValue;
  topk_r8_kernel<<<n_rows, kThreads, 0, st>>>(scores, ld, valid_len, max_len, nullptr, 0, 1, k, out_idx,
                                              nullptr, all_idx, all_k);
  return hipGetLastError();
}

hipError_t launch_topk(const float *scores, int64_t ld, int n_rows, const int32_t *valid_len,
                       const int32_t *ids, int64_t ids_ld, int ids_rows, int max_len, int k, int32_t *out_idx,
                       float *out_val, void *ws, hipStream_t st) {
  if (max_len <= kR8Max) {
    topk_r8_kernel<<<n_rows, kThreads, 0, st>>>(scores, ld, valid_len, max_len, ids, ids_ld, ids_rows, k,
                                                out_idx, out_val, nullptr, 0);
    return hipGetLastError();
  }
  if (max_len <= kLdsRow) {
    const size_t lds = sizeof(LdsRowShared);
    static DeviceOnce *const once = device_once_new();
    const hipError_t e = raise_lds_limit(once, (const void *)topk_lds_kernel, (int)lds);
    if (e != hipSuccess) return e;
    topk_lds_kernel<<<n_rows, kThreads, lds, st>>>(scores, ld, valid_len, max_len, ids, ids_ld, ids_rows, k,
                                                   out_idx, out_val);
    return hipGetLastError();
  }
  if (use_multi(n_rows, max_len))
    return launch_multi(scores, ld, n_rows, valid_len, ids, ids_ld, ids_rows, max_len,
                        FinOut{k, out_idx, out_val}, FinOut{0, nullptr, nullptr}, 1, ws, false, st);
  if (max_len <= kRegMax) {
    if (max_len <= kRegMax / 2)
      topk_reg_kernel<8><<<n_rows, kThreads, 0, st>>>(scores, ld, valid_len, ids, ids_ld, ids_rows,
                                                      k, out_idx, out_val);
    else
      topk_reg_kernel<16><<<n_rows, kThreads, 0, st>>>(scores, ld, valid_len, ids, ids_ld, ids_rows,
                                                       k, out_idx, out_val);
    return hipGetLastError();
  }
  const size_t lds = sizeof(TopkShared);
  static DeviceOnce *const once = device_once_new();
  const hipError_t e = raise_lds_limit(once, (const void *)topk_row_kernel, (int)lds);
  if (e != hipSuccess) return e;
  topk_row_kernel<<<n_rows, kThreads, lds, st>>>(scores, ld, valid_len, ids, ids_ld, ids_rows, k, out_idx,
                                                 out_val);
  return hipGetLastError();
}

size_t topk2_ws_bytes(int n_rows, int max_len) { return multi_ws_bytes(n_rows, max_len); }

int topk_single_max() { return kR8Max; }

int64_t topk2_max_len() { return (int64_t)kMaxSegs * kSeg; }

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
                      ws, true, st);
}

void topk2_count_arrays(void *ws, int n_rows, int max_len, uint32_t **hist, uint32_t **h10,
                        int *h10_words) {
  const MultiWs m = carve(ws, n_rows, max_len);
  *hist = m.hist;
  *h10 = m.h10;
  *h10_words = n_rows * 2 * 1024;
}

int topk2_counted_max_rows() { return kHeadRows; }

hipError_t launch_topk2_counted(const float *scores, int64_t ld, int n_rows, const int32_t *valid_len,
                                int max_len, int k_outer, int32_t *out_outer, int k_inner,
                                int32_t *out_inner, void *ws, hipStream_t st) {
  return launch_multi(scores, ld, n_rows, valid_len, nullptr, 0, 1, max_len,
                      FinOut{k_outer, out_outer, nullptr}, FinOut{k_inner, out_inner, nullptr}, 2,
                      ws, true, st, true);
}

}  // namespace li
