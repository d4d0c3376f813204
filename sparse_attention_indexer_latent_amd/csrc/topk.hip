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
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint32_t y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) wtot[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w2 = 0; w2 < kWaves; ++w2) {
    const uint32_t t = wtot[w2];
    before += (w2 < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();
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
  __syncthreads();
}

__global__ void __launch_bounds__(kThreads)
topk_row_kernel(const float *__restrict__ scores, int64_t ld, const int32_t *__restrict__ valid_len,
                const int32_t *__restrict__ ids, int64_t ids_ld, int k,
                int32_t *__restrict__ out_idx, float *__restrict__ out_val) {
  extern __shared__ __align__(16) unsigned char smem[];
  TopkShared &sh = *reinterpret_cast<TopkShared *>(smem);
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = valid_len[row];
  const float *u = scores + (int64_t)row * ld;
  const int32_t *idm = ids ? ids + (int64_t)row * ids_ld : nullptr;
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
  __syncthreads();
  for (int p = tid; p < n; p += kThreads) atomicAdd(&sh.hist[score_key(u[p]) >> 20], 1u);
  __syncthreads();
  find_bin(sh, kBins, (uint32_t)k);
  const uint32_t b1 = sh.sel_bin;
  uint32_t need = (uint32_t)k - sh.sel_above;  // keys to take from bin b1 (>= 1)
  const uint32_t n_b1 = sh.sel_count;
  const bool in_lds = n_b1 <= (uint32_t)kCap;

  // 2. gather bin b1 into the candidate list
  if (tid == 0) sh.n_cand = 0;
  __syncthreads();
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
  __syncthreads();

  // 3. refine the low 20 bits: digit 2 = bits 19..10, digit 3 = bits 9..0
  uint32_t prefix = b1;  // key bits known so far, right-aligned
  int known = 12;        // number of known leading bits
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = 20 - 10 * (pass + 1);
    for (int b = tid; b < 1024; b += kThreads) sh.hist[b] = 0;
    __syncthreads();
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
    __syncthreads();
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

}  // namespace

size_t topk_ws_bytes(int, int, int) { return 0; }

hipError_t launch_topk(const float *scores, int64_t ld, int n_rows, const int32_t *valid_len,
                       const int32_t *ids, int64_t ids_ld, int max_len, int k, int32_t *out_idx,
                       float *out_val, void *, hipStream_t st) {
  (void)max_len;
  const size_t lds = sizeof(TopkShared);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void *)topk_row_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr_set = true;
  }
  topk_row_kernel<<<n_rows, kThreads, lds, st>>>(scores, ld, valid_len, ids, ids_ld, k, out_idx,
                                                 out_val);
  return hipGetLastError();
}

}  // namespace li
