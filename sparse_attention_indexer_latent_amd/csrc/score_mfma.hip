// Matrix-core scorer for eq. (8) of the LatentIndex summary ("Methodology"):
// u_t = sum_h w_h ReLU(q~_h . c_t + beta_h), for H = 64 heads over a bf16
// latent cache.
//
// Why matrix cores: one cached token of r = 256 bf16 values (512 B) meets 64
// absorbed queries, 2*64*256 = 32768 flop, i.e. 64 flop per byte read, three
// times the fp32 vector ridge of MI355X (157 TFLOP/s / 8 TB/s).  The product
// [64 heads x r] x [r x tokens] is a real dense contraction even for a single
// decode query, so it runs on v_mfma_f32_32x32x16_bf16 and the kernel stays
// bound by the HBM stream of the latent.
//
// Precision: an fp32 q~ is carried as bf16 hi + lo (hi = RNE(q~), lo =
// RNE(q~ - hi)); the latent is exact in bf16, the products are exact and the
// MFMA accumulates in fp32, so the only rounding left is ~2^-16 relative in
// q~ plus fp32 accumulation.  A bf16 q~ input takes a single pass.
//
// Structure (one workgroup = 4 wavefronts):
//  * The flattened list of 64-token pages of all queries is split into
//    contiguous ranges, one per workgroup (balances ragged batches).
//  * Pages stream HBM -> LDS with direct-to-LDS loads
//    (global_load_lds_dwordx4), NSTAGE pages in flight, completion tracked
//    with explicit vmcnt waits and a bare s_barrier.  A token row of 512 B
//    sits in LDS with its 16-byte chunks XOR-swizzled by (row & 15), so the
//    MFMA operand reads (16 rows x 16 B per pass) are bank-conflict free.
//  * Wavefront (mb, nb) holds the A operand (heads 32mb..32mb+31, all of r,
//    hi and lo) in registers for the whole range and computes the 32x32 tile
//    of heads x tokens 32nb..32nb+31 of each page.
//  * Epilogue per tile: + beta, ReLU, * w, sum over the lane's 16 heads, one
//    cross-lane add (lanes l and l^32 hold the other 16 heads), then the two
//    head halves meet through LDS one page later (no extra barrier).
//  * Candidate mode (hierarchical selection): "pages" are 64 candidate slots
//    whose rows are gathered through the block table; physical rows are
//    resolved into LDS before streaming.
#include <algorithm>

#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

#define LDS3 __attribute__((address_space(3)))

constexpr int kThreads = 256;
constexpr int kMaxPagesPerWG = 512;   // page mode
constexpr int kMaxPagesGather = 16;   // candidate mode

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

union Frag {
  bf16x8 v;
  uint32_t u[4];
};

template <int R, int NSTAGE>
struct MfmaShared {
  static constexpr int kRowBytes = R * 2;
  __align__(16) char stage[NSTAGE][kPage * kRowBytes];
  float red[2][2][32];
  int32_t pq[kMaxPagesPerWG];
  int32_t ppg[kMaxPagesPerWG];
  int32_t prow[kMaxPagesPerWG];  // page mode: physical block; candidate mode: see gather_rows
  int32_t gather_rows[kMaxPagesGather * kPage];
  int32_t np;
};

__device__ __forceinline__ int qpages(const int32_t *q_len, int i) { return (q_len[i] + 63) >> 6; }

// Wave 0 works out this workgroup's page range and writes (query, page) per
// local page into LDS.  Returns nothing; sh.np holds the page count.
template <typename SH>
__device__ void plan_range(SH &sh, int n_q, const int32_t *q_len, int cap) {
  const int lane = threadIdx.x % kWave;
  if (threadIdx.x >= kWave) return;
  int64_t T = 0;
  for (int c = 0; c < n_q; c += kWave) {
    const int i = c + lane;
    int np = i < n_q ? qpages(q_len, i) : 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) np += __shfl_xor(np, o, kWave);
    T += np;
  }
  const int64_t G = gridDim.x, g = blockIdx.x;
  const int64_t f0 = g * T / G, f1 = (g + 1) * T / G;
  // The host sizes the grid so that cnt <= cap whenever every q_len honours
  // the bound it was given; the clamp keeps a violating call memory-safe.
  const int cnt = (int)min<int64_t>(f1 - f0, cap);
  int q0 = 0, pg0 = 0;
  int64_t cum = 0;
  if (cnt > 0) {
    for (int c = 0; c < n_q; c += kWave) {
      const int i = c + lane;
      const int np = i < n_q ? qpages(q_len, i) : 0;
      int incl = np;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        int y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
      }
      const unsigned long long hit = __ballot(cum + incl > f0);
      if (hit) {
        const int fl = __ffsll((long long)hit) - 1;
        const int np_f = __shfl(np, fl, kWave);
        const int incl_f = __shfl(incl, fl, kWave);
        q0 = c + fl;
        pg0 = (int)(f0 - (cum + incl_f - np_f));
        break;
      }
      cum += __shfl(incl, kWave - 1, kWave);
    }
  }
  if (lane == 0) {
    int q = q0, pg = pg0, qp = cnt > 0 ? qpages(q_len, q) : 0;
    for (int p = 0; p < cnt; ++p) {
      sh.pq[p] = q;
      sh.ppg[p] = pg;
      if (++pg == qp) {
        pg = 0;
        do {
          ++q;
        } while (q < n_q && (qp = qpages(q_len, q)) == 0);
      }
    }
    sh.np = cnt;
  }
}

template <int R, int NSTAGE, bool HILO>
__global__ void __launch_bounds__(kThreads, 1)
score_mfma_kernel(const void *__restrict__ q_tilde, const float *__restrict__ w,
                  const float *__restrict__ beta, int n_q, const int32_t *__restrict__ q_seq,
                  const int32_t *__restrict__ q_len, CacheView cv, const int32_t *__restrict__ cand,
                  int B, float *__restrict__ out, int64_t ld) {
  using SH = MfmaShared<R, NSTAGE>;
  constexpr int kRowBytes = SH::kRowBytes;
  constexpr int kChunks = R / 8;                 // 16-byte chunks per token row
  constexpr int kRowsPerInst = kWave / kChunks;  // token rows per wave-wide 1 KB load
  constexpr int kInstPerPage = kPage / kRowsPerInst;
  constexpr int kInstPerWave = kInstPerPage / 4;
  constexpr int kSwz = kChunks - 1 < 15 ? kChunks - 1 : 15;
  constexpr int KB = R / 16;  // MFMA k-steps
  static_assert(kInstPerWave * 4 == kInstPerPage, "page must split over 4 waves");

  __shared__ SH sh;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int mb = wave & 1, nb = wave >> 1;
  const bool gather = cand != nullptr;

  plan_range(sh, n_q, q_len, gather ? kMaxPagesGather : kMaxPagesPerWG);
  __syncthreads();
  const int np = sh.np;
  if (np == 0) return;
  if (!gather) {
    for (int p = tid; p < np; p += kThreads)
      sh.prow[p] = cv.block_table[(int64_t)q_seq[sh.pq[p]] * cv.max_blocks + sh.ppg[p]];
  } else {
    for (int e = tid; e < np * kPage; e += kThreads) {
      const int p = e >> 6, row = e & 63;
      const int q = sh.pq[p];
      const int n = q_len[q];
      const int slot = min(sh.ppg[p] * kPage + row, n - 1);
      const int t = cand[(int64_t)q * B + slot];
      sh.gather_rows[e] =
          cv.block_table[(int64_t)q_seq[q] * cv.max_blocks + (t >> 6)] * kPage + (t & 63);
    }
  }
  __syncthreads();

  const char *gdata = (const char *)cv.data;
  auto issue_page = [&](int p, int s) {
    LDS3 char *dst = (LDS3 char *)sh.stage[s];
#pragma unroll
    for (int m = 0; m < kInstPerWave; ++m) {
      const int gi = wave * kInstPerWave + m;
      const int row = gi * kRowsPerInst + lane / kChunks;
      const int chunk = (lane % kChunks) ^ (row & kSwz);
      int64_t grow;
      if (!gather)
        grow = (int64_t)sh.prow[p] * kPage + row;
      else
        grow = sh.gather_rows[p * kPage + row];
      const char *src = gdata + grow * kRowBytes + chunk * 16;
      __builtin_amdgcn_global_load_lds((const void *)src, (LDS3 void *)(dst + gi * 1024), 16, 0, 0);
    }
  };

  // A operand of this wavefront: heads 32*mb + (lane % 32), k = kb*16 + (lane/32)*8 + [0, 8)
  Frag ahi[KB], alo[HILO ? KB : 1];
  float wv[16], bv[16];
  int cur_q = -1;
  auto load_query = [&](int q) {
    const int head = 32 * mb + (lane & 31);
    if constexpr (HILO) {
      const float *src = (const float *)q_tilde + ((int64_t)q * 64 + head) * R + (lane >> 5) * 8;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const float4 x0 = *(const float4 *)(src + kb * 16);
        const float4 x1 = *(const float4 *)(src + kb * 16 + 4);
        const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t h0 = f32_to_bf16_bits(xs[2 * e]), h1 = f32_to_bf16_bits(xs[2 * e + 1]);
          const uint32_t l0 = f32_to_bf16_bits(xs[2 * e] - bf16_bits_to_f32(h0));
          const uint32_t l1 = f32_to_bf16_bits(xs[2 * e + 1] - bf16_bits_to_f32(h1));
          ahi[kb].u[e] = h0 | (h1 << 16);
          alo[kb].u[e] = l0 | (l1 << 16);
        }
      }
    } else {
      const uint16_t *src = (const uint16_t *)q_tilde + ((int64_t)q * 64 + head) * R + (lane >> 5) * 8;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint4 x = *(const uint4 *)(src + kb * 16);
        ahi[kb].u[0] = x.x;
        ahi[kb].u[1] = x.y;
        ahi[kb].u[2] = x.z;
        ahi[kb].u[3] = x.w;
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int h = 32 * mb + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
      wv[j] = w[(int64_t)q * 64 + h];
      bv[j] = beta ? beta[(int64_t)q * 64 + h] : 0.f;
    }
    cur_q = q;
  };

  load_query(sh.pq[0]);
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s)
    if (s < np) issue_page(s, s);

  float carry = 0.f;  // mb == 0: this wave's half of the previous page's scores
  for (int p = 0; p < np; ++p) {
    // pages issued after p and still possibly in flight: p+1 .. min(p+NSTAGE-2, np-1)
    const int after = min(NSTAGE - 2, np - 1 - p);
    if (after >= 2) wait_vmcnt<2 * kInstPerWave>();
    else if (after == 1) wait_vmcnt<kInstPerWave>();
    else wait_vmcnt<0>();
    lds_barrier();

    if (mb == 0 && p > 0 && lane < 32) {
      const int pp = p - 1, q = sh.pq[pp];
      const int t = sh.ppg[pp] * kPage + nb * 32 + lane;
      if (t < q_len[q]) out[(int64_t)q * ld + t] = carry + sh.red[pp & 1][nb][lane];
    }
    if (sh.pq[p] != cur_q) load_query(sh.pq[p]);
    if (p + NSTAGE - 1 < np) issue_page(p + NSTAGE - 1, (p + NSTAGE - 1) % NSTAGE);

    const char *sp = sh.stage[p % NSTAGE];
    const int row = nb * 32 + (lane & 31);
    const char *rp = sp + row * kRowBytes;
    f32x16 acc = {};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int chunk = (kb * 2 + (lane >> 5)) ^ (row & kSwz);
      const bf16x8 b = *(const bf16x8 *)(rp + chunk * 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[kb].v, b, acc, 0, 0, 0);
      if constexpr (HILO) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[kb].v, b, acc, 0, 0, 0);
    }
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) part = fmaf(wv[j], fmaxf(acc[j] + bv[j], 0.f), part);
    part += __shfl_xor(part, 32, kWave);
    if (mb == 1) {
      if (lane < 32) sh.red[p & 1][nb][lane] = part;
    } else {
      carry = part;
    }
  }
  lds_barrier();
  if (mb == 0 && lane < 32) {
    const int pp = np - 1, q = sh.pq[pp];
    const int t = sh.ppg[pp] * kPage + nb * 32 + lane;
    if (t < q_len[q]) out[(int64_t)q * ld + t] = carry + sh.red[pp & 1][nb][lane];
  }
}

int g_num_cu = 0;

template <int R, int NSTAGE, bool HILO>
hipError_t launch_t(const void *q_tilde, const float *w, const float *beta, int n_q,
                    const int32_t *q_seq, const int32_t *q_len, int max_len, const CacheView &cv,
                    const int32_t *cand, int B, float *out, int64_t ld, hipStream_t st) {
  if (g_num_cu == 0) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&g_num_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (g_num_cu <= 0) g_num_cu = 256;
  }
  const int64_t per_q = cand ? (B + 63) / 64 : (max_len + 63) / 64;
  const int64_t T_ub = (int64_t)n_q * per_q;
  const int cap = cand ? kMaxPagesGather : kMaxPagesPerWG;
  int64_t G = std::min<int64_t>(T_ub, g_num_cu);
  G = std::max<int64_t>(G, (T_ub + cap - 1) / cap);
  if (G <= 0) return hipSuccess;
  score_mfma_kernel<R, NSTAGE, HILO><<<(unsigned)G, kThreads, 0, st>>>(
      q_tilde, w, beta, n_q, q_seq, q_len, cv, cand, B, out, ld);
  return hipGetLastError();
}

}  // namespace

bool score_mfma_supported(int qt_dt, int H, const CacheView &cv) {
  return H == 64 && cv.dtype == LI_BF16 && cv.r == 256 && (qt_dt == LI_FP32 || qt_dt == LI_BF16);
}

hipError_t launch_score_mfma(const void *q_tilde, int qt_dt, const float *w, const float *beta,
                             int n_q, int H, const int32_t *q_seq, const int32_t *q_len,
                             int max_len, const CacheView &cv, const int32_t *cand, int B,
                             float *out, int64_t ld, hipStream_t st) {
  (void)H;
  if (qt_dt == LI_FP32)
    return launch_t<256, 4, true>(q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, cand, B, out,
                                  ld, st);
  return launch_t<256, 4, false>(q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, cand, B, out,
                                 ld, st);
}

}  // namespace li
