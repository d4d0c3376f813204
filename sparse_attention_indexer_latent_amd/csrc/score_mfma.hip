// Matrix-core scorer for eq. (8) of the LatentIndex summary ("Methodology"):
// u_t = sum_h w_h ReLU(q~_h . c_t + beta_h), for H = 64 heads over a bf16
// latent cache.
//
// Why matrix cores: one cached token of r = 256 bf16 values (512 B) meets 64
// absorbed queries, 2*64*256 = 32768 flop, i.e. 64 flop per byte read, three
// times the fp32 vector ridge of MI355X (157 TFLOP/s / 8 TB/s).  The product
// [64 heads x r] x [r x tokens] is a real dense contraction even for a single
// decode query, so it runs on v_mfma_f32_16x16x32_bf16 and the kernel stays
// bound by the HBM stream of the latent.
//
// Precision: an fp32 q~ is carried as bf16 hi + lo (hi = RNE(q~), lo =
// RNE(q~ - hi)); the latent is exact in bf16, the products are exact and the
// MFMA accumulates in fp32, so the only rounding left is ~2^-16 relative in
// q~ plus fp32 accumulation.  A bf16 q~ input takes a single pass.
//
// Structure (one workgroup = 8 wavefronts, two per SIMD, one per CU):
//  * The flattened list of 64-token pages of all queries is split into
//    contiguous ranges, one per workgroup (balances ragged batches).  The
//    exact plan and the block ids of the range cost two global round trips;
//    the common decode shape (every query max_len long, query q on
//    sequence q) is guessed at entry, so its first pages stream after one.
//  * Pages stream HBM -> LDS with direct-to-LDS loads
//    (global_load_lds_dwordx4), NSTAGE pages in flight, completion tracked
//    with explicit vmcnt waits and a bare s_barrier.  A token row of 512 B
//    sits in LDS with its 16-byte chunks XOR-swizzled by (row & 15), so the
//    MFMA operand reads (16 rows x 16 B per pass) are bank-conflict free.
//  * Wavefront w holds the A operand of heads 16*(w%4) .. +15 (all of r, hi
//    and lo: 64 VGPRs) for the whole range and computes heads x tokens
//    32*(w/4) .. +31 of each page as two 16x16 tiles.
//  * Epilogue per tile: + beta, ReLU, * w, sum over the lane's 4 heads, two
//    cross-lane adds (the 16 heads of the group), then the four head groups
//    meet through LDS one page later (no extra barrier).
//  * Candidate mode (hierarchical selection): "pages" are 64 candidate slots
//    whose physical rows were resolved beforehand; each query owns exactly
//    ceil(B/64) such pages, so the range plan needs no loads.
#include <algorithm>

#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

#define LDS3 __attribute__((address_space(3)))

constexpr int kMaxPagesPerWG = 512;   // page mode
constexpr int kMaxPagesGather = 16;   // candidate mode

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding:
// vmcnt[3:0] at bits 3:0, vmcnt[5:4] at bits 15:14, expcnt and lgkmcnt at max).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

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

__device__ __forceinline__ int qpages(const int32_t *q_len, int i) { return (q_len[i] + 63) >> 6; }

// Wave 0 works out this workgroup's contiguous range of the flattened
// (query, page) list and writes (query, page, sequence) per local page into
// LDS.  len0/seq0 hold the lengths and sequence ids of the first 64 queries
// (lane i: query i), loaded by the caller; later queries are read from
// memory.  sh.np receives the page count, clamped to cap (the host sizing
// guarantees the range fits whenever every q_len honours its bound).
template <typename SH>
__device__ void plan_range(SH &sh, int n_q, const int32_t *q_len, const int32_t *q_seq, int cap,
                           int len0, int seq0) {
  const int lane = threadIdx.x % kWave;
  const int np0 = (len0 + 63) >> 6;
  auto pages_of = [&](int q) { return q < kWave ? __shfl(np0, q, kWave) : qpages(q_len, q); };
  auto seq_of = [&](int q) { return q < kWave ? __shfl(seq0, q, kWave) : q_seq[q]; };
  int64_t T = 0;
  for (int c = 0; c < n_q; c += kWave) {
    int np = c == 0 ? np0 : (c + lane < n_q ? qpages(q_len, c + lane) : 0);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) np += __shfl_xor(np, o, kWave);
    T += np;
  }
  const int64_t G = gridDim.x, g = blockIdx.x;
  const int64_t f0 = g * T / G, f1 = (g + 1) * T / G;
  const int cnt = (int)min<int64_t>(f1 - f0, cap);
  int q0 = 0, pg0 = 0;
  int64_t cum = 0;
  if (cnt > 0) {
    for (int c = 0; c < n_q; c += kWave) {
      const int np = c == 0 ? np0 : (c + lane < n_q ? qpages(q_len, c + lane) : 0);
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
  // uniform walk over the range (the whole wavefront executes it)
  int q = q0, pg = pg0;
  int qp = cnt > 0 ? pages_of(q) : 0, sq = cnt > 0 ? seq_of(q) : 0;
  for (int p = 0; p < cnt; ++p) {
    if (lane == 0) {
      sh.pq[p] = q;
      sh.ppg[p] = pg;
      sh.pseq[p] = sq;
    }
    if (++pg == qp) {
      pg = 0;
      do {
        ++q;
      } while (q < n_q && (qp = pages_of(q)) == 0);
      if (q < n_q) sq = seq_of(q);
    }
  }
  if (lane == 0) sh.np = cnt;
}

// ---------------------------------------------------------------------------
// Eight-wavefront variant on v_mfma_f32_16x16x32_bf16: wavefront w owns heads
// 16*(w%4) .. +15 (its hi/lo operand is 64 VGPRs) and tokens 32*(w/4) .. +31
// of every page (two 16-token tiles).  Two wavefronts per SIMD hide the LDS,
// MFMA-result and barrier latencies that a single wavefront per SIMD exposes.
// The four head groups meet through LDS one page later.
// ---------------------------------------------------------------------------
template <int R, int NSTAGE>
struct MfmaShared {
  static constexpr int kRowBytes = R * 2;
  __align__(16) char stage[NSTAGE][kPage * kRowBytes];
  float red[2][4][kPage];
  int32_t pq[kMaxPagesPerWG];
  int32_t ppg[kMaxPagesPerWG];
  int32_t pseq[kMaxPagesPerWG];
  int32_t prow[kMaxPagesPerWG];
  int32_t gather_rows[kMaxPagesGather * kPage];
  int32_t np;
  int32_t spec_ok;
};

constexpr int kThreads = 512;
static_assert(kMaxPagesPerWG <= kThreads, "one block id per thread in the speculative plan");

template <int R, int NSTAGE, bool HILO, bool GATHER>
__global__ void __launch_bounds__(kThreads, 1)
score_mfma_kernel(const void *__restrict__ q_tilde, const float *__restrict__ w,
                    const float *__restrict__ beta, int n_q, const int32_t *__restrict__ q_seq,
                    const int32_t *__restrict__ q_len, int max_len, CacheView cv,
                    const int32_t *__restrict__ cand, int B, float *__restrict__ out, int64_t ld) {
  using SH = MfmaShared<R, NSTAGE>;
  constexpr int kRowBytes = SH::kRowBytes;
  constexpr int kChunks = R / 8;
  constexpr int kRowsPerInst = kWave / kChunks;
  constexpr int kInstPerPage = kPage / kRowsPerInst;
  constexpr int kWaves = kThreads / kWave;
  constexpr int kInstPerWave = kInstPerPage / kWaves;
  constexpr int kSwz = kChunks - 1 < 15 ? kChunks - 1 : 15;
  constexpr int KB = R / 32;  // MFMA k-steps of 32
  static_assert(kInstPerWave * kWaves == kInstPerPage, "page must split over the waves");

  __shared__ SH sh;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int hg = wave & 3, nh = wave >> 2;
  constexpr bool gather = GATHER;

  // A operand: head 16*hg + (lane % 16), k = kb*32 + (lane/16)*8 + [0, 8)
  Frag ahi[KB], alo[HILO ? KB : 1];
  float wv[4], bv[4];
  int cur_q = -1;
  auto load_query = [&](int q, bool drain) {
    const int head = 16 * hg + (lane & 15);
    if constexpr (HILO) {
      const float *src = (const float *)q_tilde + ((int64_t)q * 64 + head) * R + (lane >> 4) * 8;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const float4 x0 = *(const float4 *)(src + kb * 32);
        const float4 x1 = *(const float4 *)(src + kb * 32 + 4);
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
      const uint16_t *src = (const uint16_t *)q_tilde + ((int64_t)q * 64 + head) * R + (lane >> 4) * 8;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint4 x = *(const uint4 *)(src + kb * 32);
        ahi[kb].u[0] = x.x;
        ahi[kb].u[1] = x.y;
        ahi[kb].u[2] = x.z;
        ahi[kb].u[3] = x.w;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * hg + 4 * (lane >> 4) + i;
      wv[i] = w[(int64_t)q * 64 + h];
      bv[i] = beta ? beta[(int64_t)q * 64 + h] : 0.f;
    }
    cur_q = q;
    // Complete these loads here, with a wait the compiler sees: otherwise its
    // merged view of the page loop makes every later use of them wait for all
    // outstanding loads, in-flight latent pages included.
    if (drain) __builtin_amdgcn_s_waitcnt(0);
  };

  const char *gdata = (const char *)cv.data;
  auto issue_page = [&](int p, int s) {
    LDS3 char *dst = (LDS3 char *)sh.stage[s];
    const char *page_base = gdata;
    if constexpr (!gather) page_base += (int64_t)sh.prow[p] * kPage * kRowBytes;
#pragma unroll
    for (int m = 0; m < kInstPerWave; ++m) {
      const int gi = wave * kInstPerWave + m;
      const int row = gi * kRowsPerInst + lane / kChunks;
      const int chunk = (lane % kChunks) ^ (row & kSwz);
      const char *src;
      if constexpr (!gather)
        src = page_base + row * kRowBytes + chunk * 16;
      else
        src = gdata + (int64_t)max(sh.gather_rows[p * kPage + row], 0) * kRowBytes + chunk * 16;
      __builtin_amdgcn_global_load_lds((const void *)src, (LDS3 void *)(dst + gi * 1024), 16, 0, 0);
    }
  };

  int issued = 0;  // local pages whose loads are in flight
  if constexpr (!gather) {
    // Speculative plan for the common decode case, every query with
    // ceil(max_len / 64) pages and query q reading sequence q: its block ids
    // and first query operands load together with the real lengths, and the
    // first pages stream at once.  Block ids are clamped into the pool, so a
    // wrong guess costs bandwidth only; it is detected below, drained, and
    // the exact plan replaces it.
    const int PPQ = (max_len + kPage - 1) / kPage;
    const bool try_spec = n_q <= kWave && n_q <= cv.n_seq && PPQ > 0 && PPQ <= cv.max_blocks;
    int cnt_s = 0;
    int64_t f0s = 0;
    if (try_spec) {
      const int64_t T = (int64_t)n_q * PPQ, G = gridDim.x, g = blockIdx.x;
      f0s = g * T / G;
      cnt_s = (int)min<int64_t>((g + 1) * T / G - f0s, kMaxPagesPerWG);
    }
    int len0 = 0, seq0 = 0;
    if (wave == 0) {  // real lengths and sequence ids of the first 64 queries
      len0 = lane < n_q ? q_len[lane] : 0;
      seq0 = lane < n_q ? q_seq[lane] : 0;
    }
    int sq = 0, spg = 0, sblk = 0;
    if (tid < cnt_s) {
      sq = (int)((f0s + tid) / PPQ);
      spg = (int)((f0s + tid) % PPQ);
      sblk = cv.block_table[(int64_t)sq * cv.max_blocks + spg];
    }
    if (cnt_s > 0) load_query((int)(f0s / PPQ), false);
    if (tid < cnt_s) {
      sh.prow[tid] = (sblk >= 0 && sblk < cv.n_blocks) ? sblk : 0;
      sh.pq[tid] = sq;
      sh.ppg[tid] = spg;
    }
    lds_barrier();
    for (; issued < NSTAGE - 1 && issued < cnt_s; ++issued) issue_page(issued, issued);
    if (wave == 0) {
      // the guess is the exact plan iff every query has PPQ pages and reads
      // its own sequence
      const bool bad = lane < n_q && (((len0 + kPage - 1) / kPage) != PPQ || seq0 != lane);
      const bool ok = try_spec && __ballot(bad) == 0ull;
      if (lane == 0) sh.spec_ok = ok ? 1 : 0;
      if (!ok) plan_range(sh, n_q, q_len, q_seq, kMaxPagesPerWG, len0, seq0);
      else if (lane == 0) sh.np = cnt_s;
    }
    lds_barrier();
    if (!sh.spec_ok) {
      // drain the speculative page loads before their LDS slots are reused
      // (the operands of a query do not depend on the plan: cur_q stays)
      __builtin_amdgcn_s_waitcnt(0);
      issued = 0;
      for (int p = tid; p < sh.np; p += kThreads)
        sh.prow[p] = cv.block_table[(int64_t)sh.pseq[p] * cv.max_blocks + sh.ppg[p]];
      __syncthreads();
    }
  } else {
    // Every query owns exactly ceil(B / 64) candidate slot pages: the range
    // needs no loads.  Padding slots (cand == -1) read pool row 0 and store
    // -inf.
    const int PB = (B + kPage - 1) / kPage;
    const int64_t T = (int64_t)n_q * PB, G = gridDim.x, g = blockIdx.x;
    const int64_t f0 = g * T / G;
    const int cnt = (int)min<int64_t>((g + 1) * T / G - f0, kMaxPagesGather);
    for (int p = tid; p < cnt; p += kThreads) {
      sh.pq[p] = (int)((f0 + p) / PB);
      sh.ppg[p] = (int)((f0 + p) % PB);
    }
    if (tid == 0) sh.np = cnt;
    // the first query is known without loads: fetch its operands now, in
    // parallel with the candidate -> row lookups below
    if (cnt > 0) load_query((int)(f0 / PB), false);
    __syncthreads();
    for (int e = tid; e < sh.np * kPage; e += kThreads) {
      const int p = e >> 6, row = e & 63;
      const int q = sh.pq[p];
      const int slot = min(sh.ppg[p] * kPage + row, B - 1);
      const int t = cand[(int64_t)q * B + slot];
      sh.gather_rows[e] =
          t >= 0 ? cv.block_table[(int64_t)q_seq[q] * cv.max_blocks + (t >> 6)] * kPage + (t & 63)
                 : -1;
    }
    __syncthreads();
  }
  const int np = sh.np;
  if (np == 0) return;

  // Prologue: page 0's loads, then this query's operands, then the next
  // pages; waiting until at most the last pages' loads remain outstanding
  // completes page 0 and the operands (loads return in order).  A correct
  // guess has already issued them.
  if (issued == 0) {
    issue_page(0, 0);
    if (cur_q != sh.pq[0]) load_query(sh.pq[0], false);
    issued = 1;
  }
  for (; issued < NSTAGE - 1 && issued < np; ++issued) issue_page(issued, issued);
  {
    const int later = min(NSTAGE - 2, np - 1);
    if (later >= 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kInstPerWave));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kInstPerWave));
    else __builtin_amdgcn_s_waitcnt(0);
  }

  // Final score of token (or slot) nh*32 + lane of local page pp: this
  // wave's head-group share plus the other three groups' shares from LDS.
  auto store_score = [&](int pp, float own) {
    const int q = sh.pq[pp];
    const int tk = nh * 32 + lane;
    const int t = sh.ppg[pp] * kPage + tk;
    const float *rd = &sh.red[pp & 1][0][0];
    const float v = ((own + rd[kPage + tk]) + rd[2 * kPage + tk]) + rd[3 * kPage + tk];
    if constexpr (!gather) {
      if (t < q_len[q]) out[(int64_t)q * ld + t] = v;
    } else {
      if (t < B) out[(int64_t)q * ld + t] = sh.gather_rows[pp * kPage + tk] >= 0 ? v : -INFINITY;
    }
  };
  float carry = 0.f;  // hg == 0: this wave's head group share of the previous page
  for (int p = 0; p < np; ++p) {
    const int after = min(NSTAGE - 2, np - 1 - p);
    if (after >= 2) wait_vmcnt<2 * kInstPerWave>();
    else if (after == 1) wait_vmcnt<kInstPerWave>();
    else wait_vmcnt<0>();
    lds_barrier();

    if (hg == 0 && p > 0 && lane < 32) store_score(p - 1, carry);
    if (sh.pq[p] != cur_q) load_query(sh.pq[p], true);
    if (p + NSTAGE - 1 < np) issue_page(p + NSTAGE - 1, (p + NSTAGE - 1) % NSTAGE);

    const char *sp = sh.stage[p % NSTAGE];
    const int row0 = nh * 32 + (lane & 15), row1 = row0 + 16;
    const char *rp0 = sp + row0 * kRowBytes, *rp1 = sp + row1 * kRowBytes;
    f32x4 acc0 = {}, acc1 = {};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int chunk = kb * 4 + (lane >> 4);
      const bf16x8 b0 = *(const bf16x8 *)(rp0 + ((chunk ^ (row0 & kSwz)) * 16));
      const bf16x8 b1 = *(const bf16x8 *)(rp1 + ((chunk ^ (row1 & kSwz)) * 16));
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[kb].v, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[kb].v, b1, acc1, 0, 0, 0);
      if constexpr (HILO) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[kb].v, b0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[kb].v, b1, acc1, 0, 0, 0);
      }
    }
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p0 = fmaf(wv[i], fmaxf(acc0[i] + bv[i], 0.f), p0);
      p1 = fmaf(wv[i], fmaxf(acc1[i] + bv[i], 0.f), p1);
    }
    p0 += __shfl_xor(p0, 16, kWave);
    p1 += __shfl_xor(p1, 16, kWave);
    p0 += __shfl_xor(p0, 32, kWave);
    p1 += __shfl_xor(p1, 32, kWave);
    const float mine = lane < 16 ? p0 : p1;  // lanes 0..31: token nh*32 + lane
    if (hg != 0) {
      if (lane < 32) sh.red[p & 1][hg][nh * 32 + lane] = mine;
    } else {
      carry = mine;
    }
  }
  lds_barrier();
  if (hg == 0 && lane < 32) store_score(np - 1, carry);
}

int g_num_cu = 0;

template <int R, int NSTAGE, bool HILO, bool GATHER>
hipError_t launch_t(const void *q_tilde, const float *w, const float *beta, int n_q,
                      const int32_t *q_seq, const int32_t *q_len, int max_len, const CacheView &cv,
                      const int32_t *cand, int B, float *out, int64_t ld, hipStream_t st) {
  if (g_num_cu == 0) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&g_num_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (g_num_cu <= 0) g_num_cu = 256;
  }
  const int64_t per_q = GATHER ? (B + 63) / 64 : (max_len + 63) / 64;
  const int64_t T_ub = (int64_t)n_q * per_q;
  const int cap = GATHER ? kMaxPagesGather : kMaxPagesPerWG;
  int64_t G = std::min<int64_t>(T_ub, g_num_cu);
  G = std::max<int64_t>(G, (T_ub + cap - 1) / cap);
  if (G <= 0) return hipSuccess;
  score_mfma_kernel<R, NSTAGE, HILO, GATHER><<<(unsigned)G, kThreads, 0, st>>>(
      q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, cand, B, out, ld);
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
  if (qt_dt == LI_FP32) {
    if (cand)
      return launch_t<256, 4, true, true>(q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, cand,
                                            B, out, ld, st);
    return launch_t<256, 4, true, false>(q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, cand,
                                           B, out, ld, st);
  }
  if (cand)
    return launch_t<256, 4, false, true>(q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, cand,
                                           B, out, ld, st);
  return launch_t<256, 4, false, false>(q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, cand,
                                          B, out, ld, st);
}

}  // namespace li
