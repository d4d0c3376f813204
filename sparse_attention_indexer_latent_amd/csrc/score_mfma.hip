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
// Structure (one workgroup = 4 wavefronts over units of TOK = 32 tokens, two
// workgroups per CU, so one computes while the other waits at a barrier):
//  * The flattened list of units of all queries is split into contiguous
//    ranges, one per workgroup (balances ragged batches).  The exact plan
//    and the block ids of the range cost two global round trips; the common
//    decode shape (every query max_len long, query q on sequence q) is
//    guessed at entry, so its first units stream after one.
//  * Units stream HBM -> LDS with direct-to-LDS loads
//    (global_load_lds_dwordx4), NSTAGE units in flight, completion tracked
//    with explicit vmcnt waits and a bare s_barrier.  A token row of 512 B
//    sits in LDS with its 16-byte chunks XOR-swizzled by (row & 15), so the
//    MFMA operand reads (16 rows x 16 B per pass) are bank-conflict free.
//  * Wavefront w holds the A operand of heads 16w .. 16w+15 (all of r, hi
//    and lo for an fp32 q~) for the whole range and computes the unit's
//    heads x tokens as two 16x16 tiles.
//  * Epilogue per tile: + beta (bf16: the MFMAs' start value), ReLU, * w,
//    sum over the lane's 4 heads, two lane swaps (v_permlane32/16_swap) for
//    the 16 heads of the group, then the four head groups
//    meet through LDS one unit later (no extra barrier); the epilogue of
//    unit p-1 runs while the matrix core works on unit p.
//  * Candidate mode (hierarchical selection): units are candidate slots
//    whose physical rows were resolved beforehand; each query owns exactly
//    ceil(B/TOK) of them, so the range plan needs no loads.
#include <algorithm>

#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

#define LDS3 __attribute__((address_space(3)))
#define INL __attribute__((always_inline))

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

// query i's length, clamped into [0, max_len]
__device__ __forceinline__ int qlen_at(const int32_t *q_len, int i, int max_len) {
  return min(max(q_len[i], 0), max_len);
}
template <int TOK>
__device__ __forceinline__ int qpages(const int32_t *q_len, int i, int max_len) {
  return (qlen_at(q_len, i, max_len) + TOK - 1) / TOK;
}

// Wave 0 works out this workgroup's contiguous range of the flattened
// (query, page) list and writes (query, page, sequence) per local page into
// LDS.  len0/seq0 hold the lengths and sequence ids of the first 64 queries
// (lane i: query i), loaded by the caller; later queries are read from
// memory.  sh.np receives the page count, clamped to cap (the host sizing
// guarantees the range fits whenever every q_len honours its bound).
template <int TOK, typename SH>
__device__ void plan_range(SH &sh, int n_q, const int32_t *q_len, const int32_t *q_seq, int cap,
                           int len0, int seq0, int max_len) {
  const int lane = threadIdx.x % kWave;
  const int np0 = (len0 + TOK - 1) / TOK;
  auto pages_of = [&](int q) { return q < kWave ? __shfl(np0, q, kWave) : qpages<TOK>(q_len, q, max_len); };
  auto seq_of = [&](int q) { return q < kWave ? __shfl(seq0, q, kWave) : q_seq[q]; };
  int64_t T = 0;
  for (int c = 0; c < n_q; c += kWave) {
    int np = c == 0 ? np0 : (c + lane < n_q ? qpages<TOK>(q_len, c + lane, max_len) : 0);
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
      const int np = c == 0 ? np0 : (c + lane < n_q ? qpages<TOK>(q_len, c + lane, max_len) : 0);
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
// Four wavefronts per workgroup: wavefront w owns heads 16w .. 16w+15 of
// every 32-token unit (two 16-token tiles).  Two workgroups per CU (two
// wavefronts per SIMD) hide the LDS, MFMA-result and barrier latencies that
// a single wavefront per SIMD exposes.  The four head groups meet through
// LDS one unit later.
//
// bf16 cache: v_mfma_f32_16x16x32_bf16; an fp32 q~ is carried as bf16 hi + lo.
// fp8 cache (E4M3FN + per-token fp32 scale): v_mfma_f32_16x16x128_f8f6f4 with
// both operands fp8.  q~ of each head is first scaled by a power of two that
// brings its largest element into (224, 448], then split into three fp8
// terms t0 + t1 + t2 (each the E4M3 rounding of what the previous terms left),
// which represents it to about 2^-12 relative; a bf16 q~ (8 significant bits)
// needs two.  The matrix core sums a 128-long fp8 product group with about
// 2^-11 of its largest product as resolution (measured on gfx950), well inside
// the fp8 tolerance.  The token's scale and the head's power of two are applied
// to the fp32 dot product, before beta and ReLU.
// ---------------------------------------------------------------------------
template <int ROWB, int NSTAGE, int TOK>
struct MfmaShared {
  __align__(16) char stage[NSTAGE][TOK * ROWB];
  float ssc[NSTAGE][TOK];  // fp8: per-token scales of the staged unit
  float red[2][4][TOK];
  int32_t pq[kMaxPagesPerWG];
  int32_t ppg[kMaxPagesPerWG];
  int32_t pseq[kMaxPagesPerWG];
  int32_t prow[kMaxPagesPerWG];
  int32_t gather_rows[kMaxPagesGather * TOK];
  int32_t pvalid[kMaxPagesPerWG];  // page mode: valid tokens of each local unit
  int32_t qlen[kWave];  // lengths of the first 64 queries
  int32_t qcum[kWave];  // exact plan: inclusive page counts of the first 64 queries
  int32_t qseq[kWave];
  int32_t np;
  int64_t f0;
  int32_t spec_ok;
};


// s_waitcnt vmcnt(n * PER) for a runtime n in [0, NMAX]
template <int PER, int NMAX>
__device__ __forceinline__ void wait_pages(int n) {
  if constexpr (NMAX > 0) {
    if (n >= NMAX) {
      wait_vmcnt<NMAX * PER>();
      return;
    }
    wait_pages<PER, NMAX - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}
template <int PER, int NMAX>
__device__ __forceinline__ void wait_pages_builtin(int n) {
  if constexpr (NMAX > 0) {
    if (n >= NMAX) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(NMAX * PER));
      return;
    }
    wait_pages_builtin<PER, NMAX - 1>(n);
  } else {
    __builtin_amdgcn_s_waitcnt(0);
  }
}

// Power-of-two exponent k with m * 2^k in (224, 448] for m > 0 (0 for m == 0).
__device__ __forceinline__ int fp8_head_exponent(float m) {
  if (!(m > 0.f)) return 0;
  const uint32_t u = __float_as_uint(m);
  const int E = (int)((u >> 23) & 0xFF) - 127;
  const uint32_t mant = u & 0x7FFFFFu;  // m = (1 + mant/2^23) * 2^E for normal m
  int k = (mant <= 0x600000u ? 8 : 7) - E;  // 1.75 = 1 + 0x600000/2^23
  return min(k, 126);
}

template <int R, int NSTAGE, bool C8, bool QF32, bool GATHER, int TOK>
__global__ void __launch_bounds__(TOK * 8, 64 / TOK)
score_mfma_kernel(const void *__restrict__ q_tilde, const float *__restrict__ w,
                    const float *__restrict__ beta, int n_q, const int32_t *__restrict__ q_seq,
                    const int32_t *__restrict__ q_len, int max_len, CacheView cv,
                    const int32_t *__restrict__ cand, int B, int cand_rows, float *__restrict__ out,
                    int64_t ld) {
  constexpr int kRowBytes = C8 ? R : 2 * R;
  using SH = MfmaShared<kRowBytes, NSTAGE, TOK>;
  constexpr int kThreads = TOK * 8;  // one wavefront per (head group, 32 tokens)
  constexpr int kChunks = kRowBytes / 16;
  constexpr int kRowsPerInst = kWave / kChunks;
  constexpr int kInstPerPage = TOK / kRowsPerInst;
  constexpr int kWaves = kThreads / kWave;
  constexpr int kInstPerWave = kInstPerPage / kWaves;
  constexpr int kVm = kInstPerWave + (C8 ? 1 : 0);  // loads per page per wave (fp8: + scales)
  constexpr int kSwz = kChunks - 1 < 15 ? kChunks - 1 : 15;
  constexpr int KB = C8 ? R / 128 : R / 32;  // MFMA k-steps
  constexpr int NT = C8 ? (QF32 ? 3 : 2) : (QF32 ? 2 : 1);  // A operand terms
  static_assert(kInstPerWave * kWaves == kInstPerPage, "page must split over the waves");
  static_assert(!C8 || kWaves * 8 == TOK, "fp8: eight scales per wavefront");

  __shared__ SH sh;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int hg = wave & 3, nh = wave >> 2;
  constexpr bool gather = GATHER;

  // A operand of head 16*hg + (lane % 16).  bf16: k = kb*32 + (lane/16)*8 +
  // [0, 8); fp8: k = kb*128 + (lane/16)*32 + [0, 32).  Either way a lane
  // holds 64 elements in eight runs of 8 ("chunks").
  Frag abf[NT][C8 ? 1 : KB];
  i32x8 a8[NT][C8 ? KB : 1];
  float wv[4], bv[4], hs[4];  // hs: fp8 head scale 2^-k
  int cur_q = -1;
  // Raw operands: fetched first, converted once they have landed, so that the
  // loads can be issued early and overlap other round trips.
  constexpr int kRawPerChunk = QF32 ? 8 : 4;  // 32-bit words per chunk
  uint32_t qraw[8 * kRawPerChunk];
  float wraw[4], braw[4];
  auto chunk_off = [&](int c) INL -> int {  // element offset of chunk c within the head row
    if constexpr (C8) return (c >> 2) * 128 + (lane >> 4) * 32 + (c & 3) * 8;
    else return c * 32 + (lane >> 4) * 8;
  };
  auto fetch_query = [&](int q) INL {
    const int64_t row = ((int64_t)q * 64 + 16 * hg + (lane & 15)) * R;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if constexpr (QF32) {
        const float *src = (const float *)q_tilde + row + chunk_off(c);
        const uint4 x0 = *(const uint4 *)src, x1 = *(const uint4 *)(src + 4);
        qraw[8 * c + 0] = x0.x; qraw[8 * c + 1] = x0.y; qraw[8 * c + 2] = x0.z; qraw[8 * c + 3] = x0.w;
        qraw[8 * c + 4] = x1.x; qraw[8 * c + 5] = x1.y; qraw[8 * c + 6] = x1.z; qraw[8 * c + 7] = x1.w;
      } else {
        const uint4 x = *(const uint4 *)((const uint16_t *)q_tilde + row + chunk_off(c));
        qraw[4 * c + 0] = x.x; qraw[4 * c + 1] = x.y; qraw[4 * c + 2] = x.z; qraw[4 * c + 3] = x.w;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 16 * hg + 4 * (lane >> 4) + i;
      wraw[i] = w[(int64_t)q * 64 + h];
      braw[i] = beta ? beta[(int64_t)q * 64 + h] : 0.f;
    }
  };
  auto elem = [&](int c, int j) INL -> float {  // element j of chunk c as fp32
    if constexpr (QF32) return __uint_as_float(qraw[8 * c + j]);
    else {
      const uint32_t u = qraw[4 * c + (j >> 1)];
      return bf16_bits_to_f32((j & 1) ? (u >> 16) : (u & 0xFFFFu));
    }
  };
  auto finish_query = [&](int q) INL {
    if constexpr (!C8) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (QF32) {
            // v_cvt_pk_bf16_f32 rounds a pair to nearest even in one step
            const float x0 = elem(kb, 2 * e), x1 = elem(kb, 2 * e + 1);
            const bf16x2 h = {(__bf16)x0, (__bf16)x1};
            const uint32_t hu = __builtin_bit_cast(uint32_t, h);
            const bf16x2 l = {(__bf16)(x0 - __uint_as_float(hu << 16)),
                              (__bf16)(x1 - __uint_as_float(hu & 0xFFFF0000u))};
            abf[0][kb].u[e] = hu;
            abf[NT - 1][kb].u[e] = __builtin_bit_cast(uint32_t, l);
          } else {
            abf[0][kb].u[e] = qraw[4 * kb + e];
          }
        }
      }
    } else {
      float m = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(elem(c, j)));
      m = fmaxf(m, __shfl_xor(m, 16, kWave));
      m = fmaxf(m, __shfl_xor(m, 32, kWave));  // the head's largest |q~|
      const int ke = fp8_head_exponent(m);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ki = __shfl(ke, 4 * (lane >> 4) + i, kWave);  // head 16*hg + 4*(lane/16) + i
        hs[i] = ldexpf(1.f, -ki);
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {  // bytes 4j .. 4j+3 of this k-step's 32
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = ldexpf(elem(4 * kb + (j >> 1), (j & 1) * 4 + e), ke);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            int v = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
            v = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], v, true);
            a8[t][kb][j] = v;
            if (t + 1 < NT) {
              r[0] -= __builtin_amdgcn_cvt_f32_fp8(v, 0);
              r[1] -= __builtin_amdgcn_cvt_f32_fp8(v, 1);
              r[2] -= __builtin_amdgcn_cvt_f32_fp8(v, 2);
              r[3] -= __builtin_amdgcn_cvt_f32_fp8(v, 3);
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wv[i] = wraw[i];
      bv[i] = braw[i];
    }
    cur_q = q;
  };
  auto load_query = [&](int q, bool drain) INL {
    fetch_query(q);
    finish_query(q);
    // Complete these loads here, with a wait the compiler sees: otherwise its
    // merged view of the page loop makes every later use of them wait for all
    // outstanding loads, in-flight latent pages included.
    if (drain) __builtin_amdgcn_s_waitcnt(0);
  };

  // Where a page's rows come from, read from LDS ahead of the issue: page
  // mode, the physical block; candidate mode, each lane's rows (clamped to 0
  // for padding) and, for fp8, its scale row.
  struct PageSrc {
    int r[kInstPerWave];
    int srow;
  };
  auto page_src = [&](int p) INL {
    PageSrc ps;
    if constexpr (!gather) {
      ps.r[0] = sh.prow[p];
    } else {
#pragma unroll
      for (int m = 0; m < kInstPerWave; ++m) {
        const int row = (wave * kInstPerWave + m) * kRowsPerInst + lane / kChunks;
        ps.r[m] = max(sh.gather_rows[p * TOK + row], 0);
      }
      if constexpr (C8) ps.srow = max(sh.gather_rows[p * TOK + wave * 8 + (lane & 7)], 0);
    }
    return ps;
  };
  const char *gdata = (const char *)cv.data;
  auto issue_src = [&](const PageSrc &ps, int s) INL {
    LDS3 char *dst = (LDS3 char *)sh.stage[s];
#pragma unroll
    for (int m = 0; m < kInstPerWave; ++m) {
      const int gi = wave * kInstPerWave + m;
      const int row = gi * kRowsPerInst + lane / kChunks;
      const int chunk = (lane % kChunks) ^ (row & kSwz);
      const char *src;
      if constexpr (!gather)
        src = gdata + ((int64_t)ps.r[0] + row) * kRowBytes + chunk * 16;
      else
        src = gdata + (int64_t)ps.r[m] * kRowBytes + chunk * 16;
      __builtin_amdgcn_global_load_lds((const void *)src, (LDS3 void *)(dst + gi * 1024), 16, 0, 0);
    }
    if constexpr (C8) {
      // the page's 64 token scales: eight per wavefront, one dword per lane
      LDS3 float *sdst = (LDS3 float *)&sh.ssc[s][wave * 8];
      if (lane < 8) {
        const float *src;
        if constexpr (!gather)
          src = cv.scale + (int64_t)ps.r[0] + wave * 8 + lane;
        else
          src = cv.scale + ps.srow;
        __builtin_amdgcn_global_load_lds((const void *)src, (LDS3 void *)sdst, 4, 0, 0);
      }
    }
  };
  auto issue_page = [&](int p, int s) INL { issue_src(page_src(p), s); };

  int issued = 0;  // local pages whose loads are in flight
  if constexpr (!gather) {
    // Speculative plan for the common decode case, every query with
    // ceil(max_len / TOK) units and query q reading sequence q: its block ids
    // load together with the real lengths, the first unit streams one round
    // trip after entry, and the query operands load behind it.  Block ids
    // are clamped into the pool, so a wrong guess costs bandwidth only; the
    // exact plan then reissues every stage (loads of a wavefront land in
    // issue order, so the exact data overwrites the guessed data).
    //
    // The loads are unconditional (clamped indices, results dropped where
    // unused) and the guessed units are issued on one straight path: the
    // compiler then counts outstanding loads exactly, and converting the
    // operands waits for them and the first unit only.
    const int PPQ = (max_len + TOK - 1) / TOK;  // units per query
    const bool try_spec = n_q <= kWave && n_q <= cv.n_seq && PPQ > 0 && PPQ <= cv.max_blocks;
    int cnt_s = 0;
    int64_t f0s = 0;
    if (try_spec) {
      const int64_t T = (int64_t)n_q * PPQ, G = gridDim.x, g = blockIdx.x;
      f0s = g * T / G;
      cnt_s = (int)min<int64_t>((g + 1) * T / G - f0s, kMaxPagesPerWG);
      if (cnt_s > kThreads) cnt_s = 0;  // one block id per thread: no guess for longer ranges
    }
    const int ti = min(tid, max(cnt_s - 1, 0));
    const int sq = (int)((f0s + ti) / PPQ), spg = (int)((f0s + ti) % PPQ);
    const int sblk = cv.block_table[(int64_t)sq * cv.max_blocks + ((spg * TOK) >> 6)];
    const int li = min(lane, n_q - 1);
    int len0 = qlen_at(q_len, li, max_len), seq0 = q_seq[li];  // the first 64 queries' lengths and sequences
    if (lane >= n_q) len0 = seq0 = 0;
    const int slen = qlen_at(q_len, sq, max_len);
    const int q0 = cnt_s > 0 ? (int)(f0s / PPQ) : 0;
    if (tid < cnt_s) {
      sh.prow[tid] = ((sblk >= 0 && sblk < cv.n_blocks) ? sblk : 0) * kPage + ((spg * TOK) & 63);
      sh.pq[tid] = sq;
      sh.ppg[tid] = spg;
      sh.pvalid[tid] = min(TOK, slen - spg * TOK);
    }
    if (wave == 0) {
      // the guess is the exact plan iff every query has PPQ units and reads
      // its own sequence
      const bool bad = lane < n_q && (((len0 + TOK - 1) / TOK) != PPQ || seq0 != lane);
      const bool ok = try_spec && cnt_s > 0 && __ballot(bad) == 0ull;
      if (lane == 0) {
        sh.spec_ok = ok ? 1 : 0;
        if (ok) sh.np = cnt_s;
      }
      sh.qlen[lane] = len0;
      if (!ok) {
        if (n_q <= kWave) {
          // per-query unit counts -> inclusive prefix (lane = query), then
          // this workgroup's range; the unit -> (query, unit) map is built
          // by all threads below
          const int npq = lane < n_q ? (len0 + TOK - 1) / TOK : 0;
          const int incl = (int)wave_incl_scan((uint32_t)npq);
          sh.qcum[lane] = incl;
          sh.qseq[lane] = seq0;
          const int64_t T = __shfl(incl, kWave - 1, kWave);
          const int64_t G = gridDim.x, g = blockIdx.x;
          const int64_t f0 = g * T / G;
          if (lane == 0) {
            sh.np = (int)min<int64_t>((g + 1) * T / G - f0, kMaxPagesPerWG);
            sh.f0 = f0;
          }
        } else {
          plan_range<TOK>(sh, n_q, q_len, q_seq, kMaxPagesPerWG, len0, seq0, max_len);
        }
      }
    }
    lds_barrier();
    if (sh.spec_ok) {
      // unit 0, the operands, then the next units (any past the range
      // re-read the range's last unit and are never consumed)
      issue_page(0, 0);
      fetch_query(q0);
#pragma unroll
      for (int i = 1; i < NSTAGE - 1; ++i) issue_page(min(i, cnt_s - 1), i);
      issued = NSTAGE - 1;
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((NSTAGE - 2) * kVm));
      finish_query(q0);
    } else {
      const int npl = sh.np;
      if (n_q <= kWave) {
        const int64_t f0 = sh.f0;
        for (int p = tid; p < npl; p += kThreads) {
          const int f = (int)(f0 + p);
          int lo = 0, hi = n_q - 1;  // first query whose inclusive unit count exceeds f
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (sh.qcum[mid] > f) hi = mid;
            else lo = mid + 1;
          }
          const int pg = f - (lo > 0 ? sh.qcum[lo - 1] : 0);
          sh.pq[p] = lo;
          sh.ppg[p] = pg;
          sh.prow[p] = cv.block_table[(int64_t)sh.qseq[lo] * cv.max_blocks + ((pg * TOK) >> 6)] * kPage +
                       ((pg * TOK) & 63);
        }
      } else {
        for (int p = tid; p < npl; p += kThreads)
          sh.prow[p] = cv.block_table[(int64_t)sh.pseq[p] * cv.max_blocks + ((sh.ppg[p] * TOK) >> 6)] *
                           kPage + ((sh.ppg[p] * TOK) & 63);
      }
      __syncthreads();
      // valid tokens per unit (read by the stores, after the loop's barriers)
      for (int p = tid; p < npl; p += kThreads) {
        const int q = sh.pq[p];
        const int len = n_q <= kWave ? sh.qlen[q] : qlen_at(q_len, q, max_len);
        sh.pvalid[p] = min(TOK, len - sh.ppg[p] * TOK);
      }
    }
  } else {
    // Every query owns exactly ceil(B / 64) candidate slot pages: the range
    // needs no loads.  Padding slots (cand == -1) read pool row 0 and store
    // -inf.
    const int PB = (B + TOK - 1) / TOK;
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
    for (int e = tid; e < sh.np * TOK; e += kThreads) {
      const int p = e / TOK, row = e % TOK;
      const int qc = sh.pq[p] % cand_rows;  // candidate lists repeat every cand_rows queries
      const int slot = min(sh.ppg[p] * TOK + row, B - 1);
      const int t = cand[(int64_t)qc * B + slot];
      sh.gather_rows[e] =
          t >= 0 ? cv.block_table[(int64_t)q_seq[qc] * cv.max_blocks + (t >> 6)] * kPage + (t & 63)
                 : -1;
    }
    __syncthreads();
  }
  const int np = sh.np;
  if (np == 0) {
    __builtin_amdgcn_s_waitcnt(0);  // no LDS DMA may be in flight at exit
    return;
  }

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
  wait_pages_builtin<kVm, NSTAGE - 2>(min(NSTAGE - 2, np - 1));

  // Final score of token (or slot) tk of local page pp: the four head groups'
  // shares from LDS, summed in a fixed order.
  auto store_final = [&](int pp, int tk) INL {
    const int q = sh.pq[pp];
    const int t = sh.ppg[pp] * TOK + tk;
    const float *rd = &sh.red[pp & 1][0][0];
    const float v = ((rd[tk] + rd[TOK + tk]) + rd[2 * TOK + tk]) + rd[3 * TOK + tk];
    if constexpr (!gather) {
      if (tk < sh.pvalid[pp]) out[(int64_t)q * ld + t] = v;
    } else {
      if (t < B) out[(int64_t)q * ld + t] = sh.gather_rows[pp * TOK + tk] >= 0 ? v : -INFINITY;
    }
  };
  // Software pipeline over pages: iteration p issues page p's MFMAs, then
  // runs page p-1's epilogue (its results are long complete) while the matrix
  // core works, and stores page p-2's final scores; every wavefront finishes
  // eight tokens.  The epilogue uses the operands of the page's own query.
  f32x4 accO0 = {}, accO1 = {};      // page p-1 results
  float wO[4], bO[4], hO[4], s0O = 1.f, s1O = 1.f;
  auto epilogue = [&](int pp) INL {  // page pp's partial of this head group -> LDS
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x0 = accO0[i], x1 = accO1[i];  // bf16: beta is already in (the MFMAs' start value)
      if constexpr (C8) {
        x0 = (x0 * hO[i]) * s0O + bO[i];
        x1 = (x1 * hO[i]) * s1O + bO[i];
      }
      // ReLU as an integer max on the bit pattern (negative floats, -0.0
      // included, are negative integers)
      p0 = fmaf(wO[i], __int_as_float(max(__float_as_int(x0), 0)), p0);
      p1 = fmaf(wO[i], __int_as_float(max(__float_as_int(x1), 0)), p1);
    }
    // sum over the four 16-lane groups (the group's 16 heads): after the
    // 32-lane swap, lanes 0-31 hold tile 0 and lanes 32-63 tile 1, each as
    // two half sums that the 16-lane swap adds up
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false,
                                                    false);
    const float q = __uint_as_float(h[0]) + __uint_as_float(h[1]);
    const auto g = __builtin_amdgcn_permlane16_swap(__float_as_uint(q), __float_as_uint(q), false,
                                                    false);
    const float v = __uint_as_float(g[0]) + __uint_as_float(g[1]);
    // lanes 0-15: token nh*32 + lane of tile 0; lanes 32-47: of tile 1
    if ((lane & 16) == 0) sh.red[pp & 1][hg][nh * 32 + (lane & 15) + ((lane >> 5) << 4)] = v;
  };
  const int row0 = nh * 32 + (lane & 15), row1 = row0 + 16;
  for (int p = 0; p < np; ++p) {
    // bookkeeping reads ahead of the barrier (prow, pq, gather rows are
    // stable once the plan is built)
    const int nxt = p + NSTAGE - 1;
    PageSrc nsrc;
    if (nxt < np) nsrc = page_src(nxt);
    const int qp = sh.pq[p];
    wait_pages<kVm, NSTAGE - 2>(min(NSTAGE - 2, np - 1 - p));
    lds_barrier();

    if (p >= 2 && lane < 8) store_final(p - 2, wave * 8 + lane);
    if (qp != cur_q) load_query(qp, true);
    if (nxt < np) issue_src(nsrc, nxt % NSTAGE);

    const char *sp = sh.stage[p % NSTAGE];
    const char *rp0 = sp + row0 * kRowBytes, *rp1 = sp + row1 * kRowBytes;
    f32x4 acc0 = {}, acc1 = {};
    if constexpr (!C8) acc0 = acc1 = f32x4{bv[0], bv[1], bv[2], bv[3]};
    if constexpr (!C8) {
      // all of the page's B fragments first (16 LDS reads in flight), so the
      // MFMAs wait on them in order instead of once per k-step
      bf16x8 b0[KB], b1[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int chunk = kb * 4 + (lane >> 4);
        b0[kb] = *(const bf16x8 *)(rp0 + ((chunk ^ (row0 & kSwz)) * 16));
        b1[kb] = *(const bf16x8 *)(rp1 + ((chunk ^ (row1 & kSwz)) * 16));
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abf[t][kb].v, b0[kb], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abf[t][kb].v, b1[kb], acc1, 0, 0, 0);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int cc = kb * 8 + (lane >> 4) * 2;
        // Read through the same 16-byte vector type as the bf16 path: with
        // it the compiler adds no wait for the in-flight LDS DMA before these
        // reads (their stage completed at the explicit vmcnt wait and barrier).
        Frag x0, y0, x1, y1;
        x0.v = *(const bf16x8 *)(rp0 + ((cc ^ (row0 & kSwz)) * 16));
        y0.v = *(const bf16x8 *)(rp0 + (((cc + 1) ^ (row0 & kSwz)) * 16));
        x1.v = *(const bf16x8 *)(rp1 + ((cc ^ (row1 & kSwz)) * 16));
        y1.v = *(const bf16x8 *)(rp1 + (((cc + 1) ^ (row1 & kSwz)) * 16));
        const i32x8 b0 = {(int)x0.u[0], (int)x0.u[1], (int)x0.u[2], (int)x0.u[3],
                          (int)y0.u[0], (int)y0.u[1], (int)y0.u[2], (int)y0.u[3]};
        const i32x8 b1 = {(int)x1.u[0], (int)x1.u[1], (int)x1.u[2], (int)x1.u[3],
                          (int)y1.u[0], (int)y1.u[1], (int)y1.u[2], (int)y1.u[3]};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8[t][kb], b0, acc0, 0, 0, 0, 0,
                                                                  0, 0);
          acc1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8[t][kb], b1, acc1, 0, 0, 0, 0,
                                                                  0, 0);
        }
      }
    }
    if (p >= 1) epilogue(p - 1);
    accO0 = acc0;
    accO1 = acc1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wO[i] = wv[i];
      bO[i] = bv[i];
      hO[i] = C8 ? hs[i] : 1.f;
    }
    if constexpr (C8) {
      s0O = sh.ssc[p % NSTAGE][row0];
      s1O = sh.ssc[p % NSTAGE][row1];
    }
  }
  epilogue(np - 1);
  lds_barrier();
  if (lane < 8) {
    if (np >= 2) store_final(np - 2, wave * 8 + lane);
    store_final(np - 1, wave * 8 + lane);
  }
}

template <int R, int NSTAGE, bool C8, bool QF32, bool GATHER, int TOK>
hipError_t launch_t(const void *q_tilde, const float *w, const float *beta, int n_q,
                      const int32_t *q_seq, const int32_t *q_len, int max_len, const CacheView &cv,
                      const int32_t *cand, int B, int cand_rows, float *out, int64_t ld,
                      hipStream_t st) {
  const int64_t per_q = GATHER ? (B + TOK - 1) / TOK : (max_len + TOK - 1) / TOK;
  const int64_t T_ub = (int64_t)n_q * per_q;
  const int cap = GATHER ? kMaxPagesGather : kMaxPagesPerWG;
  int64_t G = std::min<int64_t>(T_ub, (int64_t)device_cu_count() * (64 / TOK));
  G = std::max<int64_t>(G, (T_ub + cap - 1) / cap);
  if (G <= 0) return hipSuccess;
  score_mfma_kernel<R, NSTAGE, C8, QF32, GATHER, TOK><<<(unsigned)G, TOK * 8, 0, st>>>(
      q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, cand, B, std::max(cand_rows, 1), out, ld);
  return hipGetLastError();
}

template <bool C8, bool QF32>
hipError_t launch_mode(const void *q_tilde, const float *w, const float *beta, int n_q,
                       const int32_t *q_seq, const int32_t *q_len, int max_len,
                       const CacheView &cv, const int32_t *cand, int B, int cand_rows, float *out,
                       int64_t ld, hipStream_t st) {
  // Workgroups of four wavefronts over 32-token units, two per CU: one can
  // compute while the other waits at its barrier.  fp8 units are half as
  // large: more of them in flight.
  constexpr int kTok = 32;
  constexpr int kStages = C8 ? 6 : 4;
  if (cand)
    return launch_t<256, kStages, C8, QF32, true, kTok>(q_tilde, w, beta, n_q, q_seq, q_len,
                                                        max_len, cv, cand, B, cand_rows, out, ld,
                                                        st);
  return launch_t<256, kStages, C8, QF32, false, kTok>(q_tilde, w, beta, n_q, q_seq, q_len, max_len,
                                                       cv, cand, B, cand_rows, out, ld, st);
}

}  // namespace

bool score_mfma_supported(int qt_dt, int H, const CacheView &cv) {
  return H == 64 && cv.r == 256 && (cv.dtype == LI_BF16 || cv.dtype == LI_FP8_E4M3) &&
         cv.scale_block == 0 && (qt_dt == LI_FP32 || qt_dt == LI_BF16);
}

hipError_t launch_score_mfma(const void *q_tilde, int qt_dt, const float *w, const float *beta,
                             int n_q, int H, const int32_t *q_seq, const int32_t *q_len,
                             int max_len, const CacheView &cv, const int32_t *cand, int B,
                             int cand_rows, float *out, int64_t ld, hipStream_t st) {
  (void)H;
  const bool f32 = qt_dt == LI_FP32;
  if (cv.dtype == LI_FP8_E4M3)
    return f32 ? launch_mode<true, true>(q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, cand,
                                         B, cand_rows, out, ld, st)
               : launch_mode<true, false>(q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, cand,
                                          B, cand_rows, out, ld, st);
  return f32 ? launch_mode<false, true>(q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, cand, B,
                                        cand_rows, out, ld, st)
             : launch_mode<false, false>(q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, cand,
                                         B, cand_rows, out, ld, st);
}

}  // namespace li
