// Matrix-core scorer for many queries over one shared cache (prefill chunk):
// eq. (8) of the LatentIndex summary ("Methodology"),
// u_{s,t} = sum_h w_{s,h} ReLU(q~_{s,h} . c_t + beta_{s,h}) for t < q_len[s],
// with bf16 absorbed queries, H = 64, r = 256 and a bf16 cache.
//
// This is a dense contraction ([queries x 64 heads] x [256] x [tokens]) with a
// ReLU and a head reduction in the epilogue, bound by the matrix cores
// (2 * 64 * 256 flop per (query, token) pair against 512 B per token shared
// by every query), so the design maximises reuse of each staged latent page:
//  * A workgroup holds 8 queries (one per wavefront, all 64 heads of its
//    query's q~ in registers: 4 head tiles x 8 k-steps of
//    v_mfma_f32_16x16x32_bf16 operands) and one token range.
//  * Pages (64 tokens, 32 KB) stream HBM/L2 -> LDS with direct-to-LDS buffer
//    loads (NSTAGE stages), stored k-block-major: [8 k-blocks of 32 latent
//    dims][64 tokens][64 B], the four 16-byte chunks of token n XOR-swizzled
//    by f(n) = (n1 ^ n3) | n2 << 1 (n_i: bit i of n), so that the 8 lanes of
//    any aligned group reading one chunk of 8 tokens cover 128 distinct bytes
//    modulo 128, and the 16 lanes of a quarter-wave 256 distinct bytes modulo
//    256.  Every operand address is then one register plus an immediate.  Each wavefront reads every page once from LDS and
//    computes 64 heads x 64 tokens (128 MFMAs).
//  * beta enters as the accumulator's initial value; the epilogue (ReLU, x w,
//    the 64-head sum: 16 heads per lane, then two cross-lane adds) stays in
//    registers and each wavefront writes one 64-token row segment per page.
//  * Token ranges are XCD-aware: workgroups are dealt round-robin over the 8
//    XCDs, so workgroup g runs on XCD g % 8; range (g % 8) + 8 j is served by
//    XCD g % 8 only, all of its query groups before range j + 1 starts, which
//    keeps the pages a range streams in that XCD's own L2.
//  * Queries of a workgroup that read different sequences are served in
//    separate rounds (one per distinct sequence); a prefill chunk has one.
#include <algorithm>

#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

#define LDS3 __attribute__((address_space(3)))
#define INL __attribute__((always_inline))

constexpr int kQ = 8;             // queries (wavefronts) per workgroup
constexpr int kThr = kQ * kWave;  // 512
constexpr int kRowB = 512;        // bf16 latent row bytes (r = 256)
constexpr int kKb = 8;             // k-blocks of 32 dims (64 B) per token
constexpr int kMaxRangePages = 256;  // pages per token range

static_assert(kKb == kQ, "wavefront w stages k-block w of every page");

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// chunk swizzle of token n (only bits 1-3 of n matter)
__device__ __forceinline__ int swz(int n) { return (((n >> 1) ^ (n >> 3)) & 1) | (n & 4) >> 1; }
__device__ __forceinline__ void bar() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int NSTAGE>
struct PrefillShared {
  __align__(16) char stage[NSTAGE][kPage * kRowB];
  int32_t blk[kMaxRangePages];
  int32_t qseq[kQ], qlen[kQ];
  int32_t round_seq, round_len;
};

union Frag {
  bf16x8 v;
  uint32_t u[4];
};

template <int NSTAGE>
__global__ void __launch_bounds__(kThr, 1)
score_prefill_kernel(const uint16_t *__restrict__ q_tilde, const float *__restrict__ w,
                     const float *__restrict__ beta, int n_q, const int32_t *__restrict__ q_seq,
                     const int32_t *__restrict__ q_len, int max_len, CacheView cv, float *__restrict__ out,
                     int64_t ld, int n_groups, int range_pages) {
  constexpr int kInstPerWave = (kPage * kRowB / 1024) / kQ;  // 1 KB per wave-instruction: 4
  __shared__ PrefillShared<NSTAGE> sh;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave, g4 = lane >> 4;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int rng = xcd + 8 * (slot / n_groups), qg = slot % n_groups;
  const int q = qg * kQ + wave;  // this wavefront's query
  const bool has_q = q < n_q;

  // operands of the wavefront's query: A[rt][kb] = q~[q][16 rt + lane%16][kb*32 + g4*8 .. +8]
  Frag A[4][8];
  float wv[4][4], bv[4][4];
  {
    const int qq = has_q ? q : 0;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const uint16_t *src = q_tilde + ((int64_t)qq * 64 + 16 * rt + (lane & 15)) * 256 + g4 * 8;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const uint4 x = *(const uint4 *)(src + kb * 32);
        A[rt][kb].u[0] = x.x;
        A[rt][kb].u[1] = x.y;
        A[rt][kb].u[2] = x.z;
        A[rt][kb].u[3] = x.w;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 16 * rt + 4 * g4 + i;
        wv[rt][i] = w[(int64_t)qq * 64 + h];
        bv[rt][i] = beta ? beta[(int64_t)qq * 64 + h] : 0.f;
      }
    }
  }
  if (tid < kQ) {
    const int qi = qg * kQ + tid;
    const int sq = qi < n_q ? q_seq[qi] : -1;
    const bool ok = sq >= 0 && sq < cv.n_seq;  // others are skipped
    sh.qseq[tid] = ok ? sq : -1;
    sh.qlen[tid] = ok ? min(max(q_len[qi], 0), max_len) : 0;
  }
  bar();
  const int myseq = sh.qseq[wave];
  const int mylen = has_q ? sh.qlen[wave] : 0;
  float *orow = out + (int64_t)(has_q ? q : 0) * ld;
  uint32_t done = 0;  // bit w: query of wavefront w served
  for (int w2 = 0; w2 < kQ; ++w2)
    if (sh.qseq[w2] < 0) done |= 1u << w2;

  const char *gdata = (const char *)cv.data;
  while (true) {
    // next round: the first unserved query's sequence, and the longest
    // length among the queries on it
    if (tid == 0) {
      int s = -1, L = 0;
      for (int w2 = 0; w2 < kQ; ++w2)
        if (!((done >> w2) & 1u) && s < 0) s = sh.qseq[w2];
      for (int w2 = 0; w2 < kQ; ++w2)
        if (!((done >> w2) & 1u) && sh.qseq[w2] == s) L = max(L, sh.qlen[w2]);
      sh.round_seq = s;
      sh.round_len = L;
    }
    bar();
    const int s = sh.round_seq, L = sh.round_len;
    if (s < 0) break;
    const bool active = has_q && myseq == s;
    for (int w2 = 0; w2 < kQ; ++w2)
      if (sh.qseq[w2] == s) done |= 1u << w2;
    // this range's pages of sequence s that some query of the round needs
    const int pg0 = rng * range_pages;
    const int npg =
        max(0, min(min(range_pages, cv.max_blocks - pg0), (L + kPage - 1) / kPage - pg0));
    for (int p = tid; p < npg; p += kThr) {
      const int b = cv.block_table[(int64_t)s * cv.max_blocks + pg0 + p];
      sh.blk[p] = (b >= 0 && b < cv.n_blocks) ? b : 0;
    }
    bar();
    // wavefront w stages k-block w of a page: 4 loads of 16 tokens x 64 B;
    // lane -> token m*16 + lane/4, LDS slot lane%4 holding chunk
    // (lane%4) ^ f(lane/4)
    const int voff = (lane >> 2) * kRowB + wave * 64 + (((lane & 3) ^ swz(lane >> 2)) << 4);
    auto issue = [&](int p, int st) INL {
      LDS3 char *dst = (LDS3 char *)sh.stage[st] + wave * (kPage * 64);
      const int blk = __builtin_amdgcn_readfirstlane(sh.blk[p]);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(gdata + (int64_t)blk * kPage * kRowB), 0, kPage * kRowB, 0x00020000);
#pragma unroll
      for (int m = 0; m < kInstPerWave; ++m)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS3 void *)(dst + m * 1024), 16, voff,
                                                 m * 16 * kRowB, 0, 0);
    };
    // operand read of lane (g4, n): token tt*16 + n, k-block kb, chunk g4
    const int roff = (lane & 15) * 64 + ((g4 ^ swz(lane & 15)) << 4);
    // Software pipeline: the epilogue of tile tt runs between the MFMAs of
    // tile tt+1, whose operands are read one k-block behind the MFMAs of tile
    // tt; a page's last tile is finished after the next page's barrier,
    // while that page's first operands are in flight.
    f32x4 accP[4];   // pending tile (epilogue not yet applied)
    float part[4];   // this lane's 16-head partial sum for each 16-token tile
    int pend_t = -1; // first token of the page whose last tile is pending
    auto relu_w = [&](const f32x4 (&acc)[4], int e, float v) INL {
      // ReLU as an integer max on the bit pattern (negative floats, -0.0
      // included, are negative integers), weighted by the head's w
      const float r = __int_as_float(max(__float_as_int(acc[e >> 2][e & 3]), 0));
      return fmaf(wv[e >> 2][e & 3], r, v);
    };
    auto flush = [&]() INL {
      float v = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) v = relu_w(accP, e, v);
      part[3] = v;
      // reduce-scatter over the four 16-lane groups: tile j's head sum lands
      // in lane group j (token pend_t + lane)
      const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]),
                                                        __float_as_uint(part[2]), false, false);
      const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]),
                                                        __float_as_uint(part[3]), false, false);
      const float q02 = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);
      const float q13 = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);
      const auto s4 = __builtin_amdgcn_permlane16_swap(__float_as_uint(q02), __float_as_uint(q13),
                                                       false, false);
      const float outv = __uint_as_float(s4[0]) + __uint_as_float(s4[1]);
      const int t = pend_t + lane;
      if (t < mylen) orow[t] = outv;
    };
    for (int p = 0; p < NSTAGE - 1; ++p)
      if (p < npg) issue(p, p);
    for (int p = 0; p < npg; ++p) {
      const int after = min(NSTAGE - 2, npg - 1 - p);
      if (after >= 2) wait_vm<2 * kInstPerWave>();
      else if (after == 1) wait_vm<kInstPerWave>();
      else wait_vm<0>();
      bar();
      if (p + NSTAGE - 1 < npg) issue(p + NSTAGE - 1, (p + NSTAGE - 1) % NSTAGE);
      const int t_page = (pg0 + p) * kPage;
      const bool act = active && t_page < mylen;
      const char *sp = sh.stage[p % NSTAGE] + roff;
      bf16x8 b[kKb];
      if (act) {
#pragma unroll
        for (int kb = 0; kb < kKb; ++kb) b[kb] = *(const bf16x8 *)(sp + kb * (kPage * 64));
      }
      if (pend_t >= 0) {
        flush();
        pend_t = -1;
      }
      if (act) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          f32x4 acc[4];
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x4{bv[rt][0], bv[rt][1], bv[rt][2], bv[rt][3]};
          float v = 0.f;
#pragma unroll
          for (int kb = 0; kb < kKb; ++kb) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
              acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[rt][kb].v, b[kb], acc[rt], 0, 0, 0);
            if (tt < 3)
              b[kb] = *(const bf16x8 *)(sp + kb * (kPage * 64) + (tt + 1) * 16 * 64);
            if (tt > 0) {
              v = relu_w(accP, 2 * kb, v);
              v = relu_w(accP, 2 * kb + 1, v);
            }
          }
          if (tt > 0) part[tt - 1] = v;
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) accP[rt] = acc[rt];
        }
        pend_t = t_page;
      }
    }
    if (pend_t >= 0) flush();
    bar();  // all reads of the stages done before the next round reuses them
  }
}

}  // namespace

bool score_prefill_supported(int qt_dt, int H, int n_q, const CacheView &cv) {
  // worth it when queries share sequences: at least kQ per sequence on average
  return qt_dt == LI_BF16 && H == 64 && cv.r == 256 && cv.dtype == LI_BF16 && n_q >= 64 &&
         n_q >= kQ * cv.n_seq;
}

hipError_t launch_score_prefill(const void *q_tilde, const float *w, const float *beta, int n_q,
                                const int32_t *q_seq, const int32_t *q_len, int max_len,
                                const CacheView &cv, float *out, int64_t ld, hipStream_t st) {
  // token ranges in multiples of 8 (one per XCD), at most kMaxRangePages
  // pages each (the page table a workgroup keeps in LDS)
  const int pages = (max_len + kPage - 1) / kPage;
  int n_ranges = 8;
  while ((pages + n_ranges - 1) / n_ranges > kMaxRangePages) n_ranges += 8;
  const int range_pages = (pages + n_ranges - 1) / n_ranges;
  const int n_groups = (n_q + kQ - 1) / kQ;
  const int64_t grid = (int64_t)n_groups * n_ranges;
  if (pages <= 0 || n_groups <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  score_prefill_kernel<4><<<(unsigned)grid, kThr, 0, st>>>(
      (const uint16_t *)q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, out, ld, n_groups,
      range_pages);
  return hipGetLastError();
}

}  // namespace li
