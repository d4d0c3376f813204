// Full-scan decode scorer: eq. (8) of the LatentIndex summary
// ("Methodology"), u_t = sum_h w_h ReLU(q~_h . c_t + beta_h) for every valid
// token t, H = 64 heads, r = 256, a bf16 cache, at most 64 queries.
//
// The scan streams the whole latent cache once per call, so it is bound by
// HBM.  Two properties of the hardware shape it:
//  * a CU holds only a few tens of KB of direct-to-LDS loads in flight, so
//    HBM stays busy only if some wavefront is always ready to issue the next
//    load; a wavefront that also computes leaves the CU's share of HBM idle
//    meanwhile.  Four issuer wavefronts therefore do nothing but stream
//    pages into LDS, and eight compute wavefronts only score them;
//  * two workgroups on one CU finish several microseconds apart (the older
//    one's wavefronts win the arbitration), so there is one workgroup per CU
//    (its LDS use rules out a second) and a static, even split of the pages.
//
// A unit is one cache page of 64 tokens (32 KB, contiguous in HBM), staged in
// one of four LDS buffers: 16-byte chunks of a token row XOR-swizzled by
// (row & 15), each issuer loading 8 of the 32 1-KB pieces.  Compute
// wavefront w scores heads 16 (w & 3) .. +15 against tokens 32 (w >> 2) ..
// +31 of the unit as two 16x16 tiles with v_mfma_f32_16x16x32_bf16 (bf16 hi
// and lo terms of an fp32 q~, or the bf16 q~); the epilogue (+beta as the
// MFMAs' start value, ReLU, x w, sum over the 16 heads) reduces across lanes
// and the four head groups are summed through LDS.  q~ of the query comes
// once per workgroup into LDS in the same round trip as the lengths, the page
// table, w and beta.  Queries get workgroups in proportion to their pages
// (at least one each); a query's pages are split evenly over its workgroups.
#include <algorithm>

#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

#define LDS3 __attribute__((address_space(3)))
#define INL __attribute__((always_inline))

constexpr int kTok = kPage;           // tokens per unit: one cache page
constexpr int kR = 256;
constexpr int kRowB = 2 * kR;         // bf16 token row
constexpr int kUnitB = kTok * kRowB;  // 32 KB
constexpr int kNst = 4;               // LDS stages
constexpr int kAhead = kNst - 1;      // units in flight
constexpr int kQst = 2;               // q~ is staged in stages kQst, kQst+1 (64 KB)
constexpr int kCW = 8;                // compute wavefronts
constexpr int kIW = 4;                // issuer wavefronts
constexpr int kThr = (kCW + kIW) * kWave;
constexpr int kPieces = kUnitB / 1024;  // 1 KB loads per unit
constexpr int kPerIssuer = kPieces / kIW;
constexpr int kMaxPages = 1024;       // page table of one workgroup's range
constexpr int kMaxCandUnits = 64;     // candidate mode: units of one workgroup's range
constexpr int kTab = kMaxCandUnits * kTok;  // table entries (pages, or candidate rows)
constexpr int kTabPer = (kTab + kThr - 1) / kThr;
static_assert(kTab >= kMaxPages, "the table holds a page range");
constexpr int kSwz = 15;
static_assert(kQst + 2 <= kNst, "q~ staging fits in the stages");
static_assert(kPerIssuer * kAhead <= 24, "issuer wait counts stay in range");

constexpr int kHistBins = 4096;  // row histogram of score keys, bits 31..20

struct ScanShared {
  __align__(16) char stage[kNst][kUnitB];
  int32_t page[kTab];  // block id of page u0 + i; candidate mode: cache row of slot 64 u0 + i (-1: none)
  // A page scan uses at most kMaxPages table entries; the rest of the table
  // and hext hold its histogram of score keys when one is asked for.
  uint32_t hext[kHistBins - (kTab - kMaxPages)];
  float red[2][4][kTok];    // per head group partial scores, two units
  int32_t ok, myq, mylen, myseq, u0, nu;
};

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// s_waitcnt vmcnt(n) for a runtime n in [0, 24]
__device__ __forceinline__ void wait_vm_rt(int n) {
  switch (n) {
#define LI_W(k) case k: wait_vm<k>(); break;
    LI_W(0) LI_W(1) LI_W(2) LI_W(3) LI_W(4) LI_W(5) LI_W(6) LI_W(7) LI_W(8) LI_W(9) LI_W(10)
    LI_W(11) LI_W(12) LI_W(13) LI_W(14) LI_W(15) LI_W(16) LI_W(17) LI_W(18) LI_W(19) LI_W(20)
    LI_W(21) LI_W(22) LI_W(23)
#undef LI_W
    default: wait_vm<24>(); break;
  }
}
// s_waitcnt immediate for vmcnt <= n only (gfx9 encoding)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

union Frag {
  bf16x8 v;
  uint32_t u[4];
};

// Workgroups of query q: [start(q), start(q+1)), start(q) = q + floor((G - n) *
// cum(q) / T) with cum(q) the pages of the queries before q and T all pages:
// every query gets at least one, the rest in proportion to its pages.
__device__ __forceinline__ int64_t wg_start(int q, int64_t cum, int64_t T, int G, int n) {
  return q + ((int64_t)(G - n) * cum) / T;
}

// CAND: candidate mode (HS followers).  Query i scores the B slots of
// candidate list c = i % cand_rows (token ids of sequence q_seq[c], -1 for
// padding) into out[i*ld + j]; units are 64 consecutive slots; q_len and
// max_len are unused.
// hist (page scan only, may be null): [n_q][kHistBins] histograms of the
// order-preserving keys of the scores written (bin = key >> 20), added to
// what the array holds; zbuf[0 .. zwords) is zeroed on the way (the
// workgroups share it out), for a consumer that accumulates there next.
template <bool QF32, bool CAND>
__global__ void __launch_bounds__(kThr, 1)
score_scan_kernel(const void *__restrict__ q_tilde, const float *__restrict__ w,
                  const float *__restrict__ beta, int n_q, const int32_t *__restrict__ q_seq,
                  const int32_t *__restrict__ q_len, int max_len, CacheView cv,
                  const int32_t *__restrict__ cand, int B, int cand_rows, int xw,
                  float *__restrict__ out, int64_t ld, uint32_t *__restrict__ hist,
                  uint32_t *__restrict__ zbuf, int zwords) {
  static_assert(kTab - kMaxPages + (kHistBins - (kTab - kMaxPages)) == kHistBins, "histogram span");
  constexpr int NT = QF32 ? 2 : 1;               // A operand terms (bf16 hi + lo, or the bf16 q~)
  constexpr int KB = kR / 32;                    // MFMA k-steps
  constexpr int QROWB = QF32 ? 4 * kR : 2 * kR;  // bytes of one head's q~ row
  __shared__ ScanShared sh;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const bool issuer = wave >= kCW;
  const int hg = wave & 3, th = (wave >> 2) & 1;  // compute: head group, token half
  const int G = gridDim.x, g = blockIdx.x;
  char *const qst = sh.stage[kQst];  // LDS copy of q~
  uint32_t *const hl = reinterpret_cast<uint32_t *>(&sh.page[kMaxPages]);  // page scan histogram

  // q~ of query q -> LDS (64 x QROWB bytes), 16-byte chunk c of head row h
  // at chunk c ^ (h & 15): 1 KB per load, each compute wavefront an eighth.
  auto fetch_q = [&](int q) INL {
    constexpr int NL = 64 * QROWB / 1024 / kCW;  // loads per compute wavefront
    constexpr int CPR = QROWB / 16;              // chunks per head row
    if (!issuer) {
#pragma unroll
      for (int m = 0; m < NL; ++m) {
        const int gi = wave * NL + m;
        const int e = gi * 64 + lane;  // chunk index over the 64 heads
        const int h = e / CPR, c = e % CPR;
        dma16_to_lds((const char *)q_tilde + ((int64_t)q * 64 + h) * QROWB + ((c ^ (h & kSwz)) * 16),
                     (LDS3 void *)((LDS3 char *)qst + gi * 1024));
      }
    }
  };
  // w and beta of heads 16 hg + 4 (lane/16) .. +3 of query q (beta 0 if absent)
  float wv[4], bv[4];
  auto load_wb = [&](int q) INL {
    const int64_t hb = (int64_t)q * 64 + 16 * hg + 4 * (lane >> 4);
    const float4 w4 = *(const float4 *)(w + hb);
    const float4 b4 = *(const float4 *)((beta ? beta : w) + hb);  // dropped when beta is absent
    const bool has_beta = beta != nullptr;
    wv[0] = w4.x; wv[1] = w4.y; wv[2] = w4.z; wv[3] = w4.w;
    bv[0] = has_beta ? b4.x : 0.f; bv[1] = has_beta ? b4.y : 0.f;
    bv[2] = has_beta ? b4.z : 0.f; bv[3] = has_beta ? b4.w : 0.f;
  };

  // issuers: page b (64 token rows) into stage u % kNst, 32 loads of 1 KB
  // (two token rows each), issuer i loading pieces 8i .. 8i+7
  const char *gdata = (const char *)cv.data;
  const int gi0 = (wave - kCW) * kPerIssuer;
  auto issue_page = [&](int u, int b) INL {
    LDS3 char *st = (LDS3 char *)sh.stage[u % kNst];
    const char *src = gdata + (int64_t)((b >= 0 && b < cv.n_blocks) ? b : 0) * kUnitB;
#pragma unroll
    for (int m = 0; m < kPerIssuer; ++m) {
      const int gi = gi0 + m;
      const int r = gi * 2 + lane / 32;
      const int chunk = (lane % 32) ^ (r & kSwz);
      dma16_to_lds(src + r * kRowB + chunk * 16, (LDS3 void *)(st + gi * 1024));
    }
  };

  // ---- plan: guess (every query max_len long, query q on sequence q) ------
  // (exact in candidate mode: every query has B slots)
  const int PPQ = ((CAND ? B : max_len) + kTok - 1) / kTok;
  const int64_t T0 = (int64_t)n_q * PPQ;
  int gq = 0;  // guessed query: the last q with start(q) <= g
  int gu0, gnu;
  if (CAND && xw > 0) {
    // Candidate lists shared by NL layers' queries (i = l * cand_rows + c),
    // xw ranges per query: the NL workgroups of one (list, range) pair sit
    // 8 apart in g, i.e. on one XCD (g mod 8) side by side, so the rows they
    // all read come from that XCD's L2 after the first.
    const int NL = n_q / cand_rows, NP = cand_rows * xw, full = NP - NP % 8;
    int j, l;
    if (g < NL * full) {
      const int within = g % (8 * NL);
      l = within / 8;
      j = (g / (8 * NL)) * 8 + within % 8;
    } else {
      const int g2 = g - NL * full, m = NP - full;
      l = g2 / m;
      j = full + g2 % m;
    }
    const int r = j % xw;
    gq = l * cand_rows + j / xw;
    gu0 = (int)((int64_t)r * PPQ / xw);
    gnu = (int)((int64_t)(r + 1) * PPQ / xw) - gu0;
  } else {
    for (int q = 1; q < n_q; ++q)
      if (wg_start(q, (int64_t)q * PPQ, T0, G, n_q) <= g) gq = q;
    const int s = (int)wg_start(gq, (int64_t)gq * PPQ, T0, G, n_q);
    const int W = (int)wg_start(gq + 1, (int64_t)(gq + 1) * PPQ, T0, G, n_q) - s;
    const int j = g - s;
    gu0 = (int)((int64_t)j * PPQ / W);
    gnu = (int)((int64_t)(j + 1) * PPQ / W) - gu0;
  }
  // One round trip: q~ of the guessed query (direct to LDS, not tracked by
  // the compiler), then the lengths and sequences of all queries (wavefront
  // 0), the guessed range's page table, w and beta; one wait covers
  // them all, the q~ loads included, before the barrier that ends the plan.
  fetch_q(gq);
  if constexpr (CAND) {
    // the range's candidate token ids, then their cache rows (a second,
    // dependent load through the block table)
    const int c = gq % cand_rows;
    const int seq = q_seq[c];
    const int s0 = gu0 * kTok, ns = min(gnu * kTok, B - s0);  // slots of the range
    int tk[kTabPer], bk[kTabPer];
#pragma unroll
    for (int k = 0; k < kTabPer; ++k) {
      const int i = tid + k * kThr;
      tk[k] = cand[(int64_t)c * B + min(s0 + min(i, max(ns - 1, 0)), B - 1)];
      if (i >= ns) tk[k] = -1;
    }
#pragma unroll
    for (int k = 0; k < kTabPer; ++k)
      bk[k] = cv.block_table[(int64_t)seq * cv.max_blocks + min(max(tk[k], 0) >> 6, cv.max_blocks - 1)];
    load_wb(gq);
#pragma unroll
    for (int k = 0; k < kTabPer; ++k) {
      const int i = tid + k * kThr;
      const int b = (bk[k] >= 0 && bk[k] < cv.n_blocks) ? bk[k] : 0;
      if (i < gnu * kTok) sh.page[i] = tk[k] < 0 ? -1 : b * kPage + (tk[k] & 63);
    }
    if (tid == 0) {
      sh.ok = 1;
      sh.myq = gq;
      sh.mylen = B;
      sh.myseq = seq;
      sh.u0 = gu0;
      sh.nu = gnu;
    }
  } else if (issuer) {
    // The guessed range's first pages stream while the plan is checked (a
    // wrong guess waits for them and loads those stages again).  The issuers
    // make no other loads here, so no wait for the plan's loads holds these.
    // All block ids first (a wait for one must not wait for pages), and all
    // kQst pages unconditionally so the loads issue together: past a short
    // range they fetch a clamped page into a stage nothing reads, and the
    // waits below, which count only the range's pages, stay conservative.
    int bid[kQst];
#pragma unroll
    for (int u = 0; u < kQst; ++u)
      bid[u] = cv.block_table[(int64_t)gq * cv.max_blocks + min(gu0 + min(u, max(gnu - 1, 0)), cv.max_blocks - 1)];
#pragma unroll
    for (int u = 0; u < kQst; ++u) asm volatile("" : "+v"(bid[u]));  // both loads land here
#pragma unroll
    for (int u = 0; u < kQst; ++u) issue_page(u, bid[u]);
  } else {
    constexpr int kCT = kCW * kWave;  // compute threads
    static_assert(2 * kCT >= kMaxPages, "two page-table entries per compute thread");
    const int li = min(lane, n_q - 1);
    int len0 = q_len[li], seq0 = q_seq[li];
    if (lane >= n_q) len0 = seq0 = 0;
    int pg[2];
  #pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = min(tid + k * kCT, max(gnu - 1, 0));
      pg[k] = cv.block_table[(int64_t)gq * cv.max_blocks + min(gu0 + i, cv.max_blocks - 1)];
    }
    load_wb(gq);
    if (hist) {
      const uint4 z = make_uint4(0u, 0u, 0u, 0u);
      for (int i = tid; i < kHistBins / 4; i += kCT) reinterpret_cast<uint4 *>(hl)[i] = z;
      const int per = (zwords + G - 1) / G, e = min(zwords, (g + 1) * per);
      for (int i = g * per + tid; i < e; i += kCT) zbuf[i] = 0u;
    }
  #pragma unroll
    for (int k = 0; k < 2; ++k)
      if (tid + k * kCT < gnu) sh.page[tid + k * kCT] = pg[k];
    if (wave == 0) {
      const bool bad = lane < n_q && (((len0 + kTok - 1) / kTok) != PPQ || seq0 != lane);
      const bool ok = __ballot(bad) == 0ull;
      const int glen = min(__shfl(len0, gq, kWave), max_len);
      if (lane == 0) {
        sh.ok = ok ? 1 : 0;
        sh.myq = gq;
        sh.mylen = glen;
        sh.myseq = gq;
        sh.u0 = gu0;
        sh.nu = gnu;
      }
      if (!ok) {
        // exact partition from the real lengths
        const int len = min(len0, max_len);
        const int units = lane < n_q ? (len + kTok - 1) / kTok : 0;
        const int incl = (int)wave_incl_scan((uint32_t)units);
        const int64_t T = max(__shfl(incl, kWave - 1, kWave), 1);
        const int64_t st = lane < n_q ? wg_start(lane, incl - units, T, G, n_q) : (int64_t)G;
        const int q = __popcll(__ballot(lane < n_q && st <= g)) - 1;
        const int s = __shfl((int)st, q, kWave);
        const int W = (q + 1 < n_q ? __shfl((int)st, q + 1, kWave) : G) - s;
        const int uq = __shfl(units, q, kWave);
        const int j = g - s;
        const int qlen = __shfl(len, q, kWave), qseq = __shfl(seq0, q, kWave);  // all lanes active
        if (lane == 0) {
          const int a = (int)((int64_t)j * uq / W), b = (int)((int64_t)(j + 1) * uq / W);
          sh.myq = q;
          sh.mylen = qlen;
          sh.myseq = qseq;
          sh.u0 = a;
          sh.nu = b - a;
        }
      }
    }
  }
  // Every loading wavefront's loads are in, the q~ copy included: the
  // compiler may sink its own waits for w and beta past the first reads of
  // that copy.  (Issuers of a page scan have only their early pages in
  // flight and go on.)
  if (CAND || !issuer) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();
  if (!sh.ok) {
    // second round trip: this range's page table and, if the query changed,
    // its q~, w and beta (the copy of the guessed q~ is not read yet)
    const int u0 = sh.u0, nu = sh.nu, sq = sh.myseq, q = sh.myq;
    if (q != gq) {
      fetch_q(q);
      load_wb(q);
    }
    for (int i = tid; i < nu; i += kThr)
      sh.page[i] = cv.block_table[(int64_t)sq * cv.max_blocks + min(u0 + i, cv.max_blocks - 1)];
    // a wait the compiler sees, so that it knows w and beta have landed too
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
  }
  const int myq = sh.myq, mylen = sh.mylen, u0 = sh.u0, nu = sh.nu;

  // ---- issuers: unit u of the range (page u0 + u, or 64 candidate rows) ----
  auto issue_unit = [&](int u) INL {
    if constexpr (CAND) {
      LDS3 char *st = (LDS3 char *)sh.stage[u % kNst];
      // every half-wavefront gathers one candidate row (a padding slot reads row 0)
#pragma unroll
      for (int m = 0; m < kPerIssuer; ++m) {
        const int gi = gi0 + m;
        const int r = gi * 2 + lane / 32;
        const int chunk = (lane % 32) ^ (r & kSwz);
        const int64_t row = max(sh.page[u * kTok + r], 0);
        dma16_to_lds(gdata + row * kRowB + chunk * 16, (LDS3 void *)(st + gi * 1024));
      }
    } else {
      issue_page(u, sh.page[u]);
    }
  };
  // prologue: units clear of the q~ copy (a page scan whose guess held has
  // issued them already; after the slow path every load has landed)
  int issued = (!CAND && sh.ok) ? min(nu, kQst) : 0;
  if (issuer)
    for (int u = issued; u < min(nu, kQst); ++u) issue_unit(u);
  issued = min(nu, kQst);

  // ---- compute: A fragments of heads 16 hg .. +15 from the q~ copy ---------
  Frag abf[NT][KB];
  if (!issuer) {
    const int h = 16 * hg + (lane & 15);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if constexpr (QF32) {
        // floats kb*32 + (lane/16)*8 .. +7: chunks c0 and c0 + 1
        const int c0 = 2 * (kb * 4 + (lane >> 4));
        const uint4 x0 = *(const uint4 *)(qst + h * QROWB + ((c0 ^ (h & kSwz)) * 16));
        const uint4 x1 = *(const uint4 *)(qst + h * QROWB + (((c0 + 1) ^ (h & kSwz)) * 16));
        const float xs[8] = {__uint_as_float(x0.x), __uint_as_float(x0.y), __uint_as_float(x0.z),
                             __uint_as_float(x0.w), __uint_as_float(x1.x), __uint_as_float(x1.y),
                             __uint_as_float(x1.z), __uint_as_float(x1.w)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // v_cvt_pk_bf16_f32 rounds a pair to nearest even in one step
          const float a0 = xs[2 * e], a1 = xs[2 * e + 1];
          const bf16x2 hi = {(__bf16)a0, (__bf16)a1};
          const uint32_t hu = __builtin_bit_cast(uint32_t, hi);
          const bf16x2 lo = {(__bf16)(a0 - __uint_as_float(hu << 16)),
                             (__bf16)(a1 - __uint_as_float(hu & 0xFFFF0000u))};
          abf[0][kb].u[e] = hu;
          abf[NT - 1][kb].u[e] = __builtin_bit_cast(uint32_t, lo);
        }
      } else {
        const int c = kb * 4 + (lane >> 4);
        const uint4 x = *(const uint4 *)(qst + h * QROWB + ((c ^ (h & kSwz)) * 16));
        abf[0][kb].u[0] = x.x; abf[0][kb].u[1] = x.y; abf[0][kb].u[2] = x.z; abf[0][kb].u[3] = x.w;
      }
    }
  }
  lds_barrier();  // the q~ copy is read: its stages take units from here on

  // ---- main loop: one barrier per unit ---------------------------------------
  const int row0 = th * 32 + (lane & 15), row1 = row0 + 16;  // B operand token rows
  f32x4 accO0 = {}, accO1 = {};
  auto epilogue = [&](int pp) INL {  // unit pp's partial of this head group -> LDS
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // ReLU as an integer max on the bit pattern (negative floats, -0.0
      // included, are negative integers); beta is already in
      p0 = fmaf(wv[i], __int_as_float(max(__float_as_int(accO0[i]), 0)), p0);
      p1 = fmaf(wv[i], __int_as_float(max(__float_as_int(accO1[i]), 0)), p1);
    }
    // reduce-scatter over the four lane groups (4 heads each): lanes 0-15
    // end with tile 0's token sums, lanes 32-47 with tile 1's
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1),
                                                    false, false);
    const float q = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(q), __float_as_uint(q), false,
                                                    false);
    const float v = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    if ((lane & 16) == 0) sh.red[pp & 1][hg][th * 32 + (lane & 15) + ((lane >> 5) << 4)] = v;
  };
  auto store_final = [&](int pp) INL {  // compute wavefront 0: the 64 scores of unit pp
    if (wave == 0) {
      const float *rd = &sh.red[pp & 1][0][0];
      const float v = ((rd[lane] + rd[kTok + lane]) + rd[2 * kTok + lane]) + rd[3 * kTok + lane];
      const int t = (u0 + pp) * kTok + lane;
      if (CAND) {
        if (t < mylen) out[(int64_t)myq * ld + t] = sh.page[pp * kTok + lane] < 0 ? -INFINITY : v;
      } else if (t < mylen) {
        out[(int64_t)myq * ld + t] = v;
        if (hist) atomicAdd(&hl[score_key(v) >> 20], 1u);
      }
    }
  };

  if (issuer) {
    for (int p = 0; p < nu; ++p) {
      // unit p has landed once this wavefront's loads of later units are
      // all that is left in flight
      wait_vm_rt(kPerIssuer * (issued - 1 - p));
      lds_barrier();  // unit p is in for everyone; unit p-1 has been read
      const int upto = min(nu, p + kAhead + 1);  // stage of unit p + kAhead = that of p - 1
      for (int u = issued; u < upto; ++u) issue_unit(u);
      issued = max(issued, upto);
    }
    if (nu > 0) lds_barrier();  // matches the compute wavefronts' last barrier
  } else {
    for (int p = 0; p < nu; ++p) {
      lds_barrier();
      if (p >= 2) store_final(p - 2);
      const char *sp = sh.stage[p % kNst];
      const char *rp0 = sp + row0 * kRowB, *rp1 = sp + row1 * kRowB;
      f32x4 acc0 = f32x4{bv[0], bv[1], bv[2], bv[3]}, acc1 = acc0;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        // half of r at a time keeps the B fragments at 32 registers
        bf16x8 b0[KB / 2], b1[KB / 2];
#pragma unroll
        for (int k = 0; k < KB / 2; ++k) {
          const int chunk = (half * KB / 2 + k) * 4 + (lane >> 4);
          b0[k] = *(const bf16x8 *)(rp0 + ((chunk ^ (row0 & kSwz)) * 16));
          b1[k] = *(const bf16x8 *)(rp1 + ((chunk ^ (row1 & kSwz)) * 16));
        }
#pragma unroll
        for (int k = 0; k < KB / 2; ++k)
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abf[t][half * KB / 2 + k].v, b0[k],
                                                           acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abf[t][half * KB / 2 + k].v, b1[k],
                                                           acc1, 0, 0, 0);
          }
      }
      if (p >= 1) epilogue(p - 1);
      accO0 = acc0;
      accO1 = acc1;
    }
    if (nu > 0) {
      epilogue(nu - 1);
      lds_barrier();
      if (nu >= 2) store_final(nu - 2);
      store_final(nu - 1);
    }
  }
  if (!CAND && hist) {
    // this range's histogram into the query's row histogram
    lds_barrier();
    uint32_t *gh = hist + (int64_t)myq * kHistBins;
    for (int i = tid; i < kHistBins; i += kThr) {
      const uint32_t c = hl[i];
      if (c) atomicAdd(gh + i, c);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load in flight at exit
}

// One workgroup per CU, two units each at least, one per query at least.
int scan_grid(int n_q, int64_t units_per_query) {
  const int64_t T = (int64_t)n_q * units_per_query;
  return (int)std::max<int64_t>(std::min<int64_t>(device_cu_count(), (T + 1) / 2), n_q);
}

// Most units one workgroup gets: a query with U units gets W > (G - n) U / T
// workgroups, so fewer than T / (G - n) + 1 units each; with G == n, U.
int64_t max_units_per_wg(int n_q, int64_t units_per_query) {
  const int G = scan_grid(n_q, units_per_query);
  const int64_t T = (int64_t)n_q * units_per_query;
  return G > n_q ? T / (G - n_q) + 1 : units_per_query;
}

// Candidate mode: with n_q a multiple of cand_rows, xw ranges per query and
// G = n_q * xw (the XCD-grouped plan); else the proportional plan (xw = 0).
void cand_plan(int n_q, int B, int cand_rows, int *G, int *xw) {
  const int64_t U = (B + kTok - 1) / kTok;
  if (n_q % cand_rows == 0) {
    *xw = (int)std::max<int64_t>(1, std::min<int64_t>(device_cu_count() / n_q, U));
    *G = n_q * *xw;
  } else {
    *xw = 0;
    *G = scan_grid(n_q, U);
  }
}

}  // namespace

bool score_scan_supported(int qt_dt, int H, int n_q, int max_len, const CacheView &cv) {
  if (!((qt_dt == LI_FP32 || qt_dt == LI_BF16) && H == 64 && cv.r == kR && cv.dtype == LI_BF16 &&
        n_q >= 1 && n_q <= kWave && n_q <= cv.n_seq && max_len >= 1))
    return false;
  return max_units_per_wg(n_q, (max_len + kTok - 1) / kTok) <= kMaxPages;  // pages fit the table
}

bool score_scan_cand_supported(int qt_dt, int H, int n_q, int B, int cand_rows,
                               const CacheView &cv) {
  if (!((qt_dt == LI_FP32 || qt_dt == LI_BF16) && H == 64 && cv.r == kR && cv.dtype == LI_BF16 &&
        n_q >= 1 && B >= 1 && cand_rows >= 1))
    return false;
  int G, xw;
  cand_plan(n_q, B, cand_rows, &G, &xw);
  const int64_t U = (B + kTok - 1) / kTok;
  const int64_t units = xw > 0 ? (U + xw - 1) / xw : max_units_per_wg(n_q, U);
  return units <= kMaxCandUnits;  // slots fit the table
}

hipError_t launch_score_scan(const void *q_tilde, int qt_dt, const float *w, const float *beta,
                             int n_q, const int32_t *q_seq, const int32_t *q_len, int max_len,
                             const CacheView &cv, float *out, int64_t ld, hipStream_t st,
                             uint32_t *hist, uint32_t *zbuf, int zwords) {
  const int G = scan_grid(n_q, (max_len + kTok - 1) / kTok);
  if (qt_dt == LI_FP32)
    score_scan_kernel<true, false><<<G, kThr, 0, st>>>(q_tilde, w, beta, n_q, q_seq, q_len, max_len,
                                                       cv, nullptr, 0, 1, 0, out, ld, hist, zbuf,
                                                       zwords);
  else
    score_scan_kernel<false, false><<<G, kThr, 0, st>>>(q_tilde, w, beta, n_q, q_seq, q_len, max_len,
                                                        cv, nullptr, 0, 1, 0, out, ld, hist, zbuf,
                                                        zwords);
  return hipGetLastError();
}

hipError_t launch_score_scan_cand(const void *q_tilde, int qt_dt, const float *w,
                                  const float *beta, int n_q, const int32_t *q_seq,
                                  const CacheView &cv, const int32_t *cand, int B, int cand_rows,
                                  float *out, int64_t ld, hipStream_t st) {
  int G, xw;
  cand_plan(n_q, B, cand_rows, &G, &xw);
  if (qt_dt == LI_FP32)
    score_scan_kernel<true, true><<<G, kThr, 0, st>>>(q_tilde, w, beta, n_q, q_seq, nullptr, 0, cv,
                                                      cand, B, cand_rows, xw, out, ld, nullptr,
                                                      nullptr, 0);
  else
    score_scan_kernel<false, true><<<G, kThr, 0, st>>>(q_tilde, w, beta, n_q, q_seq, nullptr, 0, cv,
                                                       cand, B, cand_rows, xw, out, ld, nullptr,
                                                       nullptr, 0);
  return hipGetLastError();
}

}  // namespace li
