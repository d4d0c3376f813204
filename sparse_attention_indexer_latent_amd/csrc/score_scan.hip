// Full-scan decode scorer: eq. (8) of the LatentIndex summary
// ("Methodology"), u_t = sum_h w_h ReLU(q~_h . c_t + beta_h) for every valid
// token t, H = 64 heads, at most 64 queries, over a bf16 cache (r = 192 or
// 256) or an fp8 E4M3FN cache with per-token scales (r = 128, 192 or 256; one
// scale per token, or one per 128-value block of the token).
//
// The scan streams the whole latent cache once per call, so it is bound by
// HBM.  Two properties of the hardware shape it:
//  * a CU holds only a few tens of KB of direct-to-LDS loads in flight, so
//    HBM stays busy only if some wavefront is always ready to issue the next
//    load; a wavefront that also computes leaves the CU's share of HBM idle
//    meanwhile.  Four issuer wavefronts therefore do nothing but stream
//    units into LDS, and eight compute wavefronts only score them;
//  * two workgroups on one CU finish several microseconds apart (the older
//    one's wavefronts win the arbitration), so there is one workgroup per CU
//    (its LDS use rules out a second) and a static, even split of the units.
//
// A unit is TU tokens (64 bf16 or 128 fp8: one or two cache pages), staged
// in one of NST LDS buffers as "LDS rows" of 256 bytes (fp8) or 512 bytes
// (bf16).  A token occupies one 16-byte-chunk slot range of a row: a whole
// row for r = 192 and 256 (r = 192 is padded to 256 in LDS; the pad chunks
// re-read real chunks of the same token, so they cost L2 requests but no HBM
// bytes, and meet zero query terms), half a row for r = 128 (two tokens per
// row).  Chunk c of a row sits at chunk c ^ (row & 15), so the matrix-core
// operand reads of 16 rows hit 16 different bank groups.  Compute wavefront
// w scores heads 16 (w & 3) .. +15 against half of the unit's tokens (w >> 2)
// as 16x16 tiles:
//  * bf16: v_mfma_f32_16x16x32_bf16, an fp32 q~ carried as bf16 hi + lo (a
//    bf16 q~ as is), beta as the accumulators' start value;
//  * fp8: v_mfma_f32_16x16x128_f8f6f4 with both operands fp8: each head's q~
//    is scaled by a power of two that brings its largest element into
//    (224, 448] and split into two E4M3 terms, the second the rounding of
//    what the first left (about 2^-8 relative, a bf16 q~'s precision); the
//    token's scale(s) and the head's power of two multiply the fp32 dot
//    product before beta and ReLU.
// The epilogue (ReLU, x w, sum over 16 heads) reduces across lanes and the
// four head groups are summed through LDS.  q~ of the query comes once per
// workgroup into the last two stages in the same round trip as the lengths,
// the page table, w and beta; the first NST - 2 units stream meanwhile.
// Queries get workgroups in proportion to their units (at least one each); a
// query's units are split evenly over its workgroups.
#include <algorithm>

#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

#define LDS3 __attribute__((address_space(3)))
#define INL __attribute__((always_inline))

constexpr int kCW = 8;                // compute wavefronts
constexpr int kIW = 4;                // issuer wavefronts
constexpr int kThr = (kCW + kIW) * kWave;
constexpr int kMaxPages = 1024;       // page table of one workgroup's range
constexpr int kTab = 4096;            // table entries (pages, or candidate rows)
constexpr int kTabPer = (kTab + kThr - 1) / kThr;
constexpr int kSwz = 15;
constexpr int kHistBins = 4096;       // row histogram of score keys, bits 31..20
constexpr int kStageArea = 128 * 1024;

// Shape of one instantiation: EB bytes per cache element (2 bf16, 1 fp8),
// R latent width, NSC scales per token (fp8: 1, or one per 128 values).
template <int EB, int R, int NSC>
struct Cfg {
  static constexpr bool C8 = EB == 1;
  static constexpr int RP = R <= 128 ? 128 : 256;     // width of a token slot in LDS
  static constexpr int SLOTB = RP * EB;               // bytes of a token slot
  static constexpr int LROWB = 256 * EB;              // bytes of an LDS row
  static constexpr int TPR = LROWB / SLOTB;           // tokens per LDS row (1 or 2)
  static constexpr int CPR = LROWB / 16;              // chunks per LDS row
  static constexpr int CPS = SLOTB / 16;              // chunks per token slot
  static constexpr int TOKB = R * EB;                 // bytes of a token in the cache
  static constexpr int CPT = TOKB / 16;               // real chunks per token
  static constexpr int TU = 128 / EB;                 // tokens per unit
  static constexpr int PPU = TU / kPage;              // cache pages per unit
  static constexpr int SB = TU * SLOTB;               // bytes of a stage
  static constexpr int NST = kStageArea / SB;         // LDS stages
  static constexpr int AHEAD = NST - 1;               // units in flight
  static constexpr int QST = NST - 2;                 // q~ sits in stages QST, QST + 1
  static constexpr int PIECES = SB / 1024;            // 1 KB loads per unit
  static constexpr int PER_ISSUER = PIECES / kIW;
  static constexpr int TPI = 1024 / SLOTB;            // tokens per 1 KB load
  static constexpr int MAX_CAND_UNITS = kTab / TU;
  static constexpr int NTILE = TU / 32;               // 16-token tiles per compute wavefront
  static constexpr int KB = C8 ? (R + 127) / 128 : R / 32;  // MFMA k-steps
  static_assert(PER_ISSUER * kIW == PIECES, "a unit splits evenly over the issuers");
  static_assert(kPage % (PER_ISSUER * TPI) == 0, "an issuer's pieces stay in one page");
  static_assert(PPU == 1 || PPU == 2, "a unit is one or two pages");
  static_assert(!C8 || NSC == 1 || NSC == KB, "fp8 scales: one per token or one per k-step");
  static_assert(NTILE % 2 == 0, "tiles pair up in the epilogue");
};

template <int E, int R, int NSC>
struct ScanShared {
  using C = Cfg<E, R, NSC>;
  __align__(16) char stage[C::NST][C::SB];
  int32_t page[kTab];  // block id of page i of the range; candidate mode: cache row of slot i (-1: none)
  // A page scan uses at most kMaxPages table entries; the rest of the table
  // and hext hold its histogram of score keys when one is asked for.
  uint32_t hext[kHistBins - (kTab - kMaxPages)];
  float red[2][4][C::TU];    // per head group partial scores, two units
  float ssc[C::C8 ? C::NST : 1][C::C8 ? C::TU * NSC : 1];  // fp8: token scales of each stage
  int32_t ok, myq, mylen, myseq, u0, nu;
};

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// s_waitcnt vmcnt(n) for a runtime n in [0, 47]
__device__ __forceinline__ void wait_vm_rt(int n) {
  switch (n) {
#define LI_W(k) case k: wait_vm<k>(); break;
    LI_W(0) LI_W(1) LI_W(2) LI_W(3) LI_W(4) LI_W(5) LI_W(6) LI_W(7) LI_W(8) LI_W(9) LI_W(10)
    LI_W(11) LI_W(12) LI_W(13) LI_W(14) LI_W(15) LI_W(16) LI_W(17) LI_W(18) LI_W(19) LI_W(20)
    LI_W(21) LI_W(22) LI_W(23) LI_W(24) LI_W(25) LI_W(26) LI_W(27) LI_W(28) LI_W(29) LI_W(30)
    LI_W(31) LI_W(32) LI_W(33) LI_W(34) LI_W(35) LI_W(36) LI_W(37) LI_W(38) LI_W(39) LI_W(40)
    LI_W(41) LI_W(42) LI_W(43) LI_W(44) LI_W(45) LI_W(46)
#undef LI_W
    default: wait_vm<47>(); break;
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
// cum(q) / T) with cum(q) the units of the queries before q and T all units:
// every query gets at least one, the rest in proportion to its units.
__device__ __forceinline__ int64_t wg_start(int q, int64_t cum, int64_t T, int G, int n) {
  return q + ((int64_t)(G - n) * cum) / T;
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

// Issuer wave j's scale loads per unit: the unit's scale instructions are
// dealt out round-robin (page mode: one; candidate mode: NSC * TU / 64).
template <bool C8, bool CAND, int TU, int NSC>
__device__ __forceinline__ int scale_loads(int j) {
  if constexpr (!C8) return 0;
  constexpr int n = CAND ? NSC * TU / 64 : 1;
  return j < n ? (n - 1 - j) / kIW + 1 : 0;
}

// CAND: candidate mode (HS followers).  Query i scores the B slots of
// candidate list c = i % cand_rows (token ids of sequence q_seq[c], -1 for
// padding) into out[i*ld + j]; units are TU consecutive slots; q_len and
// max_len are unused.
// hist (page scan only, may be null): [n_q][kHistBins] histograms of the
// order-preserving keys of the scores written (bin = key >> 20), added to
// what the array holds; zbuf[0 .. zwords) is zeroed on the way (the
// workgroups share it out), for a consumer that accumulates there next.
template <int EB, int R, int NSC, bool QF32, bool CAND>
__global__ void __launch_bounds__(kThr, 1)
score_scan_kernel(const void *__restrict__ q_tilde, const float *__restrict__ w,
                  const float *__restrict__ beta, int n_q, const int32_t *__restrict__ q_seq,
                  const int32_t *__restrict__ q_len, int max_len, CacheView cv,
                  const int32_t *__restrict__ cand, int B, int cand_rows, int xw,
                  float *__restrict__ out, int64_t ld, uint32_t *__restrict__ hist,
                  uint32_t *__restrict__ zbuf, int zwords) {
  using C = Cfg<EB, R, NSC>;
  constexpr bool C8 = C::C8;
  constexpr int TU = C::TU, NST = C::NST, KB = C::KB, NTILE = C::NTILE;
  // A operand terms: bf16 hi + lo of an fp32 q~, or the bf16 q~; fp8: two
  // terms (each the E4M3 rounding of what the earlier left: about 2^-8
  // relative, the precision of a bf16 q~, well inside the fp8 cache's own)
  constexpr int NT = C8 ? 2 : (QF32 ? 2 : 1);
  constexpr int QROWB = QF32 ? 4 * R : 2 * R;  // bytes of one head's q~ row
  constexpr int QCH = QROWB / 16;              // 16-byte chunks of a q~ row
  // q~ rows swizzle their chunks within aligned groups of 16 (or of 8 when
  // the row is 24 chunks), so a chunk never leaves its row
  constexpr int QSWZ = QCH % 16 == 0 ? 15 : 7;
  static_assert(QCH % (QSWZ + 1) == 0, "the q~ swizzle stays within a row");
  static_assert(64 * QROWB <= 2 * C::SB, "q~ fits in two stages");
  static_assert(64 * QROWB % (1024 * kCW) == 0, "q~ splits evenly over the compute waves");
  __shared__ ScanShared<EB, R, NSC> sh;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const bool issuer = wave >= kCW;
  const int hg = wave & 3, th = (wave >> 2) & 1;  // compute: head group, token half
  const int G = gridDim.x, g = blockIdx.x;
  char *const qst = sh.stage[C::QST];  // LDS copy of q~
  uint32_t *const hl = reinterpret_cast<uint32_t *>(&sh.page[kMaxPages]);  // page scan histogram

  // q~ of query q -> LDS (64 x QROWB bytes), 16-byte chunk c of head row h
  // at chunk c ^ (h & QSWZ) (which keeps c within its row): 1 KB per load,
  // each compute wavefront an eighth.
  auto fetch_q = [&](int q) INL {
    constexpr int NL = 64 * QROWB / 1024 / kCW;  // loads per compute wavefront
    if (!issuer) {
#pragma unroll
      for (int m = 0; m < NL; ++m) {
        const int gi = wave * NL + m;
        const int e = gi * 64 + lane;  // chunk index over the 64 heads
        const int h = e / QCH, c = e % QCH;
        dma16_to_lds((const char *)q_tilde + ((int64_t)q * 64 + h) * QROWB + ((c ^ (h & QSWZ)) * 16),
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

  // ---- issuers --------------------------------------------------------------
  // Load piece gi of a unit covers LDS chunk slots gi*64 .. +63 of its stage:
  // lane l fills slot p = gi*64 + l, i.e. LDS row p / CPR, chunk (p % CPR) ^
  // (row & 15) of that row, which is chunk c of token slot h of the row.
  const char *gdata = (const char *)cv.data;
  const int iw = wave - kCW;  // issuer index
  const int gi0 = iw * C::PER_ISSUER;
  const int nsl = scale_loads<C8, CAND, TU, NSC>(iw);  // this issuer's scale loads per unit
  const int vpu = C::PER_ISSUER + nsl;                  // its loads per unit
  // (token of the unit, chunk of the token) that lane fills in piece gi
  auto piece_src = [&](int gi, int &t, int &cc) INL {
    const int p = gi * 64 + lane;
    const int row = p / C::CPR;
    const int lc = (p % C::CPR) ^ (row & kSwz);
    const int h = lc / C::CPS, c = lc % C::CPS;
    t = row * C::TPR + h;
    cc = c < C::CPT ? c : c - C::CPT;  // pad chunks re-read real ones
  };
  // page mode: unit u's pages b0 (and b1); this issuer's pieces all fall in
  // page `mypage` of the unit
  const int mypage = (gi0 * C::TPI) / kPage;
  auto issue_page_unit = [&](int u, int b0, int b1) INL {
    const int b = mypage ? b1 : b0;
    LDS3 char *st = (LDS3 char *)sh.stage[u % NST];
    const int64_t base = (int64_t)((b >= 0 && b < cv.n_blocks) ? b : 0) * kPage;
#pragma unroll
    for (int m = 0; m < C::PER_ISSUER; ++m) {
      const int gi = gi0 + m;
      int t, cc;
      piece_src(gi, t, cc);
      dma16_to_lds(gdata + (base + (t % kPage)) * C::TOKB + cc * 16, (LDS3 void *)(st + gi * 1024));
    }
    if constexpr (C8) {
      if (nsl) {
        // the unit's PPU pages' scales, [64][NSC] floats each: lanes 16 NSC j ..
        // of page j
        constexpr int LPP = 16 * NSC;  // lanes per page
        const int j = lane / LPP;
        if (j < C::PPU) {
          const int bj = j ? b1 : b0;
          const int64_t sb = (int64_t)((bj >= 0 && bj < cv.n_blocks) ? bj : 0) * kPage * NSC;
          dma16_to_lds((const char *)(cv.scale + sb) + (lane % LPP) * 16,
                       (LDS3 void *)&sh.ssc[u % NST][0]);
        }
      }
    }
  };

  // ---- plan: guess (every query max_len long, query q on sequence q) ------
  // (exact in candidate mode: every query has B slots)
  const int UPQ = ((CAND ? B : max_len) + TU - 1) / TU;  // units per query
  const int64_t T0 = (int64_t)n_q * UPQ;
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
    gu0 = (int)((int64_t)r * UPQ / xw);
    gnu = (int)((int64_t)(r + 1) * UPQ / xw) - gu0;
  } else {
    for (int q = 1; q < n_q; ++q)
      if (wg_start(q, (int64_t)q * UPQ, T0, G, n_q) <= g) gq = q;
    const int s = (int)wg_start(gq, (int64_t)gq * UPQ, T0, G, n_q);
    const int W = (int)wg_start(gq + 1, (int64_t)(gq + 1) * UPQ, T0, G, n_q) - s;
    const int j = g - s;
    gu0 = (int)((int64_t)j * UPQ / W);
    gnu = (int)((int64_t)(j + 1) * UPQ / W) - gu0;
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
    const int s0 = gu0 * TU, ns = min(gnu * TU, B - s0);  // slots of the range
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
      if (i < gnu * TU && i < kTab) sh.page[i] = tk[k] < 0 ? -1 : b * kPage + (tk[k] & 63);
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
    // The guessed range's first units stream while the plan is checked (a
    // wrong guess waits for them and loads those stages again).  The issuers
    // make no other loads here, so no wait for the plan's loads holds these.
    // All block ids first (a wait for one must not wait for pages), and all
    // QST units unconditionally so the loads issue together: past a short
    // range they fetch a clamped page into a stage nothing reads, and the
    // waits below, which count only the range's units, stay conservative.
    int bsc[C::QST][2];
    const int npg = max(gnu * C::PPU - 1, 0);
#pragma unroll
    for (int u = 0; u < C::QST; ++u) {
#pragma unroll
      for (int j = 0; j < C::PPU; ++j)
        bsc[u][j] = cv.block_table[(int64_t)gq * cv.max_blocks +
                                   min(gu0 * C::PPU + min(u * C::PPU + j, npg), cv.max_blocks - 1)];
      if (C::PPU == 1) bsc[u][1] = bsc[u][0];
    }
#pragma unroll
    for (int u = 0; u < C::QST; ++u) {
      asm volatile("" : "+v"(bsc[u][0]));  // the loads land here
      asm volatile("" : "+v"(bsc[u][1]));
    }
#pragma unroll
    for (int u = 0; u < C::QST; ++u) issue_page_unit(u, bsc[u][0], bsc[u][1]);
  } else {
    constexpr int kCT = kCW * kWave;  // compute threads
    static_assert(2 * kCT >= kMaxPages, "two page-table entries per compute thread");
    const int li = min(lane, n_q - 1);
    int len0 = min(max(q_len[li], 0), max_len), seq0 = q_seq[li];
    if (lane >= n_q) len0 = seq0 = 0;
    const int npg = gnu * C::PPU;  // pages of the guessed range
    int pg[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = min(tid + k * kCT, max(npg - 1, 0));
      pg[k] = cv.block_table[(int64_t)gq * cv.max_blocks + min(gu0 * C::PPU + i, cv.max_blocks - 1)];
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
      if (tid + k * kCT < npg) sh.page[tid + k * kCT] = pg[k];
    if (wave == 0) {
      const bool bad = lane < n_q && (((len0 + TU - 1) / TU) != UPQ || seq0 != lane);
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
        const int units = lane < n_q ? (len + TU - 1) / TU : 0;
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
  // that copy.  (Issuers of a page scan have only their early units in
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
    for (int i = tid; i < nu * C::PPU; i += kThr)
      sh.page[i] = cv.block_table[(int64_t)sq * cv.max_blocks + min(u0 * C::PPU + i, cv.max_blocks - 1)];
    // a wait the compiler sees, so that it knows w and beta have landed too
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();
  }
  const int myq = sh.myq, mylen = sh.mylen, u0 = sh.u0, nu = sh.nu;

  // ---- issuers: unit u of the range (PPU pages, or TU candidate rows) ------
  auto issue_unit = [&](int u) INL {
    if constexpr (CAND) {
      LDS3 char *st = (LDS3 char *)sh.stage[u % NST];
#pragma unroll
      for (int m = 0; m < C::PER_ISSUER; ++m) {
        const int gi = gi0 + m;
        int t, cc;
        piece_src(gi, t, cc);
        const int64_t row = max(sh.page[u * TU + t], 0);  // a padding slot reads row 0
        dma16_to_lds(gdata + row * C::TOKB + cc * 16, (LDS3 void *)(st + gi * 1024));
      }
      if constexpr (C8) {
        // candidate scales, NSC dwords each, instruction n: entries 64 n .. +63
        for (int k = 0; k < nsl; ++k) {
          const int n = iw + k * kIW;
          const int e = n * 64 + lane;
          const int64_t row = max(sh.page[u * TU + e / NSC], 0);
          dma4_to_lds(cv.scale + row * NSC + e % NSC, (LDS3 void *)&sh.ssc[u % NST][n * 64]);
        }
      }
    } else {
      const int b0 = sh.page[u * C::PPU];
      const int b1 = C::PPU > 1 ? sh.page[u * C::PPU + 1] : b0;
      issue_page_unit(u, b0, b1);
    }
  };
  // prologue: units clear of the q~ copy (a page scan whose guess held has
  // issued them already; after the slow path every load has landed)
  int issued = (!CAND && sh.ok) ? min(nu, C::QST) : 0;
  if (issuer)
    for (int u = issued; u < min(nu, C::QST); ++u) issue_unit(u);
  issued = min(nu, C::QST);

  // ---- compute: A operands of heads 16 hg .. +15 from the q~ copy -----------
  // bf16: lane holds k = kb*32 + (lane/16)*8 + [0, 8) of head 16 hg + lane%16;
  // fp8: k = kb*128 + (lane/16)*32 + [0, 32).  k >= R holds zero.
  // The lane's raw q~ words leave LDS first; once every wavefront has them
  // the q~ stages are free, and the main loop's first barrier hands them to
  // the issuers.  (Issuing into them right here delays unit 0: those loads
  // queue ahead of the wait for it.)
  constexpr int RAW = C8 ? KB * (QF32 ? 8 : 4) : (QF32 ? 2 * KB : KB);  // 16-byte chunks
  uint4 qr[RAW];
  if (!issuer) {
    const int h = 16 * hg + (lane & 15);
    auto qchunk = [&](int c) INL -> uint4 {  // 16-byte chunk c of the head's row
      return *(const uint4 *)(qst + h * QROWB + ((c ^ (h & QSWZ)) * 16));
    };
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if constexpr (!C8) {
        if constexpr (QF32) {  // floats kb*32 + (lane/16)*8 .. +7: chunks c0, c0 + 1
          const int c0 = 2 * (kb * 4 + (lane >> 4));
          qr[2 * kb] = qchunk(c0);
          qr[2 * kb + 1] = qchunk(c0 + 1);
        } else {
          qr[kb] = qchunk(kb * 4 + (lane >> 4));
        }
      } else {
        const int k0 = kb * 128 + (lane >> 4) * 32;
        const bool in = k0 < R;  // R is a multiple of 64: a lane's 32 are all in or all out
        constexpr int NCH = QF32 ? 8 : 4;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          qr[kb * NCH + c] = in ? qchunk((k0 * (QF32 ? 4 : 2)) / 16 + c) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  lds_barrier();  // the q~ copy is read: its stages take units from here on

  Frag abf[C8 ? 1 : NT][C8 ? 1 : KB];
  i32x8 a8[C8 ? NT : 1][C8 ? KB : 1];
  float hs[4];  // fp8: the power of two of heads 16 hg + 4 (lane/16) + i, as 2^-k
  if (!issuer) {
    if constexpr (!C8) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if constexpr (QF32) {
          const uint4 x0 = qr[2 * kb], x1 = qr[2 * kb + 1];
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
          const uint4 x = qr[kb];
          abf[0][kb].u[0] = x.x; abf[0][kb].u[1] = x.y; abf[0][kb].u[2] = x.z; abf[0][kb].u[3] = x.w;
        }
      }
    } else {
      // the lane's KB x 32 elements as fp32 (zero beyond R)
      float qv[KB][32];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        constexpr int NCH = QF32 ? 8 : 4;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const uint4 x = qr[kb * NCH + c];
          if constexpr (QF32) {
            qv[kb][4 * c + 0] = __uint_as_float(x.x); qv[kb][4 * c + 1] = __uint_as_float(x.y);
            qv[kb][4 * c + 2] = __uint_as_float(x.z); qv[kb][4 * c + 3] = __uint_as_float(x.w);
          } else {
            const uint32_t xx[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              qv[kb][8 * c + 2 * e] = bf16_bits_to_f32(xx[e] & 0xFFFFu);
              qv[kb][8 * c + 2 * e + 1] = bf16_bits_to_f32(xx[e] >> 16);
            }
          }
        }
      }
      float m = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 32; ++j) m = fmaxf(m, fabsf(qv[kb][j]));
      m = fmaxf(m, __shfl_xor(m, 16, kWave));
      m = fmaxf(m, __shfl_xor(m, 32, kWave));  // the head's largest |q~|
      const int ke = fp8_head_exponent(m);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ki = __shfl(ke, 4 * (lane >> 4) + i, kWave);  // head 16 hg + 4 (lane/16) + i
        hs[i] = ldexpf(1.f, -ki);
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {  // bytes 4j .. 4j+3 of this k-step's 32
          float r[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = ldexpf(qv[kb][4 * j + e], ke);
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
  }

  // ---- main loop: one barrier per unit ---------------------------------------
  // Compute wave (hg, th): tiles j of tokens th * TU/2 + 16 j + lane%16.
  // last unit's accumulators; fp8: already times the token scale(s) (the
  // head's power of two, applied in the epilogue, is exact in either order)
  f32x4 accO[NTILE];
  auto epilogue = [&](int pp) INL {  // unit pp's partial of this head group -> LDS
#pragma unroll
    for (int jp = 0; jp < NTILE / 2; ++jp) {
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x0 = accO[2 * jp][i], x1 = accO[2 * jp + 1][i];
        if constexpr (C8) {  // bf16: beta is already in (the MFMAs' start value)
          x0 = x0 * hs[i] + bv[i];
          x1 = x1 * hs[i] + bv[i];
        }
        // ReLU as an integer max on the bit pattern (negative floats, -0.0
        // included, are negative integers)
        p0 = fmaf(wv[i], __int_as_float(max(__float_as_int(x0), 0)), p0);
        p1 = fmaf(wv[i], __int_as_float(max(__float_as_int(x1), 0)), p1);
      }
      // reduce-scatter over the four lane groups (4 heads each): lanes 0-15
      // end with tile 2 jp's token sums, lanes 32-47 with tile 2 jp + 1's
      const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1),
                                                      false, false);
      const float q = __uint_as_float(a[0]) + __uint_as_float(a[1]);
      const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(q), __float_as_uint(q), false,
                                                      false);
      const float v = __uint_as_float(b[0]) + __uint_as_float(b[1]);
      if ((lane & 16) == 0)
        sh.red[pp & 1][hg][th * (TU / 2) + 32 * jp + (lane & 15) + ((lane >> 5) << 4)] = v;
    }
  };
  auto store_final = [&](int pp) INL {  // compute wavefront 0: the TU scores of unit pp
    if (wave == 0) {
#pragma unroll
      for (int k = 0; k < TU / kWave; ++k) {
        const int tt = k * kWave + lane;
        const float *rd = &sh.red[pp & 1][0][0];
        const float v = ((rd[tt] + rd[TU + tt]) + rd[2 * TU + tt]) + rd[3 * TU + tt];
        const int t = (u0 + pp) * TU + tt;
        if (CAND) {
          if (t < mylen) out[(int64_t)myq * ld + t] = sh.page[pp * TU + tt] < 0 ? -INFINITY : v;
        } else if (t < mylen) {
          out[(int64_t)myq * ld + t] = v;
          if (hist) atomicAdd(&hl[score_key(v) >> 20], 1u);
        }
      }
    }
  };

  if (issuer) {
    for (int p = 0; p < nu; ++p) {
      // unit p has landed once this wavefront's loads of later units are
      // all that is left in flight
      wait_vm_rt(vpu * (issued - 1 - p));
      lds_barrier();  // unit p is in for everyone; unit p-1 has been read
      // At most one unit per barrier: an issue stalls while the CU's
      // outstanding loads are at their limit, so a second unit here would
      // hold this wavefront (and with it the next barrier) until part of
      // the first had landed.  After the q~ stages free up that keeps two
      // units in flight beyond the one being computed.
      const int upto = min(nu, min(p + C::AHEAD + 1, issued + 1));  // stage of p + AHEAD = that of p - 1
      for (int u = issued; u < upto; ++u) issue_unit(u);
      issued = max(issued, upto);
    }
    if (nu > 0) lds_barrier();  // matches the compute wavefronts' last barrier
  } else {
    for (int p = 0; p < nu; ++p) {
      lds_barrier();
      if (p >= 2) store_final(p - 2);
      const char *sp = sh.stage[p % NST];
      f32x4 acc[NTILE][C8 ? NSC : 1];
      float sc[NTILE][NSC];
      // tiles in pairs, their independent accumulation chains interleaved
#pragma unroll
      for (int jp = 0; jp < NTILE / 2; ++jp) {
        const int t0 = th * (TU / 2) + 32 * jp + (lane & 15), t1 = t0 + 16;  // tokens of the unit
        const int row0 = t0 / C::TPR, row1 = t1 / C::TPR;
        const int hs0 = t0 % C::TPR, hs1 = t1 % C::TPR;
        const char *rp0 = sp + row0 * C::LROWB, *rp1 = sp + row1 * C::LROWB;
        auto chunk0 = [&](int lc) INL -> uint4 {  // logical chunk lc of tile 2 jp's row
          return *(const uint4 *)(rp0 + ((lc ^ (row0 & kSwz)) * 16));
        };
        auto chunk1 = [&](int lc) INL -> uint4 {
          return *(const uint4 *)(rp1 + ((lc ^ (row1 & kSwz)) * 16));
        };
        f32x4 &a0 = acc[2 * jp][0], &a1 = acc[2 * jp + 1][0];
        if constexpr (!C8) {
          a0 = f32x4{bv[0], bv[1], bv[2], bv[3]};
          a1 = a0;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            // half of the k-steps at a time keeps the B fragments few
            constexpr int KH = (KB + 1) / 2;
            bf16x8 b0[KH], b1[KH];
#pragma unroll
            for (int k = 0; k < KH; ++k) {
              const int kb = half * KH + k;
              if (kb < KB) {
                b0[k] = __builtin_bit_cast(bf16x8, chunk0(hs0 * C::CPS + kb * 4 + (lane >> 4)));
                b1[k] = __builtin_bit_cast(bf16x8, chunk1(hs1 * C::CPS + kb * 4 + (lane >> 4)));
              }
            }
#pragma unroll
            for (int k = 0; k < KH; ++k) {
              const int kb = half * KH + k;
              if (kb < KB) {
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                  a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abf[tt][kb].v, b0[k], a0, 0, 0, 0);
                  a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(abf[tt][kb].v, b1[k], a1, 0, 0, 0);
                }
              }
            }
          }
        } else {
#pragma unroll
          for (int s2 = 0; s2 < NSC; ++s2) {
            acc[2 * jp][s2] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc[2 * jp + 1][s2] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          i32x8 bb0[KB], bb1[KB];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const int lc0 = hs0 * C::CPS + kb * 8 + 2 * (lane >> 4);
            const int lc1 = hs1 * C::CPS + kb * 8 + 2 * (lane >> 4);
            const uint4 x0 = chunk0(lc0), x1 = chunk0(lc0 + 1);
            const uint4 y0 = chunk1(lc1), y1 = chunk1(lc1 + 1);
            bb0[kb] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                            (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
            bb1[kb] = i32x8{(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w,
                            (int)y1.x, (int)y1.y, (int)y1.z, (int)y1.w};
          }
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const int s2 = NSC == 1 ? 0 : kb;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
              // operands fp8 E4M3 (format code 0) for A and B
              acc[2 * jp][s2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  a8[tt][kb], bb0[kb], acc[2 * jp][s2], 0, 0, 0, 0, 0, 0);
              acc[2 * jp + 1][s2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  a8[tt][kb], bb1[kb], acc[2 * jp + 1][s2], 0, 0, 0, 0, 0, 0);
            }
          }
#pragma unroll
          for (int s2 = 0; s2 < NSC; ++s2) {
            sc[2 * jp][s2] = sh.ssc[p % NST][t0 * NSC + s2];
            sc[2 * jp + 1][s2] = sh.ssc[p % NST][t1 * NSC + s2];
          }
        }
      }
      if (p >= 1) epilogue(p - 1);
#pragma unroll
      for (int j = 0; j < NTILE; ++j) {
        if constexpr (C8) {
          accO[j] = acc[j][0] * sc[j][0];
#pragma unroll
          for (int s = 1; s < NSC; ++s) accO[j] += acc[j][s] * sc[j][s];
        } else {
          accO[j] = acc[j][0];
        }
      }
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
void cand_plan(int n_q, int64_t U, int cand_rows, int *G, int *xw) {
  if (n_q % cand_rows == 0) {
    *xw = (int)std::max<int64_t>(1, std::min<int64_t>(device_cu_count() / n_q, U));
    *G = n_q * *xw;
  } else {
    *xw = 0;
    *G = scan_grid(n_q, U);
  }
}

// Scales per token of an fp8 cache (1, or one per 128 values), 0 if the
// cache's shape has no instantiation here.
int scan_nsc(const CacheView &cv) {
  if (cv.dtype != LI_FP8_E4M3) return 1;
  if (cv.scale_block == 0) return 1;
  return cv.scale_block == 128 ? (cv.r + 127) / 128 : 0;
}

bool shape_ok(int qt_dt, int H, const CacheView &cv) {
  if (!((qt_dt == LI_FP32 || qt_dt == LI_BF16) && H == 64)) return false;
  if (cv.dtype == LI_BF16) return cv.r == 256 || cv.r == 192;
  if (cv.dtype == LI_FP8_E4M3) {
    const int nsc = scan_nsc(cv);
    return (cv.r == 256 || cv.r == 192 || cv.r == 128) && (nsc == 1 || nsc == (cv.r + 127) / 128);
  }
  return false;
}

int unit_tokens(const CacheView &cv) { return cv.dtype == LI_FP8_E4M3 ? 128 : 64; }

template <int EB, int R, int NSC, bool CAND>
hipError_t launch_shape(const void *q_tilde, int qt_dt, const float *w, const float *beta, int n_q,
                        const int32_t *q_seq, const int32_t *q_len, int max_len,
                        const CacheView &cv, const int32_t *cand, int B, int cand_rows, int xw,
                        int G, float *out, int64_t ld, uint32_t *hist, uint32_t *zbuf,
                        int zwords, hipStream_t st) {
  if (qt_dt == LI_FP32)
    score_scan_kernel<EB, R, NSC, true, CAND><<<G, kThr, 0, st>>>(
        q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, cand, B, cand_rows, xw, out, ld, hist,
        zbuf, zwords);
  else
    score_scan_kernel<EB, R, NSC, false, CAND><<<G, kThr, 0, st>>>(
        q_tilde, w, beta, n_q, q_seq, q_len, max_len, cv, cand, B, cand_rows, xw, out, ld, hist,
        zbuf, zwords);
  return hipGetLastError();
}

template <bool CAND>
hipError_t dispatch(const void *q_tilde, int qt_dt, const float *w, const float *beta, int n_q,
                    const int32_t *q_seq, const int32_t *q_len, int max_len, const CacheView &cv,
                    const int32_t *cand, int B, int cand_rows, int xw, int G, float *out,
                    int64_t ld, uint32_t *hist, uint32_t *zbuf, int zwords, hipStream_t st) {
#define LI_SHAPE(EB, R, NSC)                                                                    \
  return launch_shape<EB, R, NSC, CAND>(q_tilde, qt_dt, w, beta, n_q, q_seq, q_len, max_len, cv, \
                                        cand, B, cand_rows, xw, G, out, ld, hist, zbuf, zwords, st)
  if (cv.dtype == LI_BF16) {
    if (cv.r == 256) LI_SHAPE(2, 256, 1);
    LI_SHAPE(2, 192, 1);
  }
  const int nsc = scan_nsc(cv);
  if (cv.r == 256) {
    if (nsc == 1) LI_SHAPE(1, 256, 1);
    LI_SHAPE(1, 256, 2);
  }
  if (cv.r == 192) {
    if (nsc == 1) LI_SHAPE(1, 192, 1);
    LI_SHAPE(1, 192, 2);
  }
  LI_SHAPE(1, 128, 1);
#undef LI_SHAPE
}

}  // namespace

bool score_scan_supported(int qt_dt, int H, int n_q, int max_len, const CacheView &cv) {
  if (!(shape_ok(qt_dt, H, cv) && n_q >= 1 && n_q <= kWave && n_q <= cv.n_seq && max_len >= 1))
    return false;
  const int TU = unit_tokens(cv);
  return max_units_per_wg(n_q, (max_len + TU - 1) / TU) * (TU / kPage) <= kMaxPages;  // pages fit
}

bool score_scan_cand_supported(int qt_dt, int H, int n_q, int B, int cand_rows,
                               const CacheView &cv) {
  if (!(shape_ok(qt_dt, H, cv) && n_q >= 1 && B >= 1 && cand_rows >= 1)) return false;
  const int TU = unit_tokens(cv);
  const int64_t U = (B + TU - 1) / TU;
  int G, xw;
  cand_plan(n_q, U, cand_rows, &G, &xw);
  const int64_t units = xw > 0 ? (U + xw - 1) / xw : max_units_per_wg(n_q, U);
  return units * TU <= kTab;  // slots fit the table
}

hipError_t launch_score_scan(const void *q_tilde, int qt_dt, const float *w, const float *beta,
                             int n_q, const int32_t *q_seq, const int32_t *q_len, int max_len,
                             const CacheView &cv, float *out, int64_t ld, hipStream_t st,
                             uint32_t *hist, uint32_t *zbuf, int zwords) {
  const int TU = unit_tokens(cv);
  const int G = scan_grid(n_q, (max_len + TU - 1) / TU);
  return dispatch<false>(q_tilde, qt_dt, w, beta, n_q, q_seq, q_len, max_len, cv, nullptr, 0, 1, 0,
                         G, out, ld, hist, zbuf, zwords, st);
}

hipError_t launch_score_scan_cand(const void *q_tilde, int qt_dt, const float *w,
                                  const float *beta, int n_q, const int32_t *q_seq,
                                  const CacheView &cv, const int32_t *cand, int B, int cand_rows,
                                  float *out, int64_t ld, hipStream_t st) {
  const int TU = unit_tokens(cv);
  int G, xw;
  cand_plan(n_q, (B + TU - 1) / TU, cand_rows, &G, &xw);
  return dispatch<true>(q_tilde, qt_dt, w, beta, n_q, q_seq, nullptr, 0, cv, cand, B, cand_rows,
                        xw, G, out, ld, nullptr, nullptr, 0, st);
}

}  // namespace li
