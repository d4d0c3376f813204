// Vector-ALU scorer for eq. (8) of the LatentIndex summary ("Methodology"):
// u_t = sum_h w_h ReLU(q~_h . c_t + beta_h).
//
// This path serves shapes where the head x latent product is small (H * r of a
// few hundred: about 4 flop per cached byte, far below the fp32 VALU ridge),
// any cache dtype, and shapes the matrix-core scorer does not take.  Each
// workgroup takes a tile of TT tokens of one query: the query's absorbed
// vectors and the tile (dequantised to fp32, row stride r+1 so that lanes
// reading different tokens hit different banks) are staged in LDS; thread
// (token, head group) accumulates its heads, and the head groups are summed
// in a fixed order.
#include <algorithm>

#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

__global__ void __launch_bounds__(256)
score_valu_kernel(const void *__restrict__ q_tilde, int qt_dt, const float *__restrict__ w,
                  const float *__restrict__ beta, int H, const int32_t *__restrict__ q_seq,
                  const int32_t *__restrict__ q_len, CacheView cv, const int32_t *__restrict__ cand,
                  int B, int cand_rows, float *__restrict__ out, int64_t ld, int TT, int max_len) {
  extern __shared__ float lds[];
  const int r = cv.r;
  const int i = blockIdx.y;
  const int t0 = blockIdx.x * TT;
  const int n = cand ? B : min(max(q_len[i], 0), max_len);
  if (t0 >= n) return;  // uniform across the workgroup, before any barrier
  const int nt = min(TT, n - t0);
  float *qs = lds;                      // [H][r]
  float *wsm = qs + H * r;              // [H]
  float *bsm = wsm + H;                 // [H]
  const int ns = max(n_scales(cv), 1);  // scales per token (fp8), else 1
  const int sbk = cv.scale_block ? cv.scale_block : r;  // values per scale
  float *ssm = bsm + H;                 // [TT][ns] token scales
  float *cs = ssm + TT * ns;            // [TT][r + 1]
  float *red = cs + TT * (r + 1);       // [256 / TT][TT]
  const int tid = threadIdx.x;
  const int64_t qoff = (int64_t)i * H * r;
  for (int e = tid; e < H * r; e += 256)
    qs[e] = qt_dt == LI_FP32 ? ((const float *)q_tilde)[qoff + e]
                             : bf16_bits_to_f32(((const uint16_t *)q_tilde)[qoff + e]);
  for (int h = tid; h < H; h += 256) {
    wsm[h] = w[(int64_t)i * H + h];
    bsm[h] = beta ? beta[(int64_t)i * H + h] : 0.f;
  }
  const int ci = cand ? i % cand_rows : i;  // candidate lists repeat every cand_rows queries
  const int seq = q_seq[ci];
  const int32_t *bt = cv.block_table + (int64_t)seq * cv.max_blocks;
  // token of a slot: the position itself, or the candidate (-1: padding,
  // which reads pool row 0 and stores -inf)
  auto token_of = [&](int slot) -> int { return cand ? cand[(int64_t)ci * B + slot] : slot; };
  auto phys_row = [&](int slot) -> int64_t {
    const int t = token_of(slot);
    return t >= 0 ? (int64_t)bt[t / kPage] * kPage + t % kPage : 0;
  };
  for (int e = tid; e < TT * ns; e += 256) {
    const int tok = e / ns, g = e % ns;
    float sc = 1.f;
    if (tok < nt && cv.dtype == LI_FP8_E4M3) sc = cv.scale[phys_row(t0 + tok) * ns + g];
    ssm[e] = sc;
  }
  for (int e = tid; e < TT * r; e += 256) {
    const int tok = e / r, j = e % r;
    float v = 0.f;
    if (tok < nt) v = load_latent(cv.data, cv.dtype, phys_row(t0 + tok) * r + j);
    cs[tok * (r + 1) + j] = v;
  }
  __syncthreads();
  const int n_groups = 256 / TT;
  const int tok = tid % TT, hg = tid / TT;
  const float *c = cs + tok * (r + 1);
  const float *sc = ssm + tok * ns;
  float acc = 0.f;
  for (int h = hg; h < H; h += n_groups) {
    const float *qh = qs + h * r;
    float x;
    if (ns == 1) {
      float dot = 0.f;
      for (int j = 0; j < r; ++j) dot = fmaf(qh[j], c[j], dot);
      x = fmaf(dot, sc[0], bsm[h]);
    } else {  // each block's dot product times its scale
      x = bsm[h];
      for (int g = 0; g < ns; ++g) {
        float dot = 0.f;
        for (int j = g * sbk; j < min(r, (g + 1) * sbk); ++j) dot = fmaf(qh[j], c[j], dot);
        x = fmaf(dot, sc[g], x);
      }
    }
    acc = fmaf(wsm[h], fmaxf(x, 0.f), acc);
  }
  red[hg * TT + tok] = acc;
  __syncthreads();
  if (tid < nt) {
    float s = 0.f;
    for (int g = 0; g < n_groups; ++g) s += red[g * TT + tid];
    out[(int64_t)i * ld + t0 + tid] = (cand && token_of(t0 + tid) < 0) ? -INFINITY : s;
  }
}

size_t valu_lds_bytes(int H, int r, int TT, int ns) {
  return sizeof(float) * ((size_t)H * r + 2 * H + (size_t)TT * ns + (size_t)TT * (r + 1) + 256);
}

}  // namespace

hipError_t launch_score_valu(const void *q_tilde, int qt_dt, const float *w, const float *beta,
                             int n_q, int H, const int32_t *q_seq, const int32_t *q_len,
                             int max_len, const CacheView &cv, const int32_t *cand, int B,
                             int cand_rows, float *out, int64_t ld, hipStream_t st) {
  int TT = 64;
  const int ns = std::max(n_scales(cv), 1);
  while (TT > 4 && valu_lds_bytes(H, cv.r, TT, ns) > 160 * 1024) TT >>= 1;
  const size_t lds = valu_lds_bytes(H, cv.r, TT, ns);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  static DeviceOnce *const once = device_once_new();
  const hipError_t e = raise_lds_limit(once, (const void *)score_valu_kernel, 160 * 1024);
  if (e != hipSuccess) return e;
  dim3 grid((max_len + TT - 1) / TT, n_q);
  score_valu_kernel<<<grid, 256, lds, st>>>(q_tilde, qt_dt, w, beta, H, q_seq, q_len, cv, cand, B,
                                            max(cand_rows, 1), out, ld, TT, max_len);
  return hipGetLastError();
}

}  // namespace li
