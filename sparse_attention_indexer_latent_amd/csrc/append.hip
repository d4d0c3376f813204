// li_append_latent: build and store the shared latent of new tokens
// (LatentIndex summary, "Methodology", eqs. 1-2).
//
//  1. (P given) project: partial[ks][tok][j] = sum_{i in slice ks} x[tok][i] P[i][j]
//     split over d_model slices so that P is streamed once per token tile;
//     the slices are summed in a fixed order in step 2 (deterministic).
//  2. one wavefront per token: y = sum of slices (or x itself), rotate the
//     leading r_R coordinates pairwise by pos * theta_j, then store as fp32,
//     bf16 (RNE) or fp8 E4M3FN with a per-token scale into the paged slot.
#include "absorb_block.h"
#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

constexpr int kProjCols = 256;   // output columns per workgroup (one per thread)
constexpr int kProjTok = 8;      // tokens per workgroup
constexpr int kProjSlice = 128;  // d_model rows per slice

template <typename T>
__device__ __forceinline__ float ld_f32(const T *p, int64_t i);
template <>
__device__ __forceinline__ float ld_f32<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_f32<uint16_t>(const uint16_t *p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

template <typename T>
__global__ void __launch_bounds__(kProjCols)
project_kernel(const T *__restrict__ x, const T *__restrict__ P, int n_tok, int d_model, int r,
               float *__restrict__ partial) {
  __shared__ float xs[kProjTok][kProjSlice];
  const int j = blockIdx.x * kProjCols + threadIdx.x;
  const int tok0 = blockIdx.y * kProjTok;
  const int i0 = blockIdx.z * kProjSlice;
  const int ni = min(kProjSlice, d_model - i0);
  for (int e = threadIdx.x; e < kProjTok * kProjSlice; e += kProjCols) {
    int t = e / kProjSlice, i = e % kProjSlice;
    xs[t][i] = (tok0 + t < n_tok && i < ni) ? ld_f32(x, (int64_t)(tok0 + t) * d_model + i0 + i) : 0.f;
  }
  __syncthreads();
  if (j >= r) return;
  float acc[kProjTok];
#pragma unroll
  for (int t = 0; t < kProjTok; ++t) acc[t] = 0.f;
  for (int i = 0; i < ni; ++i) {
    const float p = ld_f32(P, (int64_t)(i0 + i) * r + j);
#pragma unroll
    for (int t = 0; t < kProjTok; ++t) acc[t] = fmaf(xs[t][i], p, acc[t]);
  }
  const int64_t nt = n_tok;
#pragma unroll
  for (int t = 0; t < kProjTok; ++t)
    if (tok0 + t < n_tok) partial[((int64_t)blockIdx.z * nt + tok0 + t) * r + j] = acc[t];
}

// One wavefront per token, 4 per workgroup (block bx of the store launch).
// Phases are separated by block barriers (every wave reaches them; inactive
// waves just skip the work).  Needs 4 r floats of dynamic LDS.
template <typename T>
__device__ __forceinline__ void store_block(const T *__restrict__ x, const float *__restrict__ partial,
                                            int n_slices, int n_tok, int r,
                                            const float *__restrict__ theta, int r_R,
                                            const int32_t *__restrict__ seq_idx,
                                            const int32_t *__restrict__ pos, const CacheView &cv,
                                            int bx) {
  extern __shared__ float ys_all[];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int tok = bx * 4 + wave;
  const bool active = tok < n_tok;
  float *ys = ys_all + wave * r;
  if (active) {
    for (int j = lane; j < r; j += kWave) {
      float v;
      if (partial) {
        v = 0.f;
        for (int s = 0; s < n_slices; ++s) v += partial[((int64_t)s * n_tok + tok) * r + j];
      } else {
        v = ld_f32(x, (int64_t)tok * r + j);
      }
      ys[j] = v;
    }
  }
  __syncthreads();
  const int p = active ? pos[tok] : 0;
  if (active) {
    // Rotary map of eq. (1) on the R branch: pair (2m, 2m+1) as a complex number.
    for (int m = lane; m < r_R / 2; m += kWave) {
      const double ang = (double)p * (double)theta[m];
      double sn, cs;
      sincos(ang, &sn, &cs);
      const double a = ys[2 * m], b = ys[2 * m + 1];
      ys[2 * m] = (float)(cs * a - sn * b);
      ys[2 * m + 1] = (float)(sn * a + cs * b);
    }
  }
  __syncthreads();
  if (!active) return;
  const int blk = cv.block_table[(int64_t)seq_idx[tok] * cv.max_blocks + p / kPage];
  const int64_t row = (int64_t)blk * kPage + (p % kPage);
  if (cv.dtype == LI_FP32) {
    float *dst = (float *)cv.data + row * r;
    for (int j = lane; j < r; j += kWave) dst[j] = ys[j];
  } else if (cv.dtype == LI_BF16) {
    uint16_t *dst = (uint16_t *)cv.data + row * r;
    for (int j = lane; j < r; j += kWave) dst[j] = (uint16_t)f32_to_bf16_bits(ys[j]);
  } else {
    // one scale per token, or per scale_block values of it
    const int sbk = cv.scale_block ? cv.scale_block : r;
    const int ns = (r + sbk - 1) / sbk;
    uint8_t *dst = (uint8_t *)cv.data + row * r;
    for (int g = 0; g < ns; ++g) {
      const int j0 = g * sbk, j1 = min(r, j0 + sbk);
      float amax = 0.f;
      for (int j = j0 + lane; j < j1; j += kWave) amax = fmaxf(amax, fabsf(ys[j]));
      amax = wave_max(amax);
      // IEEE divisions (HIP keeps fp32 division correctly rounded by default).
      const float scale = amax == 0.f ? 1.f : amax / 448.f;
      const float inv = amax == 0.f ? 1.f : 448.f / amax;
      for (int j = j0 + lane; j < j1; j += kWave) dst[j] = (uint8_t)f32_to_e4m3(__fmul_rn(ys[j], inv));
      if (lane == 0) ((float *)cv.scale)[row * ns + g] = scale;
    }
  }
}

template <typename T>
__global__ void __launch_bounds__(256)
store_kernel(const T *__restrict__ x, const float *__restrict__ partial, int n_slices, int n_tok,
             int r, const float *__restrict__ theta, int r_R, const int32_t *__restrict__ seq_idx,
             const int32_t *__restrict__ pos, CacheView cv) {
  store_block<T>(x, partial, n_slices, n_tok, r, theta, r_R, seq_idx, pos, cv, blockIdx.x);
}

// The decode step's two independent preludes in one launch (each is far too
// small to fill the GPU, and a launch costs microseconds): the first n_abs
// workgroups absorb the queries (grid gx x gy x gz of the absorption, x
// fastest), the rest store the new tokens (no projection).
struct AbsorbArgs {
  const void *q;
  int n_q, H, d_I;
  const float *Dt;
  int64_t head_stride;
  const float *b;
  int nope_off, r;
  float *q_tilde, *beta;
  int gx, gy, n_abs;
};

template <bool BF16Q, typename T>
__global__ void __launch_bounds__(256)
append_absorb_kernel(const T *__restrict__ x, int n_tok, int r, const float *__restrict__ theta,
                     int r_R, const int32_t *__restrict__ seq_idx, const int32_t *__restrict__ pos,
                     CacheView cv, AbsorbArgs a) {
  const int blk = blockIdx.x;
  if (blk < a.n_abs) {  // uniform per workgroup
    absorb_block<BF16Q>(a.q, a.n_q, a.H, a.d_I, a.Dt, a.head_stride, a.b, a.nope_off, a.r,
                        a.q_tilde, a.beta, blk % a.gx, (blk / a.gx) % a.gy, blk / (a.gx * a.gy));
  } else {
    store_block<T>(x, nullptr, 0, n_tok, r, theta, r_R, seq_idx, pos, cv, blk - a.n_abs);
  }
}

}  // namespace

size_t append_ws_bytes(int n_tok, int d_model, int r, bool has_P) {
  if (!has_P) return 0;
  const size_t slices = (d_model + kProjSlice - 1) / kProjSlice;
  return slices * (size_t)n_tok * r * sizeof(float);
}

hipError_t launch_append(const void *x, int x_dt, int n_tok, int d_model, const void *P,
                         const float *theta, int r_R, const int32_t *seq_idx, const int32_t *pos,
                         const li_cache &cache, void *ws, hipStream_t st) {
  const int r = cache.r;
  const CacheView cv = view_of(cache);
  float *partial = nullptr;
  int n_slices = 0;
  if (P) {
    n_slices = (d_model + kProjSlice - 1) / kProjSlice;
    partial = (float *)ws;
    dim3 grid((r + kProjCols - 1) / kProjCols, (n_tok + kProjTok - 1) / kProjTok, n_slices);
    if (x_dt == LI_FP32)
      project_kernel<float><<<grid, kProjCols, 0, st>>>((const float *)x, (const float *)P, n_tok,
                                                        d_model, r, partial);
    else
      project_kernel<uint16_t><<<grid, kProjCols, 0, st>>>(
          (const uint16_t *)x, (const uint16_t *)P, n_tok, d_model, r, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid((n_tok + 3) / 4);
  const size_t lds = 4 * r * sizeof(float);
  if (x_dt == LI_FP32)
    store_kernel<float><<<grid, 256, lds, st>>>((const float *)x, partial, n_slices, n_tok, r,
                                                theta, r_R, seq_idx, pos, cv);
  else
    store_kernel<uint16_t><<<grid, 256, lds, st>>>((const uint16_t *)x, partial, n_slices, n_tok,
                                                   r, theta, r_R, seq_idx, pos, cv);
  return hipGetLastError();
}

hipError_t launch_append_absorb(const void *x, int x_dt, int n_tok, const float *theta, int r_R,
                                const int32_t *seq_idx, const int32_t *pos, const li_cache &cache,
                                const void *q, int q_dt, int n_layers, int n_q, int H, int d_I,
                                const float *Dt, int64_t Dt_head_stride, const float *b,
                                int nope_off, float *q_tilde, float *beta, hipStream_t st) {
  const int r = cache.r;
  const CacheView cv = view_of(cache);
  const bool per_head = Dt_head_stride != 0;
  const int n_rows = per_head ? n_q : n_q * H;
  AbsorbArgs a{q, n_q, H, d_I, Dt, Dt_head_stride, b, nope_off, r, q_tilde, beta,
               (r + 31) / 32, (n_rows + 31) / 32, 0};
  const int64_t n_abs = (int64_t)a.gx * a.gy * n_layers * (per_head ? H : 1);
  const int64_t n_store = (n_tok + 3) / 4;
  if (n_abs + n_store > (int64_t)1 << 30) return hipErrorInvalidConfiguration;
  a.n_abs = (int)n_abs;
  const dim3 grid((unsigned)(n_abs + n_store));
  const size_t lds = 4 * r * sizeof(float);
  const bool bq = q_dt == LI_BF16, bx = x_dt == LI_BF16;
  if (bq && bx)
    append_absorb_kernel<true, uint16_t><<<grid, 256, lds, st>>>(
        (const uint16_t *)x, n_tok, r, theta, r_R, seq_idx, pos, cv, a);
  else if (bq)
    append_absorb_kernel<true, float><<<grid, 256, lds, st>>>((const float *)x, n_tok, r, theta,
                                                              r_R, seq_idx, pos, cv, a);
  else if (bx)
    append_absorb_kernel<false, uint16_t><<<grid, 256, lds, st>>>(
        (const uint16_t *)x, n_tok, r, theta, r_R, seq_idx, pos, cv, a);
  else
    append_absorb_kernel<false, float><<<grid, 256, lds, st>>>((const float *)x, n_tok, r, theta,
                                                               r_R, seq_idx, pos, cv, a);
  return hipGetLastError();
}

}  // namespace li
