// li_absorb_queries: query-side decoder absorption (LatentIndex summary,
// "Methodology", eq. 6): q~_{s,h}[j] = sum_d Dt[j][d] q_{s,h}[d] and
// beta_{s,h} = sum_{d >= nope_off} q_{s,h}[d] b[d - nope_off].
//
// One workgroup per (query, head); q_{s,h} is staged in LDS and each
// wavefront produces whole output rows j, its lanes striding over d so that
// the row Dt[j][:] is read contiguously, then reducing across the wavefront.
// The work is tiny (n_q * H * r * d_I MACs) and applied once per new query
// instead of once per cached token.
#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

__global__ void __launch_bounds__(256)
absorb_kernel(const void *__restrict__ q, int q_dt, int H, int d_I, const float *__restrict__ Dt,
              int64_t head_stride, const float *__restrict__ b, int nope_off, int r,
              float *__restrict__ q_tilde, float *__restrict__ beta) {
  __shared__ float qs[1024];
  const int h = blockIdx.x, s = blockIdx.y;
  const int64_t qoff = ((int64_t)s * H + h) * d_I;
  for (int d = threadIdx.x; d < d_I; d += blockDim.x)
    qs[d] = q_dt == LI_FP32 ? ((const float *)q)[qoff + d]
                            : bf16_bits_to_f32(((const uint16_t *)q)[qoff + d]);
  __syncthreads();
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int n_waves = blockDim.x / kWave;
  const float *D = Dt + (int64_t)h * head_stride;
  float *out = q_tilde + ((int64_t)s * H + h) * r;
  for (int j = wave; j < r; j += n_waves) {
    const float *row = D + (int64_t)j * d_I;
    float acc = 0.f;
    for (int d = lane; d < d_I; d += kWave) acc = fmaf(row[d], qs[d], acc);
    acc = wave_sum(acc);
    if (lane == 0) out[j] = acc;
  }
  if (beta && wave == 0) {
    float acc = 0.f;
    if (b)
      for (int d = nope_off + lane; d < d_I; d += kWave) acc = fmaf(qs[d], b[d - nope_off], acc);
    acc = wave_sum(acc);
    if (lane == 0) beta[(int64_t)s * H + h] = acc;
  }
}

}  // namespace

hipError_t launch_absorb(const void *q, int q_dt, int n_q, int H, int d_I, const float *Dt,
                         int64_t Dt_head_stride, const float *b, int nope_off, int r,
                         float *q_tilde, float *beta, hipStream_t st) {
  dim3 grid(H, n_q);
  absorb_kernel<<<grid, 256, 0, st>>>(q, q_dt, H, d_I, Dt, Dt_head_stride, b, nope_off, r,
                                      q_tilde, beta);
  return hipGetLastError();
}

}  // namespace li
