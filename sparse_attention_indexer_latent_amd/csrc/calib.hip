// Normal equations of the training-free calibration (LatentIndex summary,
// "Methodology", Training-free Calibration): the ridge reduced-rank
// regression that fits the group's shared projection and the layers'
// decoders needs, over all calibration tokens, the Gram matrix X^T X of the
// anchor hidden states, their cross-products X^T Y with the layers' indexer
// keys, and the column sums of both (for centring).  These are the O(n d^2)
// part of the fit; everything after them is a small dense solve.
//
// C[i, j] (+)= sum_k A[k, i] B[k, j] for row-major A [n, da], B [n, db] on
// the fp32 matrix cores (v_mfma_f32_16x16x4f32, exact fp32 products, fp32
// sums).  A workgroup owns one 64 x 64 block of C (no split over k, so the
// sums are deterministic and the block is read-modified-written without
// atomics); 32-row slabs of both operands are staged through LDS with
// coalesced loads and each of the four wavefronts accumulates a 32 x 32
// quarter as 2 x 2 tiles.
#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

constexpr int kBT = 64;   // block of C per workgroup
constexpr int kKS = 32;   // rows per staged slab
constexpr int kPadC = 4;  // LDS row padding (floats)

template <bool BF>
__device__ __forceinline__ float ld1(const void *p, int64_t off) {
  if constexpr (BF) return bf16_bits_to_f32(((const uint16_t *)p)[off]);
  else return ((const float *)p)[off];
}

// SYM (A == B, C = A^T A): only blocks on or above the diagonal run; an
// off-diagonal block also writes its transpose, so every element of C is
// still owned by exactly one workgroup.
template <bool ABF, bool BBF, bool SYM>
__global__ void __launch_bounds__(256)
gram_kernel(const void *__restrict__ A, int64_t n, int da, const void *__restrict__ B, int db,
            float *__restrict__ C, int64_t ldc, int accumulate) {
  __shared__ float As[kKS][kBT + kPadC];
  __shared__ float Bs[kKS][kBT + kPadC];
  if (SYM && blockIdx.y > blockIdx.x) return;  // uniform
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int i0 = blockIdx.y * kBT, j0 = blockIdx.x * kBT;
  const int wi = wave >> 1, wj = wave & 1;
  const int li = lane % 16, g = lane / 16;
  f32x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // staging: thread t covers row t / 8 of the slab, columns 8 (t % 8) .. +7
  const int sr = tid / 8, sc = (tid % 8) * 8;
  for (int64_t k0 = 0; k0 < n; k0 += kKS) {
    const int64_t k = k0 + sr;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int ca = i0 + sc + c, cb = j0 + sc + c;
      As[sr][sc + c] = (k < n && ca < da) ? ld1<ABF>(A, k * da + ca) : 0.f;
      Bs[sr][sc + c] = (k < n && cb < db) ? ld1<BBF>(B, k * db + cb) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kKS; kk += 4) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const float av = As[kk + g][32 * wi + 16 * a + li];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const float bv = Bs[kk + g][32 * wj + 16 * b + li];
          // acc[a][b][v] += A-column (row 4 g + v of the tile) . B-column li
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[a][b], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  // acc[a][b][v] = C[i0 + 32 wi + 16 a + 4 g + v][j0 + 32 wj + 16 b + li]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = i0 + 32 * wi + 16 * a + 4 * g + v, j = j0 + 32 * wj + 16 * b + li;
        if (i < da && j < db) {
          float *o = C + (int64_t)i * ldc + j;
          *o = (accumulate ? *o : 0.f) + acc[a][b][v];
          if (SYM && i0 != j0) {  // the mirrored element, below the diagonal
            float *t = C + (int64_t)j * ldc + i;
            *t = (accumulate ? *t : 0.f) + acc[a][b][v];
          }
        }
      }
}

template <bool BF>
__global__ void __launch_bounds__(256)
colsum_kernel(const void *__restrict__ A, int64_t n, int da, float *__restrict__ s, int accumulate) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= da) return;
  float acc = 0.f;
  for (int64_t k = 0; k < n; ++k) acc += ld1<BF>(A, k * da + j);
  s[j] = (accumulate ? s[j] : 0.f) + acc;
}

template <bool ABF, bool BBF, bool SYM = false>
hipError_t gram(const void *A, int64_t n, int da, const void *B, int db, float *C, int accumulate,
                hipStream_t st) {
  dim3 grid((db + kBT - 1) / kBT, (da + kBT - 1) / kBT);
  gram_kernel<ABF, BBF, SYM><<<grid, 256, 0, st>>>(A, n, da, B, db, C, db, accumulate);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_calib_gram(const void *X, int x_bf16, int64_t n, int d, const void *Y,
                             int y_bf16, int e, float *G_xx, float *G_xy, float *x_sum,
                             float *y_sum, int accumulate, hipStream_t st) {
  hipError_t err = x_bf16 ? gram<true, true, true>(X, n, d, X, d, G_xx, accumulate, st)
                          : gram<false, false, true>(X, n, d, X, d, G_xx, accumulate, st);
  if (err != hipSuccess) return err;
  if (Y && G_xy) {
    if (x_bf16)
      err = y_bf16 ? gram<true, true>(X, n, d, Y, e, G_xy, accumulate, st)
                   : gram<true, false>(X, n, d, Y, e, G_xy, accumulate, st);
    else
      err = y_bf16 ? gram<false, true>(X, n, d, Y, e, G_xy, accumulate, st)
                   : gram<false, false>(X, n, d, Y, e, G_xy, accumulate, st);
    if (err != hipSuccess) return err;
  }
  if (x_sum) {
    if (x_bf16) colsum_kernel<true><<<(d + 255) / 256, 256, 0, st>>>(X, n, d, x_sum, accumulate);
    else colsum_kernel<false><<<(d + 255) / 256, 256, 0, st>>>(X, n, d, x_sum, accumulate);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (Y && y_sum) {
    if (y_bf16) colsum_kernel<true><<<(e + 255) / 256, 256, 0, st>>>(Y, n, e, y_sum, accumulate);
    else colsum_kernel<false><<<(e + 255) / 256, 256, 0, st>>>(Y, n, e, y_sum, accumulate);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace li
