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
// sums).  A workgroup of four wavefronts owns one 128 x 128 block of C (no
// split over k, so the sums are deterministic and the block is
// read-modified-written without atomics); each wavefront accumulates a
// 64 x 64 quarter as 4 x 4 tiles.  16-row slabs of both operands are loaded
// with 16-byte vector loads, widened to fp32 and stored into one of two LDS
// stages while the matrix cores work on the other (one barrier per slab).
// LDS rows are padded to 144 floats, so the 16-lane groups of a wavefront
// that read four consecutive slab rows hit disjoint banks.
#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

constexpr int kBT = 128;        // block of C per workgroup
constexpr int kKS = 16;         // rows per staged slab
constexpr int kRow = kBT + 16;  // padded LDS row (floats)

template <bool BF>
__device__ __forceinline__ float ld1(const void *p, int64_t off) {
  if constexpr (BF) return bf16_bits_to_f32(((const uint16_t *)p)[off]);
  else return ((const float *)p)[off];
}

// One thread's share of a slab of one operand: 8 consecutive columns of one
// row (bf16: one 16-byte load; fp32: two).
template <bool BF>
struct SlabPart {
  float v[8];
};

template <bool BF>
__device__ __forceinline__ void load_part(SlabPart<BF> &o, const void *P, int64_t n, int dp, int64_t k,
                                          int c0, bool vec) {
  const bool rowok = k < n;
  if (vec && rowok && c0 + 8 <= dp) {
    if constexpr (BF) {
      const uint4 x = *reinterpret_cast<const uint4 *>((const uint16_t *)P + k * dp + c0);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o.v[2 * e] = __uint_as_float(w[e] << 16);
        o.v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    } else {
      const float4 a = *reinterpret_cast<const float4 *>((const float *)P + k * dp + c0);
      const float4 b = *reinterpret_cast<const float4 *>((const float *)P + k * dp + c0 + 4);
      o.v[0] = a.x; o.v[1] = a.y; o.v[2] = a.z; o.v[3] = a.w;
      o.v[4] = b.x; o.v[5] = b.y; o.v[6] = b.z; o.v[7] = b.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = c0 + e;
      float x = 0.f;
      if (rowok && c < dp) {
        if constexpr (BF) x = bf16_bits_to_f32(((const uint16_t *)P)[k * dp + c]);
        else x = ((const float *)P)[k * dp + c];
      }
      o.v[e] = x;
    }
  }
}

template <bool BF>
__device__ __forceinline__ void store_part(float *row, const SlabPart<BF> &o) {
  *reinterpret_cast<float4 *>(row) = make_float4(o.v[0], o.v[1], o.v[2], o.v[3]);
  *reinterpret_cast<float4 *>(row + 4) = make_float4(o.v[4], o.v[5], o.v[6], o.v[7]);
}

// SYM (A == B, C = A^T A): only blocks on or above the diagonal run; an
// off-diagonal block also writes its transpose, so every element of C is
// still owned by exactly one workgroup.
//
// csum (may be null): column sums of B's columns j0 .. j0 + 127, taken from
// the staged slabs by the workgroups of the first block row (for SYM, the
// diagonal blocks), each thread over the rows it stages, then combined in a
// fixed order (deterministic).
template <bool ABF, bool BBF, bool SYM>
__global__ void __launch_bounds__(256)
gram_kernel(const void *__restrict__ A, int64_t n, int da, const void *__restrict__ B, int db,
            float *C, int64_t ldc, float *__restrict__ csum, int accumulate) {
  __shared__ __align__(16) float As[2][kKS][kRow];
  __shared__ __align__(16) float Bs[2][kKS][kRow];
  if (SYM && blockIdx.y > blockIdx.x) return;  // uniform
  const bool sums = csum && (SYM ? blockIdx.x == blockIdx.y : blockIdx.y == 0);  // uniform
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int i0 = blockIdx.y * kBT, j0 = blockIdx.x * kBT;
  const int wi = wave >> 1, wj = wave & 1;
  const int li = lane % 16, g = lane / 16;
  // 16-byte loads need 16-byte aligned rows
  const bool avec = ((uintptr_t)A % 16 == 0) && (da % (ABF ? 8 : 4) == 0);
  const bool bvec = ((uintptr_t)B % 16 == 0) && (db % (BBF ? 8 : 4) == 0);
  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  // staging: thread t covers slab row t / 16, columns 8 (t % 16) .. +7
  const int sr = tid / 16, sc = (tid % 16) * 8;
  const int64_t nslab = (n + kKS - 1) / kKS;
  SlabPart<ABF> pa;
  SlabPart<BBF> pb;
  float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  load_part<ABF>(pa, A, n, da, sr, i0 + sc, avec);
  load_part<BBF>(pb, B, n, db, sr, j0 + sc, bvec);
  store_part<ABF>(&As[0][sr][sc], pa);
  store_part<BBF>(&Bs[0][sr][sc], pb);
  if (sums) {
#pragma unroll
    for (int e = 0; e < 8; ++e) cs[e] += pb.v[e];
  }
  __syncthreads();
  for (int64_t s = 0; s < nslab; ++s) {
    const int cur = (int)(s & 1);
    const bool more = s + 1 < nslab;
    if (more) {  // the next slab's loads fly while this one is multiplied
      load_part<ABF>(pa, A, n, da, (s + 1) * kKS + sr, i0 + sc, avec);
      load_part<BBF>(pb, B, n, db, (s + 1) * kKS + sr, j0 + sc, bvec);
    }
#pragma unroll
    for (int kk = 0; kk < kKS; kk += 4) {
      float av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = As[cur][kk + g][64 * wi + 16 * a + li];
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = Bs[cur][kk + g][64 * wj + 16 * b + li];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          // acc[a][b][v] += A-column (row 4 g + v of the tile) . B-column li
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    if (more) {
      store_part<ABF>(&As[cur ^ 1][sr][sc], pa);
      store_part<BBF>(&Bs[cur ^ 1][sr][sc], pb);
      if (sums) {
#pragma unroll
        for (int e = 0; e < 8; ++e) cs[e] += pb.v[e];
      }
    }
    __syncthreads();
  }
  if (sums) {  // the 16 row groups' partial sums, combined in row-group order
    float *part = &As[0][0][0];  // [16][kRow], free after the last barrier
#pragma unroll
    for (int e = 0; e < 8; ++e) part[sr * kRow + sc + e] = cs[e];
    __syncthreads();
    if (tid < kBT && j0 + tid < db) {
      float t = 0.f;
#pragma unroll
      for (int r = 0; r < kKS; ++r) t += part[r * kRow + tid];
      csum[j0 + tid] = (accumulate ? csum[j0 + tid] : 0.f) + t;
    }
  }
  if (!C) return;  // column sums only
  // acc[a][b][v] = C[i0 + 64 wi + 16 a + 4 g + v][j0 + 64 wj + 16 b + li]
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = i0 + 64 * wi + 16 * a + 4 * g + v, j = j0 + 64 * wj + 16 * b + li;
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

template <bool ABF, bool BBF, bool SYM = false>
hipError_t gram(const void *A, int64_t n, int da, const void *B, int db, float *C, float *csum,
                int accumulate, hipStream_t st) {
  dim3 grid((db + kBT - 1) / kBT, (da + kBT - 1) / kBT);
  gram_kernel<ABF, BBF, SYM><<<grid, 256, 0, st>>>(A, n, da, B, db, C, db, csum, accumulate);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_calib_gram(const void *X, int x_bf16, int64_t n, int d, const void *Y,
                             int y_bf16, int e, float *G_xx, float *G_xy, float *x_sum,
                             float *y_sum, int accumulate, hipStream_t st) {
  hipError_t err = x_bf16 ? gram<true, true, true>(X, n, d, X, d, G_xx, x_sum, accumulate, st)
                          : gram<false, false, true>(X, n, d, X, d, G_xx, x_sum, accumulate, st);
  if (err != hipSuccess || !Y || (!G_xy && !y_sum)) return err;
  if (x_bf16)
    return y_bf16 ? gram<true, true>(X, n, d, Y, e, G_xy, y_sum, accumulate, st)
                  : gram<true, false>(X, n, d, Y, e, G_xy, y_sum, accumulate, st);
  return y_bf16 ? gram<false, true>(X, n, d, Y, e, G_xy, y_sum, accumulate, st)
                : gram<false, false>(X, n, d, Y, e, G_xy, y_sum, accumulate, st);
}

}  // namespace li
