// li_absorb_queries: query-side decoder absorption (LatentIndex summary,
// "Methodology", eq. 6): q~_{s,h}[j] = sum_d Dt_h[j][d] q_{s,h}[d] and
// beta_{s,h} = sum_{d >= nope_off} q_{s,h}[d] b[d - nope_off].
//
// For a decoder shared by the heads this is one small GEMM,
// [n_q*H x d_I] x [d_I x r]; with per-head decoders it is one GEMM per head
// over that head's queries.  Several layers (each with its own decoder) go
// in one launch: blockIdx.z enumerates (layer, head).  Each workgroup computes a 32 x 32 output tile in
// fp32 from LDS-staged 32 x 128 slices of q and Dt (each thread 2 x 2
// outputs); a decode layer (4 x 64 heads, r = 256) spreads over 64 workgroups,
// so the call costs about one load round trip.  The work is applied once per
// new query instead of once per cached token.
#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

constexpr int kT = 32;   // tile rows and columns
constexpr int kKC = 128;  // d slice per LDS stage (d_I <= 128 takes one round trip)

// Rows of the output are "row slots": with a shared decoder, slot = s*H + h
// (all rows); with per-head decoders, blockIdx.z selects the head and
// slot = s (its queries).
template <bool BF16Q>
__device__ __forceinline__ float ldq(const void *q, int64_t off) {
  if constexpr (BF16Q) return bf16_bits_to_f32(((const uint16_t *)q)[off]);
  else return ((const float *)q)[off];
}

// Four consecutive q values as fp32 (d_I % 4 == 0, so never split by a row end).
template <bool BF16Q>
__device__ __forceinline__ float4 ldq4(const void *q, int64_t off) {
  if constexpr (BF16Q) {
    const uint2 v = *(const uint2 *)((const uint16_t *)q + off);
    return make_float4(bf16_bits_to_f32(v.x & 0xFFFFu), bf16_bits_to_f32(v.x >> 16),
                       bf16_bits_to_f32(v.y & 0xFFFFu), bf16_bits_to_f32(v.y >> 16));
  } else {
    return *(const float4 *)((const float *)q + off);
  }
}

template <bool BF16Q>
__global__ void __launch_bounds__(256)
absorb_kernel(const void *__restrict__ q, int n_q, int H, int d_I, const float *__restrict__ Dt,
              int64_t head_stride, const float *__restrict__ b, int nope_off, int r,
              float *__restrict__ q_tilde, float *__restrict__ beta) {
  // layer-major stacking of every operand
  const bool per_head = head_stride != 0;
  const int zH = per_head ? H : 1;
  const int layer = blockIdx.z / zH;
  const int64_t q_layer = (int64_t)layer * n_q * H * d_I;  // elements
  Dt += (int64_t)layer * (per_head ? (int64_t)H * head_stride : (int64_t)r * d_I);
  if (b) b += (int64_t)layer * (d_I - nope_off);
  q_tilde += (int64_t)layer * n_q * H * r;
  if (beta) beta += (int64_t)layer * n_q * H;
  __shared__ float As[kKC][kT + 4];  // As[d][row]
  __shared__ float Bs[kKC][kT + 4];  // Bs[d][j]
  constexpr int kPer4 = kT * kKC / 4 / 256;  // float4 loads of each operand per thread
  const int h_fixed = blockIdx.z % zH;
  const int n_rows = per_head ? n_q : n_q * H;
  const int row0 = blockIdx.y * kT, j0 = blockIdx.x * kT;
  const float *D = Dt + (per_head ? (int64_t)h_fixed * head_stride : 0);
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  auto qrow = [&](int slot) -> int64_t {  // element offset of q row `slot`
    return q_layer + (per_head ? ((int64_t)slot * H + h_fixed) * d_I : (int64_t)slot * d_I);
  };
  float acc[2][2] = {};
  for (int d0 = 0; d0 < d_I; d0 += kKC) {
    // Out-of-range elements load from a clamped, valid address and are
    // zeroed afterwards, so all loads issue back to back without branches.
    float4 av[kPer4], bv[kPer4];
#pragma unroll
    for (int m = 0; m < kPer4; ++m) {
      const int e = tid + 256 * m, rr = e / (kKC / 4), d = d0 + 4 * (e % (kKC / 4));
      const int slot = row0 + rr, j = j0 + rr;
      const int dc = d < d_I ? d : 0;
      av[m] = ldq4<BF16Q>(q, qrow(slot < n_rows ? slot : 0) + dc);
      bv[m] = *(const float4 *)(D + (int64_t)(j < r ? j : 0) * d_I + dc);
      if (!(d < d_I && slot < n_rows)) av[m] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (!(d < d_I && j < r)) bv[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int m = 0; m < kPer4; ++m) {
      const int e = tid + 256 * m, rr = e / (kKC / 4), dd = 4 * (e % (kKC / 4));
      As[dd][rr] = av[m].x;
      As[dd + 1][rr] = av[m].y;
      As[dd + 2][rr] = av[m].z;
      As[dd + 3][rr] = av[m].w;
      Bs[dd][rr] = bv[m].x;
      Bs[dd + 1][rr] = bv[m].y;
      Bs[dd + 2][rr] = bv[m].z;
      Bs[dd + 3][rr] = bv[m].w;
    }
    __syncthreads();
    const int nd = min(kKC, d_I - d0);
#pragma unroll 16
    for (int dd = 0; dd < nd; ++dd) {
      float a[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = As[dd][ty * 2 + i];
#pragma unroll
      for (int c = 0; c < 2; ++c) bb[c] = Bs[dd][tx + 16 * c];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[i][c] = fmaf(a[i], bb[c], acc[i][c]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int slot = row0 + ty * 2 + i;
    if (slot >= n_rows) continue;
    const int64_t orow = per_head ? ((int64_t)slot * H + h_fixed) : slot;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int j = j0 + tx + 16 * c;
      if (j < r) q_tilde[orow * r + j] = acc[i][c];
    }
  }
  // beta for this tile's rows, computed once (by the column-0 tiles): eight
  // threads per row, a fixed-order combination of their partial sums.
  if (beta && blockIdx.x == 0) {
    const int rr = tid / 8, part = tid % 8;
    const int slot = row0 + rr;
    float s = 0.f;
    if (b && slot < n_rows) {
      const int64_t off = qrow(slot);
      for (int d = nope_off + part; d < d_I; d += 8) s = fmaf(ldq<BF16Q>(q, off + d), b[d - nope_off], s);
    }
    s += __shfl_xor(s, 1, kWave);
    s += __shfl_xor(s, 2, kWave);
    s += __shfl_xor(s, 4, kWave);
    if (part == 0 && slot < n_rows) beta[per_head ? ((int64_t)slot * H + h_fixed) : slot] = s;
  }
}

}  // namespace

hipError_t launch_absorb(const void *q, int q_dt, int n_layers, int n_q, int H, int d_I, const float *Dt,
                         int64_t Dt_head_stride, const float *b, int nope_off, int r,
                         float *q_tilde, float *beta, hipStream_t st) {
  const bool per_head = Dt_head_stride != 0;
  const int n_rows = per_head ? n_q : n_q * H;
  dim3 grid((r + kT - 1) / kT, (n_rows + kT - 1) / kT, n_layers * (per_head ? H : 1));
  if (q_dt == LI_BF16)
    absorb_kernel<true><<<grid, 256, 0, st>>>(q, n_q, H, d_I, Dt, Dt_head_stride, b, nope_off, r,
                                              q_tilde, beta);
  else
    absorb_kernel<false><<<grid, 256, 0, st>>>(q, n_q, H, d_I, Dt, Dt_head_stride, b, nope_off, r,
                                               q_tilde, beta);
  return hipGetLastError();
}

}  // namespace li
