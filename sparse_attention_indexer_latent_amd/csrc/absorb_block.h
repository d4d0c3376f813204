// Query absorption, one workgroup's share: the device code of absorb_kernel,
// shared with the launch that also appends new tokens (append.hip).  The
// contraction and its layout are described in absorb.hip.
#pragma once

#include "li_device.h"

namespace li {
namespace {

constexpr int kT = 32;    // output block rows and columns per workgroup
constexpr int kKC = 128;  // d per slice: 32 per k slot
static_assert(kT * kKC % (4 * 256) == 0, "a chunk's tiles stage in whole float4s per thread");

// Rows of the output are "row slots": with a shared decoder, slot = s*H + h
// (all rows); with per-head decoders, bz selects the head and
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

// One workgroup's share (block (bx, by, bz) of the grid launch_absorb uses).
template <bool BF16Q>
__device__ __forceinline__ void absorb_block(const void *__restrict__ q, int n_q, int H, int d_I,
                                             const float *__restrict__ Dt, int64_t head_stride,
                                             const float *__restrict__ b, int nope_off, int r,
                                             float *__restrict__ q_tilde, float *__restrict__ beta,
                                             int bx, int by, int bz) {
  // layer-major stacking of every operand
  const bool per_head = head_stride != 0;
  const int zH = per_head ? H : 1;
  const int layer = bz / zH;
  const int64_t q_layer = (int64_t)layer * n_q * H * d_I;  // elements
  Dt += (int64_t)layer * (per_head ? (int64_t)H * head_stride : (int64_t)r * d_I);
  if (b) b += (int64_t)layer * (d_I - nope_off);
  q_tilde += (int64_t)layer * n_q * H * r;
  if (beta) beta += (int64_t)layer * n_q * H;
  const int h_fixed = bz % zH;
  const int n_rows = per_head ? n_q : n_q * H;
  const float *D = Dt + (per_head ? (int64_t)h_fixed * head_stride : 0);
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  auto qrow = [&](int slot) -> int64_t {  // element offset of q row `slot`
    return q_layer + (per_head ? ((int64_t)slot * H + h_fixed) * d_I : (int64_t)slot * d_I);
  };
  // this wavefront's 16 x 16 tile; lane supplies row i of A and of B, slot g
  const int ti = wave >> 1, tj = wave & 1;
  const int i = lane % 16, g = lane / 16;
  // The workgroup's 32 query rows and 32 decoder rows of each d-chunk are
  // staged in LDS once (each row serves two wavefronts); rows and dims out of
  // range are staged as zeros.
  __shared__ __align__(16) float qs[kT][kKC + 4];
  __shared__ __align__(16) float ds[kT][kKC + 4];
  // four independent accumulation chains (one per float4 lane), summed in a
  // fixed order at the end, so consecutive matrix-core ops do not wait on
  // each other
  f32x4 acc4[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f},
                   {0.f, 0.f, 0.f, 0.f}};
  // beta for this block's rows, computed once (by the column-0 blocks): eight
  // threads per row, each a chain over its dims in ascending order (from the
  // staged rows), then a fixed-order combination of the eight partial sums.
  const bool want_beta = beta && bx == 0;  // uniform
  const int rr = tid / 8, part = tid % 8;
  const int sl = by * kT + rr;
  float bs = 0.f;
  for (int d0 = 0; d0 < d_I; d0 += kKC) {
#pragma unroll
    for (int k4 = 0; k4 < kT * kKC / 4 / 256; ++k4) {
      const int e = (int)threadIdx.x + 256 * k4;
      const int row = e / (kKC / 4), c4 = e % (kKC / 4);
      const int d = d0 + 4 * c4;
      const int qslot = by * kT + row, jrow = bx * kT + row;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
      if (qslot < n_rows && d < d_I) x = ldq4<BF16Q>(q, qrow(qslot) + d);
      if (jrow < r && d < d_I) y = *(const float4 *)(D + (int64_t)jrow * d_I + d);
      *reinterpret_cast<float4 *>(&qs[row][4 * c4]) = x;
      *reinterpret_cast<float4 *>(&ds[row][4 * c4]) = y;
    }
    __syncthreads();
    float4 av[8], bv[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      av[c] = *reinterpret_cast<const float4 *>(&qs[16 * ti + i][32 * g + 4 * c]);
      bv[c] = *reinterpret_cast<const float4 *>(&ds[16 * tj + i][32 * g + 4 * c]);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      acc4[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[c].x, bv[c].x, acc4[0], 0, 0, 0);
      acc4[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[c].y, bv[c].y, acc4[1], 0, 0, 0);
      acc4[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[c].z, bv[c].z, acc4[2], 0, 0, 0);
      acc4[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[c].w, bv[c].w, acc4[3], 0, 0, 0);
    }
    if (want_beta && b && sl < n_rows) {
      // this thread's dims d = nope_off + part (mod 8), d >= nope_off, in the chunk
      int d = nope_off + part;
      if (d < d0) d += ((d0 - d + 7) / 8) * 8;
      for (; d < min(d_I, d0 + kKC); d += 8) bs = fmaf(qs[rr][d - d0], b[d - nope_off], bs);
    }
    __syncthreads();  // the next chunk reuses the tiles
  }
  const f32x4 acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
  // acc[v] = D[4 g + v][i] of the tile
  const int jo = bx * kT + 16 * tj + i;
  if (jo < r) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int so = by * kT + 16 * ti + 4 * g + v;
      if (so >= n_rows) continue;
      const int64_t orow = per_head ? ((int64_t)so * H + h_fixed) : so;
      q_tilde[orow * r + jo] = acc[v];
    }
  }
  if (want_beta) {
    float s = bs;
    s += __shfl_xor(s, 1, kWave);
    s += __shfl_xor(s, 2, kWave);
    s += __shfl_xor(s, 4, kWave);
    if (part == 0 && sl < n_rows) beta[per_head ? ((int64_t)sl * H + h_fixed) : sl] = s;
  }
}

}  // namespace
}  // namespace li
