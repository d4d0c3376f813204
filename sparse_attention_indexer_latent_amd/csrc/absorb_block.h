// Query absorption, one workgroup's share: the device code of absorb_kernel,
// shared with the launch that also appends new tokens (append.hip).  The
// contraction and its layout are described in absorb.hip.
#pragma once

#include "li_device.h"

namespace li {
namespace {

constexpr int kT = 32;    // output block rows and columns per workgroup
constexpr int kKC = 128;  // d per slice: 32 per k slot

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
  const int slot = by * kT + 16 * ti + i, j = bx * kT + 16 * tj + i;
  const bool a_ok = slot < n_rows, b_ok = j < r;
  // out-of-range rows read a valid row and are zeroed, so loads need no branches
  const int64_t qo = qrow(a_ok ? slot : 0);
  const float *dr = D + (int64_t)(b_ok ? j : 0) * d_I;
  // four independent accumulation chains (one per float4 lane), summed in a
  // fixed order at the end, so consecutive matrix-core ops do not wait on
  // each other
  f32x4 acc4[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f},
                   {0.f, 0.f, 0.f, 0.f}};
  for (int d0 = 0; d0 < d_I; d0 += kKC) {
    float4 av[8], bv[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int d = d0 + 32 * g + 4 * c;
      const int dc = d < d_I ? d : 0;
      av[c] = ldq4<BF16Q>(q, qo + dc);
      bv[c] = *(const float4 *)(dr + dc);
      if (!(a_ok && d < d_I)) av[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (!(b_ok && d < d_I)) bv[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      acc4[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[c].x, bv[c].x, acc4[0], 0, 0, 0);
      acc4[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[c].y, bv[c].y, acc4[1], 0, 0, 0);
      acc4[2] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[c].z, bv[c].z, acc4[2], 0, 0, 0);
      acc4[3] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[c].w, bv[c].w, acc4[3], 0, 0, 0);
    }
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
  // beta for this block's rows, computed once (by the column-0 blocks): eight
  // threads per row, a fixed-order combination of their partial sums.
  if (beta && bx == 0) {
    const int rr = tid / 8, part = tid % 8;
    const int sl = by * kT + rr;
    float s = 0.f;
    if (b && sl < n_rows) {
      const int64_t off = qrow(sl);
      for (int d = nope_off + part; d < d_I; d += 8) s = fmaf(ldq<BF16Q>(q, off + d), b[d - nope_off], s);
    }
    s += __shfl_xor(s, 1, kWave);
    s += __shfl_xor(s, 2, kWave);
    s += __shfl_xor(s, 4, kWave);
    if (part == 0 && sl < n_rows) beta[per_head ? ((int64_t)sl * H + h_fixed) : sl] = s;
  }
}

}  // namespace
}  // namespace li
