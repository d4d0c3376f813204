// Device-side helpers shared by the LatentIndex kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace li {

constexpr int kWave = 64;
constexpr int kPage = 64;  // tokens per cache block

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round a finite fp32 to bf16, nearest, ties to even.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// OCP E4M3FN code -> fp32 (exact).  0x7F/0xFF (NaN) never occur in a cache
// written by the quantiser.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -v : v;
}

// fp32 -> OCP E4M3FN, round to nearest even, saturating at +-448.  The sign
// bit follows the input (so -0.0 and tiny negatives give 0x80).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __uint_as_float(u & 0x7FFFFFFFu);
  if (!(a < 448.0f)) return sign | 0x7Eu;
  if (a < 0.015625f) {  // below 2^-6: subnormal codes m * 2^-9, m = 0..8 (8 = 2^-6)
    return sign | (uint32_t)rintf(a * 512.0f);
  }
  const uint32_t ua = __float_as_uint(a);
  uint32_t e = (ua >> 23) - 120u;  // biased e4m3 exponent, 1..15
  uint32_t keep = (ua >> 20) & 7u;
  const uint32_t rest = ua & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) { keep = 0; ++e; }
  return sign | (e << 3) | keep;
}

// Order-preserving map fp32 -> uint32 (larger float => larger key); -0.0 is
// mapped like +0.0 so the two tie.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Workgroup barrier for LDS data only: waits for this wave's LDS operations,
// not for its outstanding global loads and stores (which __syncthreads()'s
// fence would also drain).
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct HBM -> LDS load of 16 bytes per lane: lane i's 16 bytes at `g` land
// at lds + 16 i (the LDS address is taken from the first active lane).
// Written as inline assembly on purpose: the compiler then does not track the
// load, so it adds none of its own waits for it (with the builtin form it
// drains every load in flight before any LDS read that might alias the
// target, which serialises a multi-stage pipeline).  The caller owns all
// synchronisation: s_waitcnt vmcnt(n) for the data, then a barrier before
// other wavefronts read it, and no overwrite before all reads of the old
// contents are done.  The s_nop is the one wait state required between the
// M0 write (made by the compiler for the "{m0}" operand) and the load.
__device__ __forceinline__ void dma16_to_lds(const void *g,
                                             __attribute__((address_space(3))) void *lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m0) : "memory");
}

// As dma16_to_lds for 4 bytes per lane (lane i's dword lands at lds + 4 i).
__device__ __forceinline__ void dma4_to_lds(const void *g,
                                            __attribute__((address_space(3))) void *lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(m0) : "memory");
}

// Inclusive prefix sum across a wavefront with DPP moves (row shifts within
// 16-lane rows, then row broadcasts 15 and 31 across rows).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return (uint32_t)x;
}

// Load a latent row element range as fp32 (generic paths).
__device__ __forceinline__ float load_latent(const void *data, int dtype, int64_t off) {
  if (dtype == 0) return ((const float *)data)[off];
  if (dtype == 1) return bf16_bits_to_f32(((const uint16_t *)data)[off]);
  return e4m3_to_f32(((const uint8_t *)data)[off]);
}

}  // namespace li
