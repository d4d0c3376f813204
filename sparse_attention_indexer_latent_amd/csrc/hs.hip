// Hierarchical selection helpers (LatentIndex summary, "Methodology",
// "Hierarchical Selection"): the follower rescores only the anchor's
// candidate set.  The candidate list of a query is ascending token ids padded
// at the end with -1; its valid count bounds the rescore and the selection.
#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

// One workgroup per query: count the non-negative entries and write -inf to
// the score slots of the padding.
__global__ void __launch_bounds__(256)
count_valid_kernel(const int32_t *__restrict__ cand, int B, int32_t *__restrict__ counts,
                   float *__restrict__ cand_scores) {
  __shared__ int32_t part[4];
  const int q = blockIdx.x, tid = threadIdx.x;
  const int32_t *c = cand + (int64_t)q * B;
  int n = 0;
  for (int j = tid; j < B; j += 256) n += c[j] >= 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o, kWave);
  if (tid % kWave == 0) part[tid / kWave] = n;
  __syncthreads();
  const int total = part[0] + part[1] + part[2] + part[3];
  if (tid == 0) counts[q] = total;
  for (int j = total + tid; j < B; j += 256) cand_scores[(int64_t)q * B + j] = -INFINITY;
}

}  // namespace

hipError_t launch_count_valid(const int32_t *cand, int n_q, int B, int32_t *counts,
                              float *cand_scores, hipStream_t st) {
  count_valid_kernel<<<n_q, 256, 0, st>>>(cand, B, counts, cand_scores);
  return hipGetLastError();
}

}  // namespace li
