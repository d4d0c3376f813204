// li_absorb_queries: query-side decoder absorption (LatentIndex summary,
// "Methodology", eq. 6): q~_{s,h}[j] = sum_d Dt_h[j][d] q_{s,h}[d] and
// beta_{s,h} = sum_{d >= nope_off} q_{s,h}[d] b[d - nope_off].
//
// For a decoder shared by the heads this is one small GEMM,
// [n_q*H x d_I] x [d_I x r]; with per-head decoders it is one GEMM per head
// over that head's queries.  Several layers (each with its own decoder) go
// in one launch: blockIdx.z enumerates (layer, head).  Both operands are
// contiguous along d, and the GEMM runs on the fp32 matrix cores
// (v_mfma_f32_16x16x4f32): a workgroup computes a 32 x 32 output block, one
// wavefront per 16 x 16 tile, from its 32 query rows and 32 decoder rows of
// each 128-wide slice of d, staged in LDS once (each row feeds two
// wavefronts).  The instruction takes, for each of its 4 k slots g, A[i][g]
// from lane i + 16 g and B[g][j] from lane j + 16 g; slot g is given the
// contiguous quarter d in [32 g, 32 g + 32) of the slice, so every lane reads
// its own row of q and of Dt in 16-byte pieces, and step t of the chain pairs
// d = 32 g + t across the slots.  The work is applied once per new query
// instead of once per cached token.
#include "absorb_block.h"
#include "li_device.h"
#include "li_internal.h"

namespace li {
namespace {

template <bool BF16Q>
__global__ void __launch_bounds__(256)
absorb_kernel(const void *__restrict__ q, int n_q, int H, int d_I, const float *__restrict__ Dt,
              int64_t head_stride, const float *__restrict__ b, int nope_off, int r,
              float *__restrict__ q_tilde, float *__restrict__ beta) {
  absorb_block<BF16Q>(q, n_q, H, d_I, Dt, head_stride, b, nope_off, r, q_tilde, beta, blockIdx.x,
                      blockIdx.y, blockIdx.z);
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
