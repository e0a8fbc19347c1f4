// GEMM epilogues shared by the bf16 MFMA GEMM and the fp32 debug GEMM:
// one output element (row, col, fp32 accumulator) at a time.
#pragma once
#include "common.h"
#include "kernels.h"

namespace stb {

// Store of the head-split layouts: Q and K as [B*heads][npad][64] rows,
// V as its transpose [B*heads][64][npad] so that the attention kernel reads
// keys contiguously for both of its products.
template <typename TA>
__device__ __forceinline__ void store_heads(const HeadSplit& hs, int row,
                                            int col, float v) {
  const int which = col / hs.C;
  const int s = which % hs.nsplit;
  const int layer = which / hs.nsplit;
  const int within = col - which * hs.C;
  const int head = within >> 6;
  const int dim = within & 63;
  const int b = row / hs.rows_per_batch;
  const int n = row - b * hs.rows_per_batch;
  const long long bh = static_cast<long long>(b) * hs.heads + head;
  TA* base = static_cast<TA*>(hs.dst[s]) + layer * hs.layer_stride;
  long long idx;
  if ((hs.transposed_mask >> s) & 1)
    idx = (bh * kHeadDim + dim) * hs.npad + n;
  else
    idx = (bh * hs.npad + n) * kHeadDim + dim;
  base[idx] = from_f32<TA>(v * hs.scale[s]);
}

template <int EPI, typename TA>
__device__ __forceinline__ void epi_store(const EpiParams& e, int row, int col,
                                          float acc) {
  if constexpr (EPI == EPI_STORE_F32) {
    e.out_f32[static_cast<long long>(row) * e.ldo + col] =
        acc + (e.bias ? e.bias[col] : 0.f);
  } else if constexpr (EPI == EPI_RESID_F32) {
    float* p = e.out_f32 + static_cast<long long>(row) * e.ldo + col;
    *p = *p + (acc + (e.bias ? e.bias[col] : 0.f));
  } else if constexpr (EPI == EPI_HEADS) {
    store_heads<TA>(e.hs, row, col, acc + (e.bias ? e.bias[col] : 0.f));
  } else if constexpr (EPI == EPI_NCHW) {
    // row = channel c, col = token t = b*ntok + n;  y[b][c][n]
    const int b = col / e.ntok;
    const int n = col - b * e.ntok;
    const int Cc = e.ldo;  // channels
    const long long idx = (static_cast<long long>(b) * Cc + row) * e.ntok + n;
    const float xv = to_f32<TA>(static_cast<const TA*>(e.resid_act)[idx]);
    static_cast<TA*>(e.out_act)[idx] =
        from_f32<TA>(acc + (e.bias ? e.bias[row] : 0.f) + xv);
  }
}

}  // namespace stb
