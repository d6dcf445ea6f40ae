// Context fusion, many-row path (Strata PR #1426 page, "Drafter runtime":
// ctx = rms(fc . concat(taps)) * g_hidden): the GEMM writes the fused rows in
// bf16 from its epilogue, with each row's fp32 sum of squares per 256-column
// output tile, and a row kernel finishes the RMSNorm from those sums.
#pragma once
#include "common.h"

namespace dfl {

struct FuseEpi {
  uint16_t* y;  // [M][H] bf16 fused rows, before the norm
  float* ss;    // [M][H / 256] fp32 sums of squares of each row's 256-column tiles
};

// y = A . W^T (K columns, N = H rows of W) with the sums of squares; the k
// range is not split.
hipError_t launch_gemm_fuse_bf16(const uint16_t* A, int lda, int M, const SegTable& w, bool w_packed,
                                 int K, const FuseEpi& fe, hipStream_t st);

// out[r] = bf16(y[r] * rsqrt(sum_t ss[r][t] / H + eps) * gain), the ten tile
// sums added in order.
hipError_t launch_rownorm_tiles(const uint16_t* y, const float* ss, int rows, const uint16_t* gain,
                                float eps, uint16_t* out, int out_stride, hipStream_t st);

}  // namespace dfl
