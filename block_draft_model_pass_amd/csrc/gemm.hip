// bf16 "NT" GEMM on MFMA for the long-context steps: context fusion
// (taps [n][12800] x fc^T) and the context K/V projection
// (ctx [n][2560] x [Wk_0; Wv_0; ...; Wk_4; Wv_4]^T).  Both operands are
// k-contiguous, which is the native operand layout of MFMA 16x16x32: a lane
// reads 8 consecutive k of one row of A and of one row of W.
//
// Tile 128 x 128 x 64, 256 threads (2 x 2 waves of 64 x 64 = 4 x 4 MFMA
// tiles), double-buffered LDS with padded rows.
#include "common.h"

namespace dfl {

namespace {

constexpr int BM = 128, BN = 128, BK = 64, LDSK = BK + 8;

__global__ __launch_bounds__(256) void k_gemm_bf16_nt(const uint16_t* __restrict__ A, int lda,
                                                      int M, SegTable w, int K,
                                                      float* __restrict__ C, int ldc) {
  __shared__ uint16_t As[2][BM][LDSK];
  __shared__ uint16_t Ws[2][BN][LDSK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Tiles of one block row of C are spread over consecutive block ids so
  // that the blocks sharing an A panel run close together in time.
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  int seg = 0, base = 0;
  for (int i = 0; i + 1 < w.nseg; ++i)
    if (n0 >= w.row_end[i]) { seg = i + 1; base = w.row_end[i]; }
  const uint16_t* wb = static_cast<const uint16_t*>(w.ptr[seg]) + static_cast<size_t>(n0 - base) * K;

  uint4 ra[4], rw[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i, row = idx >> 3, kc = idx & 7;
      ra[i] = (m0 + row < M)
                  ? *reinterpret_cast<const uint4*>(A + static_cast<size_t>(m0 + row) * lda + k0 + 8 * kc)
                  : make_uint4(0, 0, 0, 0);
      rw[i] = *reinterpret_cast<const uint4*>(wb + static_cast<size_t>(row) * K + k0 + 8 * kc);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i, row = idx >> 3, kc = idx & 7;
      *reinterpret_cast<uint4*>(&As[buf][row][8 * kc]) = ra[i];
      *reinterpret_cast<uint4*>(&Ws[buf][row][8 * kc]) = rw[i];
    }
  };

  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 15, g = lane >> 4;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) acc[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  sstore(0);
  __syncthreads();
  const int nk = K / BK;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      uint4 af[4], wf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = *reinterpret_cast<const uint4*>(&As[cur][wm * 64 + i * 16 + r][ks * 32 + 8 * g]);
        wf[i] = *reinterpret_cast<const uint4*>(&Ws[cur][wn * 64 + i * 16 + r][ks * 32 + 8 * g]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) acc[i][jn] = mfma_bf16(af[i], wf[jn], acc[i][jn]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm * 64 + i * 16 + 4 * g + e;
        const int col = n0 + wn * 64 + jn * 16 + r;
        if (row < M) C[static_cast<size_t>(row) * ldc + col] = acc[i][jn][e];
      }
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* A, int lda, int M, const SegTable& w, int K, float* C,
                            int ldc, int N, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (N % BN || K % BK || lda % 8) return hipErrorInvalidValue;
  dim3 grid(N / BN, (M + BM - 1) / BM);
  hipLaunchKernelGGL(k_gemm_bf16_nt, grid, dim3(256), 0, st, A, lda, M, w, K, C, ldc);
  return hipGetLastError();
}

}  // namespace dfl
