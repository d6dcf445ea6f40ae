// Streaming copy of a bf16 weight matrix [N][K] for the persistent pass:
// 16-row tiles, then 32-wide k blocks, then the 64 lanes of an MFMA
// 16x16x32 A operand (lane L: row L % 16, k 8 (L / 16) .. +8), 16 bytes each.
// A 64-lane load of one k block then reads 1 KiB of contiguous memory
// (instead of 64 bytes from each of 16 rows 5 KiB or more apart, which
// streams at about 2/3 of the rate on MI355X).
#include "common.h"

namespace dfl {

namespace {

__global__ __launch_bounds__(256) void k_pack_bf16(const uint16_t* __restrict__ src, int N, int K,
                                                   uint16_t* __restrict__ dst) {
  const size_t nq = static_cast<size_t>(N) * K / 8;  // 16-byte pieces
  const size_t kb_per_tile = static_cast<size_t>(K / 32);
  for (size_t q = blockIdx.x * 256ull + threadIdx.x; q < nq; q += static_cast<size_t>(gridDim.x) * 256) {
    const size_t blk = q >> 6;
    const int L = static_cast<int>(q & 63);
    const size_t t = blk / kb_per_tile, kb = blk % kb_per_tile;
    const size_t row = 16 * t + (L & 15), col = 32 * kb + 8 * (L >> 4);
    *reinterpret_cast<uint4*>(dst + 8 * q) = *reinterpret_cast<const uint4*>(src + row * K + col);
  }
}

}  // namespace

hipError_t launch_pack_bf16(const void* src, int N, int K, void* dst, hipStream_t st) {
  if (N <= 0 || N % 16 || K % 32) return hipErrorInvalidValue;
  const size_t nq = static_cast<size_t>(N) * K / 8;
  const int grid = static_cast<int>(nq / 256 < 8192 ? (nq + 255) / 256 : 8192);
  hipLaunchKernelGGL(k_pack_bf16, dim3(grid), dim3(256), 0, st, static_cast<const uint16_t*>(src), N,
                     K, static_cast<uint16_t*>(dst));
  return hipGetLastError();
}

}  // namespace dfl
