// Streaming copy of a bf16 weight matrix [N][K] for the persistent pass:
// 16-row tiles, then 32-wide k blocks, then the 64 lanes of an MFMA
// 16x16x32 A operand (lane L: row L % 16, k 8 (L / 16) .. +8), 16 bytes each.
// A 64-lane load of one k block then reads 1 KiB of contiguous memory
// (instead of 64 bytes from each of 16 rows 5 KiB or more apart, which
// streams at about 2/3 of the rate on MI355X).  The same byte shuffle packs
// Q8_0 / Q4_0 / Q5_0 quants (64-byte row pieces = 64 or 128 k); their fp16
// block scales (and Q5_0's high-bit words) are packed per 16-row tile and k
// piece as 16 rows x U bytes.
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

// Units of U bytes: dst unit ((r / 16) * per_row + j) * 16 + r % 16 takes
// source unit r * per_row + j.
template <int U>
__global__ __launch_bounds__(256) void k_pack_units(const uint8_t* __restrict__ src, int N, int per_row,
                                                    uint8_t* __restrict__ dst) {
  const size_t n = static_cast<size_t>(N) * per_row;
  for (size_t q = blockIdx.x * 256ull + threadIdx.x; q < n; q += static_cast<size_t>(gridDim.x) * 256) {
    const size_t blk = q >> 4, r16 = q & 15;
    const size_t t = blk / per_row, j = blk % per_row;
    const size_t row = 16 * t + r16;
    if constexpr (U == 4)
      *reinterpret_cast<uint32_t*>(dst + U * q) = *reinterpret_cast<const uint32_t*>(src + U * (row * per_row + j));
    else
      *reinterpret_cast<uint2*>(dst + U * q) = *reinterpret_cast<const uint2*>(src + U * (row * per_row + j));
  }
}

// Fifth bit of block element e = 8 a + 4 b + c moves to bit 2 a + b + 8 c.
__device__ __forceinline__ uint32_t q5_reorder(uint32_t w) {
  uint32_t o = 0;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const int a = e >> 3, b = (e >> 2) & 1, c = e & 3;
    o |= ((w >> e) & 1u) << (2 * a + b + 8 * c);
  }
  return o;
}

// 16-byte units (the 4 words of one 128-k piece of a row): dst unit
// ((r / 16) * per_row + j) * 16 + r % 16 takes source unit r * per_row + j.
__global__ __launch_bounds__(256) void k_pack_q5_bits(const uint32_t* __restrict__ src, int N,
                                                      int per_row, uint32_t* __restrict__ dst) {
  const size_t n = static_cast<size_t>(N) * per_row;
  for (size_t q = blockIdx.x * 256ull + threadIdx.x; q < n; q += static_cast<size_t>(gridDim.x) * 256) {
    const size_t blk = q >> 4, r16 = q & 15;
    const size_t t = blk / per_row, j = blk % per_row;
    const uint4 v = *reinterpret_cast<const uint4*>(src + 4 * ((16 * t + r16) * per_row + j));
    *reinterpret_cast<uint4*>(dst + 4 * q) =
        make_uint4(q5_reorder(v.x), q5_reorder(v.y), q5_reorder(v.z), q5_reorder(v.w));
  }
}

}  // namespace

hipError_t launch_pack_q5_bits(const void* src, int N, int per_row, void* dst, hipStream_t st) {
  if (N <= 0 || N % 16 || per_row <= 0) return hipErrorInvalidValue;
  const size_t n = static_cast<size_t>(N) * per_row;
  const int grid = static_cast<int>(n / 256 < 8192 ? (n + 255) / 256 : 8192);
  hipLaunchKernelGGL(k_pack_q5_bits, dim3(grid), dim3(256), 0, st, static_cast<const uint32_t*>(src),
                     N, per_row, static_cast<uint32_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_pack_units(const void* src, int N, int per_row, int unit, void* dst,
                             hipStream_t st) {
  if (N <= 0 || N % 16 || per_row <= 0 || (unit != 4 && unit != 8)) return hipErrorInvalidValue;
  const size_t n = static_cast<size_t>(N) * per_row;
  const int grid = static_cast<int>(n / 256 < 8192 ? (n + 255) / 256 : 8192);
  if (unit == 4)
    hipLaunchKernelGGL(k_pack_units<4>, dim3(grid), dim3(256), 0, st, static_cast<const uint8_t*>(src),
                       N, per_row, static_cast<uint8_t*>(dst));
  else
    hipLaunchKernelGGL(k_pack_units<8>, dim3(grid), dim3(256), 0, st, static_cast<const uint8_t*>(src),
                       N, per_row, static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_pack_bf16(const void* src, int N, int K, void* dst, hipStream_t st) {
  if (N <= 0 || N % 16 || K % 32) return hipErrorInvalidValue;
  const size_t nq = static_cast<size_t>(N) * K / 8;
  const int grid = static_cast<int>(nq / 256 < 8192 ? (nq + 255) / 256 : 8192);
  hipLaunchKernelGGL(k_pack_bf16, dim3(grid), dim3(256), 0, st, static_cast<const uint16_t*>(src), N,
                     K, static_cast<uint16_t*>(dst));
  return hipGetLastError();
}

}  // namespace dfl
