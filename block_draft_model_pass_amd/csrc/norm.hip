// Row-wise epilogues of the context path: sum of split partials + RMSNorm of
// fused context rows, and the per-head k RMSNorm + NeoX RoPE of context K/V
// cells (Strata PR #1426 page, "Drafter runtime": full-head NeoX
// RoPE, theta 1e7; "Parity validation": q raw -> q normed -> q).
#include "common.h"

namespace dfl {

namespace {

constexpr int NT = 128;             // threads per row
constexpr int PER4 = H / (4 * NT);  // 5 groups of 4 consecutive elements per thread

// One row per block; thread t owns elements 4 (t + 128 i) .. +3, so every
// access is a 16-byte (fp32) or 8-byte (bf16) vector access.
template <int S>
__global__ __launch_bounds__(NT) void k_rownorm(float* h, const float* part, size_t sstride,
                                                int rstride, const uint16_t* gain, float eps,
                                                uint16_t* out, int ostride, uint16_t* out2) {
  __shared__ float red[NT / 64];
  const int b = blockIdx.x;
  f32x4 v[PER4];
  f32x4 pv[S][PER4];
  uint2 gv[PER4];
#pragma unroll
  for (int i = 0; i < PER4; ++i) {
    const int e = 4 * (threadIdx.x + NT * i);
    v[i] = h ? *reinterpret_cast<const f32x4*>(h + static_cast<size_t>(b) * H + e)
             : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S; ++s)
      pv[s][i] = *reinterpret_cast<const f32x4*>(part + s * sstride + static_cast<size_t>(b) * rstride + e);
    gv[i] = *reinterpret_cast<const uint2*>(gain + e);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < PER4; ++i) {
#pragma unroll
    for (int s = 0; s < S; ++s) v[i] += pv[s][i];
#pragma unroll
    for (int q = 0; q < 4; ++q) ss += v[i][q] * v[i][q];
  }
  if (h) {
#pragma unroll
    for (int i = 0; i < PER4; ++i)
      *reinterpret_cast<f32x4*>(h + static_cast<size_t>(b) * H + 4 * (threadIdx.x + NT * i)) = v[i];
  }
  ss = block_sum<NT>(ss, red);
  const float sc = 1.0f / sqrtf(ss / static_cast<float>(H) + eps);
#pragma unroll
  for (int i = 0; i < PER4; ++i) {
    const int e = 4 * (threadIdx.x + NT * i);
    const uint32_t g01 = gv[i].x, g23 = gv[i].y;
    const uint32_t y0 = f32_to_bf16(v[i][0] * sc * bf16_to_f32(static_cast<uint16_t>(g01)));
    const uint32_t y1 = f32_to_bf16(v[i][1] * sc * bf16_to_f32(static_cast<uint16_t>(g01 >> 16)));
    const uint32_t y2 = f32_to_bf16(v[i][2] * sc * bf16_to_f32(static_cast<uint16_t>(g23)));
    const uint32_t y3 = f32_to_bf16(v[i][3] * sc * bf16_to_f32(static_cast<uint16_t>(g23 >> 16)));
    const uint2 o = make_uint2(y0 | (y1 << 16), y2 | (y3 << 16));
    *reinterpret_cast<uint2*>(out + static_cast<size_t>(b) * ostride + e) = o;
    if (out2) *reinterpret_cast<uint2*>(out2 + static_cast<size_t>(b) * H + e) = o;
  }
}

// cos/sin of the NeoX RoPE angle pos * theta^(-2t/256), computed in fp64.
__device__ __forceinline__ void rope_cs(int64_t pos, int t, double theta, float& fc, float& fs) {
  const double inv = pow(theta, -2.0 * static_cast<double>(t) / static_cast<double>(D));
  const double ang = static_cast<double>(pos) * inv;
  double sn, cs;
  sincos(ang, &sn, &cs);
  fc = static_cast<float>(cs);
  fs = static_cast<float>(sn);
}

// RMSNorm over one 256-wide head held as (a, c) = elements (t, t + 128) of
// thread t, then NeoX rotation of the pair by the angle whose cos/sin are
// (fc, fs).
__device__ __forceinline__ void norm_rope(float& a, float& c, const uint16_t* gain, float eps,
                                          float fc, float fs, float* red) {
  const int t = threadIdx.x;
  const float ss = block_sum<128>(a * a + c * c, red);
  const float sc = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
  a *= sc * bf16_to_f32(gain[t]);
  c *= sc * bf16_to_f32(gain[t + 128]);
  const float a2 = a * fc - c * fs;
  const float c2 = c * fc + a * fs;
  a = a2;
  c = c2;
}

struct KNorms {
  const uint16_t* g[L];
};

// grid (n, 20): for layer l = y/4, w = y%4: w<2 key head w, else value head w-2.
__global__ __launch_bounds__(128) void k_kv_post(const float* y, int S, size_t split_stride,
                                                 int ldy, int64_t pos0, KNorms kn, float eps,
                                                 double theta, uint16_t* ring_k,
                                                 uint16_t* ring_vt, int cap) {
  __shared__ float red[2];
  const int row = blockIdx.x, l = blockIdx.y >> 2, w = blockIdx.y & 3, t = threadIdx.x;
  const int col = l * (2 * NKV * D) + w * D;
  float a = 0.f, c = 0.f;
  for (int s = 0; s < S; ++s) {
    const float* r = y + s * split_stride + static_cast<size_t>(row) * ldy + col;
    a += r[t];
    c += r[t + 128];
  }
  const int64_t pos = pos0 + row;
  const size_t cell = static_cast<size_t>(pos % cap);
  if (w < NKV) {
    float fc, fs;
    rope_cs(pos, t, theta, fc, fs);
    norm_rope(a, c, kn.g[l], eps, fc, fs, red);
    uint16_t* k = ring_k + ((static_cast<size_t>(l) * NKV + w) * cap + cell) * D;
    k[t] = f32_to_f16_bits(a);
    k[t + 128] = f32_to_f16_bits(c);
  } else {
    uint16_t* v = ring_vt + (static_cast<size_t>(l) * NKV + (w - NKV)) * D * cap +
                  (cell / BLK_CELLS) * (D * BLK_CELLS) + (cell % BLK_CELLS);
    v[static_cast<size_t>(t) * BLK_CELLS] = f32_to_f16_bits(a);
    v[static_cast<size_t>(t + 128) * BLK_CELLS] = f32_to_f16_bits(c);
  }
}

}  // namespace

hipError_t launch_rownorm(float* h, const float* part, int S, size_t part_split_stride,
                          int part_row_stride, int rows, const uint16_t* gain, float eps,
                          uint16_t* out, int out_stride, uint16_t* out2, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  switch (S) {
    case 1:
      hipLaunchKernelGGL(k_rownorm<1>, dim3(rows), dim3(NT), 0, st, h, part, part_split_stride,
                         part_row_stride, gain, eps, out, out_stride, out2);
      break;
    case 3:
      hipLaunchKernelGGL(k_rownorm<3>, dim3(rows), dim3(NT), 0, st, h, part, part_split_stride,
                         part_row_stride, gain, eps, out, out_stride, out2);
      break;
    case 5:
      hipLaunchKernelGGL(k_rownorm<5>, dim3(rows), dim3(NT), 0, st, h, part, part_split_stride,
                         part_row_stride, gain, eps, out, out_stride, out2);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_kv_post(const float* y, int S, size_t split_stride, int ldy, int n,
                          int64_t pos0, const void* const* k_norms, float eps, double theta,
                          uint16_t* ring_k, uint16_t* ring_vt, int capacity, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  KNorms kn;
  for (int l = 0; l < L; ++l) kn.g[l] = static_cast<const uint16_t*>(k_norms[l]);
  hipLaunchKernelGGL(k_kv_post, dim3(n, L * 2 * NKV), dim3(128), 0, st, y, S, split_stride, ldy,
                     pos0, kn, eps, theta, ring_k, ring_vt, capacity);
  return hipGetLastError();
}

}  // namespace dfl
