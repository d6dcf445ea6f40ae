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

struct KNorms {
  const uint16_t* g[L];
};

constexpr int KV_NT = 256;  // threads of a k_kv_post block

// Context K/V cells of n fused rows at positions pos0 .. pos0+n-1 (cell
// pos % cap): keys get the per-head RMSNorm with the layer's k gain and the
// NeoX rotation by pos * theta^(-2i/256) (pairs i, i+128; angle, sin and cos
// in fp64), values are stored as they are; both in fp16.
//
// grid (groups, L, 2): block (b, l, z) covers the 32 cells of the b-th
// aligned 32-cell group that the rows touch -- rows rb .. rb+31 with
// rb = 32 (pos0 / 32 + b) - pos0, only those in [0, n) written -- for layer
// l's two key heads (z = 0) or two value heads (z = 1).  Groups are the
// blocks of the value layout (32 cells, head dim outer), and cap % 32 == 0,
// so a group never wraps.
//  - keys: 8 threads per cell, thread p holding pairs 16p .. 16p+15 (two
//    64-byte runs of the row); the fp64 cos/sin of its 16 angles serve both
//    heads, the sum of squares is an 8-lane shuffle reduction, stores are
//    32-byte runs.
//  - values: thread t holds head dimension t and writes its 32 cells as 64
//    contiguous bytes (per-element stores where the group is partial).
__global__ __launch_bounds__(KV_NT) void k_kv_post(const float* y, int ldy, int n, int64_t pos0,
                                                   KNorms kn, float eps, double theta,
                                                   uint16_t* ring_k, uint16_t* ring_vt, int cap) {
  const int b = blockIdx.x, l = blockIdx.y, t = threadIdx.x;
  const int64_t gp = (pos0 / BLK_CELLS + b) * BLK_CELLS;  // position of the group's cell 0
  const int rb = static_cast<int>(gp - pos0);               // its row (negative if before pos0)
  const size_t gcell = static_cast<size_t>(gp % cap);
  if (blockIdx.z == 0) {
    __shared__ double invf[D / 2];
    if (t < D / 2) invf[t] = pow(theta, -2.0 * static_cast<double>(t) / static_cast<double>(D));
    __syncthreads();
    const int c = t >> 3, p = t & 7, row = rb + c;
    const bool valid = row >= 0 && row < n;
    const int rowc = row < 0 ? 0 : (row < n ? row : n - 1);  // in-bounds reads for unused cells
    float fc[16], fs[16];
    const double pos = static_cast<double>(gp + c);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      double sn, cs;
      sincos(pos * invf[16 * p + k], &sn, &cs);
      fc[k] = static_cast<float>(cs);
      fs[k] = static_cast<float>(sn);
    }
    const uint16_t* g = kn.g[l];
    const uint4* gl = reinterpret_cast<const uint4*>(g + 16 * p);
    const uint4* gh = reinterpret_cast<const uint4*>(g + D / 2 + 16 * p);
    const uint4 gv[4] = {gl[0], gl[1], gh[0], gh[1]};
#pragma unroll
    for (int j = 0; j < NKV; ++j) {
      const float* yr = y + static_cast<size_t>(rowc) * ldy + l * (2 * NKV * D) + j * D + 16 * p;
      float lo[16], hi[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 u = *reinterpret_cast<const f32x4*>(yr + 4 * q);
        const f32x4 v = *reinterpret_cast<const f32x4*>(yr + D / 2 + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[4 * q + e] = u[e];
          hi[4 * q + e] = v[e];
        }
      }
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) ss += lo[k] * lo[k] + hi[k] * hi[k];
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      ss += __shfl_xor(ss, 4);
      const float sc = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
      uint32_t olo[8], ohi[8];
#pragma unroll
      for (int k = 0; k < 16; k += 2) {
        float a[2], cc[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int kk = k + e;
          const uint32_t gw = reinterpret_cast<const uint32_t*>(&gv[kk / 8])[(kk % 8) / 2];
          const uint32_t hw = reinterpret_cast<const uint32_t*>(&gv[2 + kk / 8])[(kk % 8) / 2];
          const float ga = bf16_to_f32(static_cast<uint16_t>(kk & 1 ? gw >> 16 : gw));
          const float gc = bf16_to_f32(static_cast<uint16_t>(kk & 1 ? hw >> 16 : hw));
          const float x = lo[kk] * (sc * ga), z = hi[kk] * (sc * gc);
          a[e] = x * fc[kk] - z * fs[kk];
          cc[e] = z * fc[kk] + x * fs[kk];
        }
        olo[k / 2] = f32_to_f16_bits(a[0]) | (static_cast<uint32_t>(f32_to_f16_bits(a[1])) << 16);
        ohi[k / 2] = f32_to_f16_bits(cc[0]) | (static_cast<uint32_t>(f32_to_f16_bits(cc[1])) << 16);
      }
      if (valid) {
        uint16_t* k = ring_k + ((static_cast<size_t>(l) * NKV + j) * cap + gcell + c) * D + 16 * p;
        uint4* kl = reinterpret_cast<uint4*>(k);
        uint4* kh = reinterpret_cast<uint4*>(k + D / 2);
        kl[0] = make_uint4(olo[0], olo[1], olo[2], olo[3]);
        kl[1] = make_uint4(olo[4], olo[5], olo[6], olo[7]);
        kh[0] = make_uint4(ohi[0], ohi[1], ohi[2], ohi[3]);
        kh[1] = make_uint4(ohi[4], ohi[5], ohi[6], ohi[7]);
      }
    }
  } else {
    const bool full = rb >= 0 && rb + BLK_CELLS <= n;
#pragma unroll
    for (int j = 0; j < NKV; ++j) {
      const float* ycol = y + l * (2 * NKV * D) + (NKV + j) * D + t;
      uint16_t* v = ring_vt + (static_cast<size_t>(l) * NKV + j) * D * cap + (gcell / BLK_CELLS) * (D * BLK_CELLS) +
                    static_cast<size_t>(t) * BLK_CELLS;
      if (full) {
        uint32_t o[BLK_CELLS / 2];
#pragma unroll
        for (int c = 0; c < BLK_CELLS; c += 2) {
          const float v0 = ycol[static_cast<size_t>(rb + c) * ldy];
          const float v1 = ycol[static_cast<size_t>(rb + c + 1) * ldy];
          o[c / 2] = f32_to_f16_bits(v0) | (static_cast<uint32_t>(f32_to_f16_bits(v1)) << 16);
        }
        uint4* v4 = reinterpret_cast<uint4*>(v);
#pragma unroll
        for (int q = 0; q < 4; ++q) v4[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
      } else {
        for (int c = 0; c < BLK_CELLS; ++c) {
          const int row = rb + c;
          if (row >= 0 && row < n) v[c] = f32_to_f16_bits(ycol[static_cast<size_t>(row) * ldy]);
        }
      }
    }
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

hipError_t launch_kv_post(const float* y, int ldy, int n, int64_t pos0, const void* const* k_norms,
                          float eps, double theta, uint16_t* ring_k, uint16_t* ring_vt, int capacity,
                          hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (capacity % BLK_CELLS || pos0 < 0 || ldy % 4) return hipErrorInvalidValue;
  KNorms kn;
  for (int l = 0; l < L; ++l) kn.g[l] = static_cast<const uint16_t*>(k_norms[l]);
  const int64_t groups = (pos0 + n - 1) / BLK_CELLS - pos0 / BLK_CELLS + 1;
  if (groups > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_kv_post, dim3(static_cast<unsigned>(groups), L, 2), dim3(KV_NT), 0, st, y, ldy,
                     n, pos0, kn, eps, theta, ring_k, ring_vt, capacity);
  return hipGetLastError();
}

}  // namespace dfl
