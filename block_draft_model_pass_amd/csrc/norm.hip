// Row-wise epilogues of the context path: sum of split partials + RMSNorm of
// fused context rows, and the per-head k RMSNorm + NeoX RoPE of context K/V
// cells (Strata PR #1426 page, "Drafter runtime": full-head NeoX
// RoPE, theta 1e7; "Parity validation": q raw -> q normed -> q).
#include "common.h"
#include "fuse.h"

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

// The RMSNorm of fused rows held in bf16 with their per-tile sums of squares
// (fuse_epilogue): one row per block, the H / 256 tile sums added in order
// (fp32, from the unrounded GEMM outputs), then each element scaled with the
// gain.
__global__ __launch_bounds__(NT) void k_rownorm_tiles(const uint16_t* y, const float* ss,
                                                      const uint16_t* gain, float eps, uint16_t* out,
                                                      int ostride) {
  constexpr int NTILE = H / 256;
  const int b = blockIdx.x;
  uint2 yv[PER4], gv[PER4];
#pragma unroll
  for (int i = 0; i < PER4; ++i) {
    const int e = 4 * (threadIdx.x + NT * i);
    yv[i] = *reinterpret_cast<const uint2*>(y + static_cast<size_t>(b) * H + e);
    gv[i] = *reinterpret_cast<const uint2*>(gain + e);
  }
  float sum = 0.f;
#pragma unroll
  for (int t = 0; t < NTILE; ++t) sum += ss[static_cast<size_t>(b) * NTILE + t];
  const float sc = 1.0f / sqrtf(sum / static_cast<float>(H) + eps);
#pragma unroll
  for (int i = 0; i < PER4; ++i) {
    const int e = 4 * (threadIdx.x + NT * i);
    const uint32_t w[2] = {yv[i].x, yv[i].y}, gw[2] = {gv[i].x, gv[i].y};
    uint32_t o[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t lo = f32_to_bf16(bf16_to_f32(static_cast<uint16_t>(w[q])) * sc *
                                      bf16_to_f32(static_cast<uint16_t>(gw[q])));
      const uint32_t hi = f32_to_bf16(bf16_to_f32(static_cast<uint16_t>(w[q] >> 16)) * sc *
                                      bf16_to_f32(static_cast<uint16_t>(gw[q] >> 16)));
      o[q] = lo | (hi << 16);
    }
    *reinterpret_cast<uint2*>(out + static_cast<size_t>(b) * ostride + e) = make_uint2(o[0], o[1]);
  }
}

struct KNorms {
  const uint16_t* g[L];
};

constexpr int KV_NT = 256;  // threads of a k_kv_post block

// Context K/V cells of n fused rows at positions pos0 .. pos0+n-1 (cell
// pos % cap): keys get the per-head RMSNorm with the layer's k gain and the
// NeoX rotation by pos * theta^(-2i/256) (pairs i, i+128; angle, sin and cos
// in fp64), values are stored as they are; both in fp16.  NS = 2: y is the
// sum of two k-split partials, ys floats apart.
//
// grid (groups8, L, 2 nz): keys (z < nz) or values, layer l = y, both heads
// of the kind per block (nz = 1) or one (nz = 2, calls of at most 64 rows):
//  - keys: block b covers the 8 cells of the b-th aligned 8-cell group the
//    rows touch (rows rb .. rb+7, rb = 8 (pos0 / 8 + b) - pos0; only rows in
//    [0, n) are written), 32 threads per cell, thread p holding pairs
//    4p .. 4p+3: its 4 fp64 angles (inverse frequencies from a per-block
//    table) serve both key heads of the layer -- a short chain per thread, so
//    a commit of a few rows is not held up by them; the sum of squares is a
//    32-lane shuffle reduction, stores are 8-byte runs.
//  - values: block b < groups32 covers the b-th aligned 32-cell group (the
//    blocks of the value layout: 32 cells, head dim outer; cap % 32 == 0, so a
//    group never wraps); thread t holds head dimension t and writes its 32
//    cells as 64 contiguous bytes (per-element stores where the group is
//    partial).  Blocks past groups32 have nothing to do.
template <int NS>
__global__ __launch_bounds__(KV_NT) void k_kv_post(const float* y, int ldy, size_t ys, int n,
                                                   int64_t pos0, KNorms kn, float eps, double theta,
                                                   uint16_t* ring_k, uint16_t* ring_vt, int cap) {
  const int b = blockIdx.x, l = blockIdx.y, t = threadIdx.x;
  // gridDim.z = 2 nz: nz = 1 (a block takes both heads of its kind) or NKV
  // (one head per block, for calls of a few rows, where latency matters more
  // than sharing the angles).
  const int nz = gridDim.z / 2, kind = blockIdx.z / nz, hpb = NKV / nz, j0 = (blockIdx.z % nz) * hpb;
  if (kind == 0) {
    constexpr int CPB = 8, TPC = KV_NT / CPB;  // cells per block, threads per cell (4 pairs each)
    const int64_t gp = (pos0 / CPB + b) * CPB;
    const int c = t / TPC, p = t % TPC, row = static_cast<int>(gp - pos0) + c;
    const bool valid = row >= 0 && row < n;
    const int rowc = row < 0 ? 0 : (row < n ? row : n - 1);  // in-bounds reads for unused cells
    const size_t cell = static_cast<size_t>((gp + c) % cap);
    // The projected values and the gains are loaded first, so that the
    // angles below are computed while they are in flight (head slots past
    // this block's heads re-read its first head and are never used).
    f32x4 lo[NKV], hi[NKV];
#pragma unroll
    for (int jj = 0; jj < NKV; ++jj) {
      const int j = jj < hpb ? j0 + jj : j0;
      const float* yr = y + static_cast<size_t>(rowc) * ldy + l * (2 * NKV * D) + j * D + 4 * p;
      lo[jj] = *reinterpret_cast<const f32x4*>(yr);
      hi[jj] = *reinterpret_cast<const f32x4*>(yr + D / 2);
      if constexpr (NS == 2) {
        lo[jj] += *reinterpret_cast<const f32x4*>(yr + ys);
        hi[jj] += *reinterpret_cast<const f32x4*>(yr + ys + D / 2);
      }
    }
    const uint16_t* g = kn.g[l];
    const uint2 gl = *reinterpret_cast<const uint2*>(g + 4 * p);
    const uint2 gh = *reinterpret_cast<const uint2*>(g + D / 2 + 4 * p);
    __shared__ double invf[D / 2];
    if (t < D / 2) invf[t] = pow(theta, -2.0 * static_cast<double>(t) / static_cast<double>(D));
    __syncthreads();
    float fc[4], fs[4];
    const double pos = static_cast<double>(gp + c);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      double sn, cs;
      sincos(pos * invf[4 * p + k], &sn, &cs);
      fc[k] = static_cast<float>(cs);
      fs[k] = static_cast<float>(sn);
    }
    const float ga[4] = {bf16_to_f32(static_cast<uint16_t>(gl.x)), bf16_to_f32(static_cast<uint16_t>(gl.x >> 16)),
                         bf16_to_f32(static_cast<uint16_t>(gl.y)), bf16_to_f32(static_cast<uint16_t>(gl.y >> 16))};
    const float gc[4] = {bf16_to_f32(static_cast<uint16_t>(gh.x)), bf16_to_f32(static_cast<uint16_t>(gh.x >> 16)),
                         bf16_to_f32(static_cast<uint16_t>(gh.y)), bf16_to_f32(static_cast<uint16_t>(gh.y >> 16))};
#pragma unroll
    for (int jj = 0; jj < NKV; ++jj) {
      if (jj >= hpb) break;
      const int j = j0 + jj;
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) ss += fmaf(hi[jj][k], hi[jj][k], lo[jj][k] * lo[jj][k]);
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      ss += __shfl_xor(ss, 4);
      ss += __shfl_xor(ss, 8);
      ss += __shfl_xor(ss, 16);
      const float sc = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
      uint32_t olo[2], ohi[2];
#pragma unroll
      for (int k = 0; k < 4; k += 2) {
        float a[2], cc[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float x = lo[jj][k + e] * (sc * ga[k + e]), z = hi[jj][k + e] * (sc * gc[k + e]);
          a[e] = fmaf(x, fc[k + e], -(z * fs[k + e]));
          cc[e] = fmaf(z, fc[k + e], x * fs[k + e]);
        }
        olo[k / 2] = f32_to_f16_bits(a[0]) | (static_cast<uint32_t>(f32_to_f16_bits(a[1])) << 16);
        ohi[k / 2] = f32_to_f16_bits(cc[0]) | (static_cast<uint32_t>(f32_to_f16_bits(cc[1])) << 16);
      }
      if (valid) {
        uint16_t* k = ring_k + ((static_cast<size_t>(l) * NKV + j) * cap + cell) * D + 4 * p;
        *reinterpret_cast<uint2*>(k) = make_uint2(olo[0], olo[1]);
        *reinterpret_cast<uint2*>(k + D / 2) = make_uint2(ohi[0], ohi[1]);
      }
    }
  } else {
    const int64_t groups32 = (pos0 + n - 1) / BLK_CELLS - pos0 / BLK_CELLS + 1;
    if (b >= groups32) return;
    const int64_t gp = (pos0 / BLK_CELLS + b) * BLK_CELLS;  // position of the group's cell 0
    const int rb = static_cast<int>(gp - pos0);               // its row (negative if before pos0)
    const size_t gcell = static_cast<size_t>(gp % cap);
    const bool full = rb >= 0 && rb + BLK_CELLS <= n;
#pragma unroll
    for (int jj = 0; jj < NKV; ++jj) {
      if (jj >= hpb) break;
      const int j = j0 + jj;
      const float* ycol = y + l * (2 * NKV * D) + (NKV + j) * D + t;
      uint16_t* v = ring_vt + (static_cast<size_t>(l) * NKV + j) * D * cap + (gcell / BLK_CELLS) * (D * BLK_CELLS) +
                    static_cast<size_t>(t) * BLK_CELLS;
      // All 32 loads go out together (rows outside [0, n) re-read a row of
      // the call and are never stored).
      uint32_t o[BLK_CELLS / 2];
#pragma unroll
      for (int c = 0; c < BLK_CELLS; c += 2) {
        const int r0 = rb + c < 0 ? 0 : (rb + c < n ? rb + c : n - 1);
        const int r1 = rb + c + 1 < 0 ? 0 : (rb + c + 1 < n ? rb + c + 1 : n - 1);
        float v0 = ycol[static_cast<size_t>(r0) * ldy];
        float v1 = ycol[static_cast<size_t>(r1) * ldy];
        if constexpr (NS == 2) {
          v0 += ycol[static_cast<size_t>(r0) * ldy + ys];
          v1 += ycol[static_cast<size_t>(r1) * ldy + ys];
        }
        o[c / 2] = f32_to_f16_bits(v0) | (static_cast<uint32_t>(f32_to_f16_bits(v1)) << 16);
      }
      if (full) {
        uint4* v4 = reinterpret_cast<uint4*>(v);
#pragma unroll
        for (int q = 0; q < 4; ++q) v4[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
      } else {
#pragma unroll
        for (int c = 0; c < BLK_CELLS; ++c) {
          const int row = rb + c;
          if (row >= 0 && row < n) v[c] = static_cast<uint16_t>(o[c / 2] >> (16 * (c & 1)));
        }
      }
    }
  }
}

// RoPE table of rows pos0 .. pos0 + n - 1: block b takes rows rpb b ..
// rpb b + rpb - 1, thread i the pair i: its inverse frequency once, then the
// angle of each row; in fp64 exactly as k_kv_post computes them.
__global__ __launch_bounds__(D / 2) void k_rope_rows(float2* tab, int64_t pos0, int n, int rpb, double theta) {
  const int i = threadIdx.x, r0 = rpb * blockIdx.x;
  const double invf = pow(theta, -2.0 * static_cast<double>(i) / static_cast<double>(D));
  const int r1 = n - r0 < rpb ? n - r0 : rpb;
  for (int r = 0; r < r1; ++r) {
    double sn, cs;
    sincos(static_cast<double>(pos0 + r0 + r) * invf, &sn, &cs);
    tab[static_cast<size_t>(r0 + r) * (D / 2) + i] = make_float2(static_cast<float>(cs), static_cast<float>(sn));
  }
}

}  // namespace

hipError_t launch_rope_rows(float2* tab, int64_t pos0, int n, double theta, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (pos0 < 0 || !tab) return hipErrorInvalidValue;
  // rows per block: up to 32 (one pow per thread for many rows), while the
  // grid keeps at least ~512 blocks for the fp64 sincos
  const int rpb = n >= 32 * 512 ? 32 : (n >= 2 * 512 ? n / 512 : 1);
  hipLaunchKernelGGL(k_rope_rows, dim3(static_cast<unsigned>((n + rpb - 1) / rpb)), dim3(D / 2), 0, st, tab,
                     pos0, n, rpb, theta);
  return hipGetLastError();
}

hipError_t launch_rownorm(float* h, const float* part, int S, size_t part_split_stride,
                          int part_row_stride, int rows, const uint16_t* gain, float eps,
                          uint16_t* out, int out_stride, uint16_t* out2, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  switch (S) {
    case 1:
      hipLaunchKernelGGL(k_rownorm<1>, dim3(rows), dim3(NT), 0, st, h, part, part_split_stride,
                         part_row_stride, gain, eps, out, out_stride, out2);
      break;
    case 2:
      hipLaunchKernelGGL(k_rownorm<2>, dim3(rows), dim3(NT), 0, st, h, part, part_split_stride,
                         part_row_stride, gain, eps, out, out_stride, out2);
      break;
    case 10:
      hipLaunchKernelGGL(k_rownorm<10>, dim3(rows), dim3(NT), 0, st, h, part, part_split_stride,
                         part_row_stride, gain, eps, out, out_stride, out2);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rownorm_tiles(const uint16_t* y, const float* ss, int rows, const uint16_t* gain,
                                float eps, uint16_t* out, int out_stride, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rownorm_tiles, dim3(rows), dim3(NT), 0, st, y, ss, gain, eps, out, out_stride);
  return hipGetLastError();
}

hipError_t launch_kv_post(const float* y, int ldy, int nsplit, size_t split_stride, int n,
                          int64_t pos0, const void* const* k_norms, float eps, double theta,
                          uint16_t* ring_k, uint16_t* ring_vt, int capacity, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (capacity % BLK_CELLS || pos0 < 0 || ldy % 4 || nsplit < 1 || nsplit > 2 || split_stride % 4)
    return hipErrorInvalidValue;
  KNorms kn;
  for (int l = 0; l < L; ++l) kn.g[l] = static_cast<const uint16_t*>(k_norms[l]);
  // 8-cell key groups; the value blocks use the first groups32 of them.
  const int64_t groups = (pos0 + n - 1) / 8 - pos0 / 8 + 1;
  if (groups > 0x7fffffff) return hipErrorInvalidValue;
  const int nz = n <= 64 ? NKV : 1;
  const dim3 grid(static_cast<unsigned>(groups), L, 2 * nz);
  if (nsplit == 2)
    hipLaunchKernelGGL(k_kv_post<2>, grid, dim3(KV_NT), 0, st, y, ldy, split_stride, n, pos0, kn, eps,
                       theta, ring_k, ring_vt, capacity);
  else
    hipLaunchKernelGGL(k_kv_post<1>, grid, dim3(KV_NT), 0, st, y, ldy, size_t{0}, n, pos0, kn, eps,
                       theta, ring_k, ring_vt, capacity);
  return hipGetLastError();
}

}  // namespace dfl
