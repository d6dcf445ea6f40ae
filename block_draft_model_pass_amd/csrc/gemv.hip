// Skinny GEMV kernels of the block pass: at most 16 activation rows against a
// weight matrix streamed once from HBM.  The contraction runs on MFMA
// 16x16x32 bf16: the weight tile is the A operand (16 output rows) and the
// activations the B operand (up to 16 rows, zero-padded), so each wave turns
// 1 KiB of weights into 4 MFMAs with no cross-lane reduction.
//
// Per 128-wide k block a lane of k-group g (0..3) loads four 16-byte pieces
// at k = 8*(4j + g), j = 0..3: every load instruction reads 64 contiguous
// bytes of each of 16 rows, and the same k slots are used for the weights and
// the activations, so the k order inside the MFMA does not matter.
#include "common.h"

namespace dfl {

namespace {

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ const uint16_t* seg_row(const SegTable& t, int row, int K) {
  int seg = 0, base = 0;
  for (int i = 0; i + 1 < t.nseg; ++i)
    if (row >= t.row_end[i]) { seg = i + 1; base = t.row_end[i]; }
  return static_cast<const uint16_t*>(t.ptr[seg]) + static_cast<size_t>(row - base) * K;
}

// Partial dot products of one wave: 16 weight rows x KBW*128 k, bf16.
template <int KBW>
__device__ __forceinline__ f32x4 wave_tile_bf16(const uint16_t* wrow, const uint16_t* xrow,
                                                bool xvalid, int kbeg, int g) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb) {
    uint4 w[4], x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = kbeg + kb * 128 + 8 * (4 * j + g);
      w[j] = ld16(wrow + k);
      x[j] = xvalid ? ld16(xrow + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = mfma_bf16(w[j], x[j], acc);
  }
  return acc;
}

template <int NW>
__device__ __forceinline__ f32x4 reduce_waves(f32x4 acc, f32x4 (*red)[64], int wave, int lane) {
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < NW - 1; ++w) acc += red[w][lane];
  }
  return acc;
}

// out[split][b][n] for one 16-row tile; grid = (N/16, S), block = NW waves.
template <int NW, int KBW>
__global__ __launch_bounds__(NW * 64) void k_gemv_bf16(GemvArgs a) {
  __shared__ f32x4 red[NW > 1 ? NW - 1 : 1][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const uint16_t* wrow = seg_row(a.w, row0, a.K) + static_cast<size_t>(r) * a.K;
  const bool xv = r < a.B;
  const uint16_t* xrow = a.x + static_cast<size_t>(xv ? r : 0) * a.x_stride;
  const int kbeg = (blockIdx.y * NW + wave) * (KBW * 128);
  f32x4 acc = wave_tile_bf16<KBW>(wrow, xrow, xv, kbeg, g);
  acc = reduce_waves<NW>(acc, red, wave, lane);
  if (wave == 0 && xv) {
    float* o = a.out + (static_cast<size_t>(blockIdx.y) * a.B + r) * a.N + row0 + 4 * g;
    *reinterpret_cast<f32x4*>(o) = acc;
  }
}

// u[b][n] = silu(gate) * up for one 16-row tile of the MLP; each wave streams
// both the gate and the up rows of its k range against the same activations.
template <int NW, int KBW>
__global__ __launch_bounds__(NW * 64) void k_gateup_bf16(const uint16_t* wg, const uint16_t* wu,
                                                         const uint16_t* x, int B, uint16_t* u) {
  __shared__ f32x4 red[2][NW - 1][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const bool xv = r < B;
  const uint16_t* xrow = x + static_cast<size_t>(xv ? r : 0) * H;
  const size_t roff = static_cast<size_t>(row0 + r) * H;
  const int kbeg = wave * (KBW * 128);
  f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < KBW; ++kb) {
    uint4 w1[4], w2[4], xx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = kbeg + kb * 128 + 8 * (4 * j + g);
      w1[j] = ld16(wg + roff + k);
      w2[j] = ld16(wu + roff + k);
      xx[j] = xv ? ld16(xrow + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ag = mfma_bf16(w1[j], xx[j], ag);
      au = mfma_bf16(w2[j], xx[j], au);
    }
  }
  if (wave > 0) {
    red[0][wave - 1][lane] = ag;
    red[1][wave - 1][lane] = au;
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < NW - 1; ++w) {
      ag += red[0][w][lane];
      au += red[1][w][lane];
    }
    if (xv) {
      uint16_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float z = ag[i];
        o[i] = f32_to_bf16(z / (1.0f + __expf(-z)) * au[i]);
      }
      uint2 pk = make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16),
                            o[2] | (static_cast<uint32_t>(o[3]) << 16));
      *reinterpret_cast<uint2*>(u + static_cast<size_t>(r) * F + row0 + 4 * g) = pk;
    }
  }
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  lo = __shfl_xor(lo, m, 64);
  hi = __shfl_xor(hi, m, 64);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// LM head: grid-stride over 16-row vocabulary tiles; each block keeps the
// best (value, lowest index) key per activation row and writes it once.
template <int NW, int KBW>
__global__ __launch_bounds__(NW * 64) void k_lmhead_bf16(const uint16_t* lm, int ntiles, int vocab,
                                                         const uint16_t* z, int B, uint64_t* keys,
                                                         uint16_t* logits) {
  __shared__ f32x4 red[NW - 1][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const bool xv = r < B;
  const uint16_t* xrow = z + static_cast<size_t>(xv ? r : 0) * H;
  const int kbeg = wave * (KBW * 128);
  uint64_t best = 0;
  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int row0 = t * 16;
    const uint16_t* wrow = lm + static_cast<size_t>(row0 + r) * H;
    f32x4 acc = wave_tile_bf16<KBW>(wrow, xrow, xv, kbeg, g);
    acc = reduce_waves<NW>(acc, red, wave, lane);
    if (wave == 0 && xv) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint64_t k = argmax_key(acc[i], static_cast<uint32_t>(row0 + 4 * g + i));
        best = k > best ? k : best;
      }
      if (logits) {
        uint16_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16(acc[i]);
        uint2 pk = make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16),
                              o[2] | (static_cast<uint32_t>(o[3]) << 16));
        *reinterpret_cast<uint2*>(logits + static_cast<size_t>(r) * vocab + row0 + 4 * g) = pk;
      }
    }
    __syncthreads();  // red[] is reused by the next tile
  }
  if (wave == 0) {
    uint64_t o = shfl_xor_u64(best, 16);
    best = o > best ? o : best;
    o = shfl_xor_u64(best, 32);
    best = o > best ? o : best;
    if (g == 0 && xv) keys[static_cast<size_t>(blockIdx.x) * MAXB + r] = best;
  }
}

// cand[b] = index part of the largest key over all blocks.
__global__ __launch_bounds__(256) void k_argmax_reduce(const uint64_t* keys, int nblk, int B,
                                                       int32_t* cand) {
  __shared__ uint64_t s[256];
  for (int b = 0; b < B; ++b) {
    uint64_t best = 0;
    for (int i = threadIdx.x; i < nblk; i += 256) {
      const uint64_t k = keys[static_cast<size_t>(i) * MAXB + b];
      best = k > best ? k : best;
    }
    s[threadIdx.x] = best;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (threadIdx.x < w) {
        const uint64_t o = s[threadIdx.x + w];
        if (o > s[threadIdx.x]) s[threadIdx.x] = o;
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) cand[b] = static_cast<int32_t>(~static_cast<uint32_t>(s[0]));
    __syncthreads();
  }
}

__global__ void k_verify(const int32_t* cand, const int32_t* target, int k, int32_t* out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int a = 0;
  while (a < k && cand[a] == target[a]) ++a;
  out[0] = a;
  out[1] = target[a];
}

}  // namespace

hipError_t launch_gemv(const GemvArgs& a, hipStream_t st) {
  if (a.fmt != W_BF16) return hipErrorInvalidValue;
  if (a.B < 1 || a.B > GEMV_ROWS || a.N % 16 || a.K % 128) return hipErrorInvalidValue;
  const int kblocks = a.K / 128;
  constexpr int NW = 4;
  if (kblocks % (NW * 5) == 0 && a.S == kblocks / (NW * 5)) {
    hipLaunchKernelGGL((k_gemv_bf16<NW, 5>), dim3(a.N / 16, a.S), dim3(NW * 64), 0, st, a);
  } else if (kblocks % (NW * 4) == 0 && a.S == kblocks / (NW * 4)) {
    hipLaunchKernelGGL((k_gemv_bf16<NW, 4>), dim3(a.N / 16, a.S), dim3(NW * 64), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gateup(const void* wg, const void* wu, int fmt, const uint16_t* x, int B,
                         uint16_t* u, hipStream_t st) {
  if (fmt != W_BF16 || B < 1 || B > GEMV_ROWS) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gateup_bf16<4, 5>), dim3(F / 16), dim3(256), 0, st,
                     static_cast<const uint16_t*>(wg), static_cast<const uint16_t*>(wu), x, B, u);
  return hipGetLastError();
}

hipError_t launch_lmhead_argmax(const uint16_t* lm, int vocab, const uint16_t* z, int B,
                                uint64_t* keys, int grid, uint16_t* logits_opt, int32_t* cand,
                                hipStream_t st) {
  if (B < 1 || B > MAXB || vocab % 16) return hipErrorInvalidValue;
  const int ntiles = vocab / 16;
  if (grid > ntiles) grid = ntiles;
  hipLaunchKernelGGL((k_lmhead_bf16<4, 5>), dim3(grid), dim3(256), 0, st, lm, ntiles, vocab, z, B,
                     keys, logits_opt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_argmax_reduce, dim3(1), dim3(256), 0, st, keys, grid, B, cand);
  return hipGetLastError();
}

hipError_t launch_verify(const int32_t* cand, const int32_t* target, int k, int32_t* out,
                         hipStream_t st) {
  hipLaunchKernelGGL(k_verify, dim3(1), dim3(64), 0, st, cand, target, k, out);
  return hipGetLastError();
}

}  // namespace dfl
