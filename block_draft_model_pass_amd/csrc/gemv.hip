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
//
// Bytes in flight decide the achieved bandwidth: every wave issues all the
// weight loads of its slice (KBW blocks = KBW KiB per wave) before its first
// MFMA (a scheduling barrier keeps the compiler from interleaving them), and
// the LM head double-buffers whole tiles while reusing the activation
// fragments it loaded once.
#include "common.h"

namespace dfl {

namespace {

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Streamed once: keep weights from displacing reusable lines in the caches.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16_stream(const uint16_t* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

__device__ __forceinline__ const uint16_t* seg_row(const SegTable& t, int row, int K) {
  int seg = 0, base = 0;
  for (int i = 0; i + 1 < t.nseg; ++i)
    if (row >= t.row_end[i]) { seg = i + 1; base = t.row_end[i]; }
  return static_cast<const uint16_t*>(t.ptr[seg]) + static_cast<size_t>(row - base) * K;
}

template <int KBW>
__device__ __forceinline__ void load_w(uint4 (&w)[4 * KBW], const uint16_t* wrow, int kbeg,
                                       int g) {
#pragma unroll
  for (int i = 0; i < 4 * KBW; ++i) w[i] = ld16_stream(wrow + kbeg + 8 * (4 * i + g));
}

// Tile t's 16 rows from the LM head: row-major, or its streaming copy
// (16-row tiles, 32-wide k blocks, 64 MFMA lanes of 16 bytes: one 1 KiB
// contiguous run per wave load).
template <int KBW, bool PACKED>
__device__ __forceinline__ void load_lm(uint4 (&w)[4 * KBW], const uint16_t* lm, int t, int r,
                                        int kbeg, int g) {
  if constexpr (PACKED) {
    const uint16_t* b = lm + ((static_cast<size_t>(t) * (H / 32) + kbeg / 32) * 64 + r + 16 * g) * 8;
#pragma unroll
    for (int i = 0; i < 4 * KBW; ++i) w[i] = ld16_stream(b + 512 * i);
  } else {
    load_w<KBW>(w, lm + (static_cast<size_t>(t) * 16 + r) * H, kbeg, g);
  }
}

template <int KBW>
__device__ __forceinline__ void load_x(uint4 (&x)[4 * KBW], const uint16_t* xrow, bool valid,
                                       int kbeg, int g) {
#pragma unroll
  for (int i = 0; i < 4 * KBW; ++i)
    x[i] = valid ? ld16(xrow + kbeg + 8 * (4 * i + g)) : make_uint4(0, 0, 0, 0);
}

template <int KBW>
__device__ __forceinline__ f32x4 mma_chain(const uint4 (&w)[4 * KBW], const uint4 (&x)[4 * KBW]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4 * KBW; ++i) acc = mfma_bf16(w[i], x[i], acc);
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

// The matrix segment holding rows row0 .. row0+15 (segments are whole
// multiples of 16 rows): its buffer, its row count and row0 inside it.
struct SegRef {
  const uint8_t* base;
  int rows, row0;
};

__device__ __forceinline__ SegRef seg_ref(const SegTable& t, int row0) {
  int seg = 0, prev = 0;
  for (int i = 0; i + 1 < t.nseg; ++i)
    if (row0 >= t.row_end[i]) { seg = i + 1; prev = t.row_end[i]; }
  return SegRef{static_cast<const uint8_t*>(t.ptr[seg]), t.row_end[seg] - prev, row0 - prev};
}

template <int FMT> struct KPerLoad;  // k covered by one 16-byte load of all four lane groups
template <> struct KPerLoad<W_BF16> { static constexpr int v = 32; };
template <> struct KPerLoad<W_Q8_0> { static constexpr int v = 64; };
template <> struct KPerLoad<W_Q4_0> { static constexpr int v = 128; };
template <> struct KPerLoad<W_Q5_0> { static constexpr int v = 128; };

// k offset (from the wave's kbeg) of the i-th 8-element activation group of
// lane group g, matching the weight slots of each format:
//   bf16 load i -> k = 32 i + 8 g;  Q8_0 load i -> 16 elements at 64 i + 16 g;
//   Q4_0 / Q5_0 load i -> the 32-element quant block at 128 i + 32 g.
template <int FMT>
__device__ __forceinline__ int xslot(int i, int g) {
  if constexpr (FMT == W_BF16) return 32 * i + 8 * g;
  else if constexpr (FMT == W_Q8_0) return 64 * (i >> 1) + 16 * g + 8 * (i & 1);
  else return 128 * (i >> 2) + 32 * g + 8 * (i & 3);
}

// 8 bf16 -> 8 fp16 (round to nearest even).
__device__ __forceinline__ uint4 bf16x8_to_f16(uint4 v) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xffff0000u);
    w[i] = static_cast<uint32_t>(f32_to_f16_bits(lo)) | (static_cast<uint32_t>(f32_to_f16_bits(hi)) << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// out[split][b][n] for one 16-row tile; grid = (N/16, S), block = NW waves.
// Quantized weights are decoded to fp16 in registers (the same slot scheme
// and decode as the pass kernel) and run on MFMA f16 against the
// activations converted to fp16.
template <int FMT, int NW, int KBW, bool PACKED>
__global__ __launch_bounds__(NW * 64) void k_gemv(GemvArgs a) {
  __shared__ f32x4 red[NW > 1 ? NW - 1 : 1][64];
  constexpr int NX = 4 * KBW;                           // 8-element activation groups per lane
  constexpr int NL = KBW * 128 / KPerLoad<FMT>::v;      // 16-byte weight loads per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const SegRef sr = seg_ref(a.w, blockIdx.x * 16);
  const int row = sr.row0 + r;
  const bool xv = r < a.B;
  const uint16_t* xrow = a.x + static_cast<size_t>(xv ? r : 0) * a.x_stride;
  const int kbeg = (blockIdx.y * NW + wave) * (KBW * 128);
  const size_t rk = static_cast<size_t>(row) * a.K;
  const size_t sb = static_cast<size_t>(row) * (a.K / 32) + kbeg / 32;
  uint4 w[NL];
  uint32_t sc[NL], hw[FMT == W_Q5_0 ? NL : 1];
  // Q5_0 high-bit words follow the quants and the scales
  const uint8_t* hb = sr.base + static_cast<size_t>(sr.rows) * a.K / 2 + static_cast<size_t>(sr.rows) * a.K / 16;
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    if constexpr (PACKED) {
      // streaming copy: 16-row tile, then 64-byte row pieces (32 bf16, 64
      // Q8_0 or 128 Q4_0 / Q5_0 k), then the lanes; scales (and high-bit
      // words) per tile and piece
      constexpr int PK = FMT == W_BF16 ? 32 : (FMT == W_Q8_0 ? 64 : 128);
      const size_t pc = static_cast<size_t>(row >> 4) * (a.K / PK) + kbeg / PK + i;
      w[i] = ld16_stream(reinterpret_cast<const uint16_t*>(sr.base + (pc * 64 + r + 16 * g) * 16));
      if constexpr (FMT == W_BF16)
        sc[i] = 0;
      else if constexpr (FMT == W_Q8_0)
        sc[i] = *reinterpret_cast<const uint16_t*>(sr.base + static_cast<size_t>(sr.rows) * a.K +
                                                   2 * (pc * 32 + r * 2 + (g >> 1)));
      else
        sc[i] = *reinterpret_cast<const uint16_t*>(sr.base + static_cast<size_t>(sr.rows) * a.K / 2 +
                                                   2 * (pc * 64 + r * 4 + g));
      if constexpr (FMT == W_Q5_0) hw[i] = *reinterpret_cast<const uint32_t*>(hb + 4 * (pc * 64 + r * 4 + g));
    } else if constexpr (FMT == W_BF16) {
      w[i] = ld16_stream(reinterpret_cast<const uint16_t*>(sr.base) + rk + kbeg + 32 * i + 8 * g);
      sc[i] = 0;
    } else if constexpr (FMT == W_Q8_0) {
      w[i] = ld16_stream(reinterpret_cast<const uint16_t*>(sr.base + rk + kbeg + 64 * i + 16 * g));
      sc[i] = *reinterpret_cast<const uint16_t*>(sr.base + static_cast<size_t>(sr.rows) * a.K +
                                                 2 * (sb + 2 * i + (g >> 1)));
    } else {
      w[i] = ld16_stream(reinterpret_cast<const uint16_t*>(sr.base + (rk + kbeg) / 2 + 64 * i + 16 * g));
      sc[i] = *reinterpret_cast<const uint16_t*>(sr.base + static_cast<size_t>(sr.rows) * a.K / 2 +
                                                 2 * (sb + 4 * i + g));
      if constexpr (FMT == W_Q5_0) hw[i] = *reinterpret_cast<const uint32_t*>(hb + 4 * (sb + 4 * i + g));
    }
  }
  uint4 x[NX];
#pragma unroll
  for (int i = 0; i < NX; ++i)
    x[i] = xv ? ld16(xrow + kbeg + xslot<FMT>(i, g)) : make_uint4(0, 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    if constexpr (FMT == W_BF16) {
      acc = mfma_bf16(w[i], x[i], acc);
    } else if constexpr (FMT == W_Q8_0) {
      const h2 s2 = scale_h2(sc[i]);
      acc = mfma_f16(dq8(w[i].x, w[i].y, s2), bf16x8_to_f16(x[2 * i]), acc);
      acc = mfma_f16(dq8(w[i].z, w[i].w, s2), bf16x8_to_f16(x[2 * i + 1]), acc);
    } else if constexpr (FMT == W_Q4_0) {
      const h2 s2 = scale_h2(sc[i]);
      acc = mfma_f16(dq4(w[i].x, w[i].y, false, s2), bf16x8_to_f16(x[4 * i]), acc);
      acc = mfma_f16(dq4(w[i].z, w[i].w, false, s2), bf16x8_to_f16(x[4 * i + 1]), acc);
      acc = mfma_f16(dq4(w[i].x, w[i].y, true, s2), bf16x8_to_f16(x[4 * i + 2]), acc);
      acc = mfma_f16(dq4(w[i].z, w[i].w, true, s2), bf16x8_to_f16(x[4 * i + 3]), acc);
    } else {  // Q5_0: elements 4 C .. 4 C + 3 take the fifth bits of group C
      const h2 s2 = scale_h2(sc[i]);
      uint32_t b[8];
      if constexpr (PACKED) {
        b[0] = q5_bits_packed<0>(hw[i]), b[1] = q5_bits_packed<1>(hw[i]);
        b[2] = q5_bits_packed<2>(hw[i]), b[3] = q5_bits_packed<3>(hw[i]);
        b[4] = q5_bits_packed<4>(hw[i]), b[5] = q5_bits_packed<5>(hw[i]);
        b[6] = q5_bits_packed<6>(hw[i]), b[7] = q5_bits_packed<7>(hw[i]);
      } else {
        b[0] = q5_bits_rowmajor<0>(hw[i]), b[1] = q5_bits_rowmajor<1>(hw[i]);
        b[2] = q5_bits_rowmajor<2>(hw[i]), b[3] = q5_bits_rowmajor<3>(hw[i]);
        b[4] = q5_bits_rowmajor<4>(hw[i]), b[5] = q5_bits_rowmajor<5>(hw[i]);
        b[6] = q5_bits_rowmajor<6>(hw[i]), b[7] = q5_bits_rowmajor<7>(hw[i]);
      }
      acc = mfma_f16(dq5(w[i].x, w[i].y, false, b[0], b[1], s2), bf16x8_to_f16(x[4 * i]), acc);
      acc = mfma_f16(dq5(w[i].z, w[i].w, false, b[2], b[3], s2), bf16x8_to_f16(x[4 * i + 1]), acc);
      acc = mfma_f16(dq5(w[i].x, w[i].y, true, b[4], b[5], s2), bf16x8_to_f16(x[4 * i + 2]), acc);
      acc = mfma_f16(dq5(w[i].z, w[i].w, true, b[6], b[7], s2), bf16x8_to_f16(x[4 * i + 3]), acc);
    }
  }
  acc = reduce_waves<NW>(acc, red, wave, lane);
  if (wave == 0 && xv) {
    float* o = a.out + (static_cast<size_t>(blockIdx.y) * a.B + r) * a.N + blockIdx.x * 16 + 4 * g;
    *reinterpret_cast<f32x4*>(o) = acc;
  }
}

// Quantized [rows][K] (fmt Q8_0 / Q4_0 / Q5_0) -> rows row0.. of a bf16 [.][K]
// matrix in the streaming layout (the 8 bf16 values of an output group are
// one lane's contiguous 16 bytes there).  One thread per 8 output elements.
// The source is either the row-major blocks (quants row-major, then scales
// row-major) or, with PACKED, the matrix's streaming copy (quants as 64-byte
// row pieces in MFMA lane order, scales regrouped per 16-row tile and piece).
template <int FMT, bool PACKED>
__global__ __launch_bounds__(256) void k_dequant_bf16(const uint8_t* src, int rows, int K,
                                                      uint16_t* dst, int row0) {
  const size_t n8 = static_cast<size_t>(rows) * K / 8;
  const size_t qbytes = FMT == W_Q8_0 ? static_cast<size_t>(rows) * K : static_cast<size_t>(rows) * K / 2;
  for (size_t e = blockIdx.x * 256ull + threadIdx.x; e < n8; e += static_cast<size_t>(gridDim.x) * 256) {
    const size_t r = e * 8 / K, k = e * 8 % K;  // row and first element of the group
    // byte offset of the group's quants (8 bytes for Q8_0; for Q4_0 / Q5_0 the 8
    // bytes holding its nibbles) and element offset of its block scale
    size_t qoff, soff;
    if constexpr (!PACKED) {
      qoff = FMT == W_Q8_0 ? r * K + k : r * K / 2 + 16 * (k / 32) + (k % 16);
      soff = r * (K / 32) + k / 32;
    } else {
      const size_t kpc = FMT == W_Q8_0 ? 64 : 128;  // k per 64-byte piece
      const size_t P = K / kpc, pc = (r / 16) * P + k / kpc;
      const size_t jb = FMT == W_Q8_0 ? k % 64 : 16 * ((k % 128) / 32) + (k % 16);
      qoff = (pc * 64 + r % 16 + 16 * (jb / 16)) * 16 + jb % 16;
      soff = (pc * 16 + r % 16) * (FMT == W_Q8_0 ? 2 : 4) + (k % kpc) / 32;
    }
    const float s = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(src + qbytes + 2 * soff));
    const uint2 q = *reinterpret_cast<const uint2*>(src + qoff);
    // Q5_0: the block's high-bit word (same index as its scale), after the scales
    uint32_t hw = 0;
    if constexpr (FMT == W_Q5_0)
      hw = *reinterpret_cast<const uint32_t*>(src + qbytes + static_cast<size_t>(rows) * (K / 32) * 2 +
                                              4 * soff);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t word = i < 4 ? q.x : q.y;
      const uint32_t byte = (word >> (8 * (i & 3))) & 0xffu;
      if constexpr (FMT == W_Q8_0) {
        v[i] = static_cast<float>(static_cast<int8_t>(byte)) * s;
      } else {  // element j of a block: byte j % 16, low nibble if j < 16 else high
        const int nib = k % 32 < 16 ? static_cast<int>(byte & 15u) : static_cast<int>(byte >> 4);
        if constexpr (FMT == W_Q4_0) {
          v[i] = static_cast<float>(nib - 8) * s;
        } else {  // fifth bit of element j: bit j, or bit 2 (j/8) + (j/4)%2 + 8 (j%4) when packed
          const int j = static_cast<int>(k % 32) + i;
          const int bit = PACKED ? 2 * (j >> 3) + ((j >> 2) & 1) + 8 * (j & 3) : j;
          v[i] = static_cast<float>((nib | static_cast<int>(((hw >> bit) & 1u) << 4)) - 16) * s;
        }
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
    const size_t n = row0 + r;
    const size_t at = ((n / 16 * (K / 32) + k / 32) * 64 + n % 16 + 16 * ((k % 32) / 8)) * 8;
    *reinterpret_cast<uint4*>(dst + at) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  lo = __shfl_xor(lo, m, 64);
  hi = __shfl_xor(hi, m, 64);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// One LM-head tile's epilogue on wave 0: argmax key update and optional
// bf16 logits.
__device__ __forceinline__ void lm_epilogue(f32x4 acc, int row0, int r, int g, bool xv,
                                            int vocab, uint16_t* logits, uint64_t& best) {
  if (!xv) return;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    best = umax64(best, argmax_key(acc[i], static_cast<uint32_t>(row0 + 4 * g + i)));
  if (logits) {
    uint16_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16(acc[i]);
    uint2 pk = make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16),
                          o[2] | (static_cast<uint32_t>(o[3]) << 16));
    *reinterpret_cast<uint2*>(logits + static_cast<size_t>(r) * vocab + row0 + 4 * g) = pk;
  }
}

// LM head: grid-stride over 16-row vocabulary tiles.  Each wave keeps the
// activation fragments of its k quarter in registers and double-buffers the
// weight tiles; each block keeps the best (value, lowest index) key per
// activation row and writes it once.
template <int NW, int KBW, bool PACKED>
__global__ __launch_bounds__(NW * 64) void k_lmhead_bf16(const uint16_t* lm, int ntiles, int vocab,
                                                         const uint16_t* z, int B, uint64_t* keys,
                                                         uint16_t* logits) {
  __shared__ f32x4 red[2][NW - 1][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const bool xv = r < B;
  const int kbeg = wave * (KBW * 128);
  uint4 x[4 * KBW];
  load_x<KBW>(x, z + static_cast<size_t>(xv ? r : 0) * H, xv, kbeg, g);
  uint64_t best = 0;
  const int step = gridDim.x;
  int t = blockIdx.x;
  uint4 wa[4 * KBW], wb[4 * KBW];
  if (t < ntiles) load_lm<KBW, PACKED>(wa, lm, t, r, kbeg, g);
  int parity = 0;
  while (t < ntiles) {
    // tile t is in wa; prefetch t + step into wb, compute wa (then the roles swap)
    const int tn = t + step;
    if (tn < ntiles) load_lm<KBW, PACKED>(wb, lm, tn, r, kbeg, g);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc = mma_chain<KBW>(wa, x);
    if (wave > 0) red[parity][wave - 1][lane] = acc;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < NW - 1; ++w) acc += red[parity][w][lane];
      lm_epilogue(acc, t * 16, r, g, xv, vocab, logits, best);
    }
    parity ^= 1;
    t = tn;
    if (t >= ntiles) break;
    const int tn2 = t + step;
    if (tn2 < ntiles) load_lm<KBW, PACKED>(wa, lm, tn2, r, kbeg, g);
    __builtin_amdgcn_sched_barrier(0);
    acc = mma_chain<KBW>(wb, x);
    if (wave > 0) red[parity][wave - 1][lane] = acc;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < NW - 1; ++w) acc += red[parity][w][lane];
      lm_epilogue(acc, t * 16, r, g, xv, vocab, logits, best);
    }
    parity ^= 1;
    t = tn2;
  }
  if (wave == 0) {
    best = umax64(best, shfl_xor_u64(best, 16));
    best = umax64(best, shfl_xor_u64(best, 32));
    if (g == 0 && xv) keys[static_cast<size_t>(blockIdx.x) * MAXB + r] = best;
  }
}

// Q8_0 LM head: the same sweep as k_lmhead_bf16 over a [vocab][2560] matrix of
// Q8_0 blocks (row-major quants then scales, or the streaming copy: 64-byte
// row pieces in MFMA lane order, scales per 16-row tile and piece).  One
// 16-byte load holds 16 int8 of one quant block (64 k per load over the four
// lane groups); decoded to fp16 in registers (scale * q, one rounding) and
// run on MFMA f16 against the activations converted once to fp16.
template <int NW, int KBW, bool PACKED>
__device__ __forceinline__ void load_lm_q8(uint4 (&w)[2 * KBW], uint32_t (&sc)[2 * KBW],
                                           const uint8_t* lm, int vocab, int t, int r, int kbeg,
                                           int g) {
  const size_t qbytes = static_cast<size_t>(vocab) * H;
  const size_t row = static_cast<size_t>(t) * 16 + r;
#pragma unroll
  for (int i = 0; i < 2 * KBW; ++i) {
    if constexpr (PACKED) {
      const size_t pc = static_cast<size_t>(t) * (H / 64) + kbeg / 64 + i;
      w[i] = ld16_stream(reinterpret_cast<const uint16_t*>(lm + (pc * 64 + r + 16 * g) * 16));
      sc[i] = *reinterpret_cast<const uint16_t*>(lm + qbytes + 2 * (pc * 32 + r * 2 + (g >> 1)));
    } else {
      const size_t k = static_cast<size_t>(kbeg) + 64 * i + 16 * g;
      w[i] = ld16_stream(reinterpret_cast<const uint16_t*>(lm + row * H + k));
      sc[i] = *reinterpret_cast<const uint16_t*>(lm + qbytes + 2 * (row * (H / 32) + k / 32));
    }
  }
}

template <int KBW>
__device__ __forceinline__ f32x4 mma_chain_q8(const uint4 (&w)[2 * KBW],
                                              const uint32_t (&sc)[2 * KBW],
                                              const uint4 (&x)[4 * KBW]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 2 * KBW; ++i) {
    const h2 s2 = scale_h2(sc[i]);
    acc = mfma_f16(dq8(w[i].x, w[i].y, s2), x[2 * i], acc);
    acc = mfma_f16(dq8(w[i].z, w[i].w, s2), x[2 * i + 1], acc);
  }
  return acc;
}

template <int NW, int KBW, bool PACKED>
__global__ __launch_bounds__(NW * 64) void k_lmhead_q8(const uint8_t* lm, int ntiles, int vocab,
                                                       const uint16_t* z, int B, uint64_t* keys,
                                                       uint16_t* logits) {
  __shared__ f32x4 red[2][NW - 1][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const bool xv = r < B;
  const int kbeg = wave * (KBW * 128);
  uint4 x[4 * KBW];
  const uint16_t* xrow = z + static_cast<size_t>(xv ? r : 0) * H;
#pragma unroll
  for (int i = 0; i < 4 * KBW; ++i)
    x[i] = xv ? bf16x8_to_f16(ld16(xrow + kbeg + xslot<W_Q8_0>(i, g))) : make_uint4(0, 0, 0, 0);
  uint64_t best = 0;
  const int step = gridDim.x;
  int t = blockIdx.x;
  uint4 wa[2 * KBW], wb[2 * KBW];
  uint32_t sa[2 * KBW], sb[2 * KBW];
  if (t < ntiles) load_lm_q8<NW, KBW, PACKED>(wa, sa, lm, vocab, t, r, kbeg, g);
  int parity = 0;
  while (t < ntiles) {
    const int tn = t + step;
    if (tn < ntiles) load_lm_q8<NW, KBW, PACKED>(wb, sb, lm, vocab, tn, r, kbeg, g);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 acc = mma_chain_q8<KBW>(wa, sa, x);
    if (wave > 0) red[parity][wave - 1][lane] = acc;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < NW - 1; ++w) acc += red[parity][w][lane];
      lm_epilogue(acc, t * 16, r, g, xv, vocab, logits, best);
    }
    parity ^= 1;
    t = tn;
    if (t >= ntiles) break;
    const int tn2 = t + step;
    if (tn2 < ntiles) load_lm_q8<NW, KBW, PACKED>(wa, sa, lm, vocab, tn2, r, kbeg, g);
    __builtin_amdgcn_sched_barrier(0);
    acc = mma_chain_q8<KBW>(wb, sb, x);
    if (wave > 0) red[parity][wave - 1][lane] = acc;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < NW - 1; ++w) acc += red[parity][w][lane];
      lm_epilogue(acc, t * 16, r, g, xv, vocab, logits, best);
    }
    parity ^= 1;
    t = tn2;
  }
  if (wave == 0) {
    best = umax64(best, shfl_xor_u64(best, 16));
    best = umax64(best, shfl_xor_u64(best, 32));
    if (g == 0 && xv) keys[static_cast<size_t>(blockIdx.x) * MAXB + r] = best;
  }
}

// cand[b] = index part of the largest key over all blocks; wave b takes row b.
__global__ __launch_bounds__(MAXB * 64) void k_argmax_reduce(const uint64_t* keys, int nblk,
                                                             int B, int32_t* cand) {
  const int b = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (b >= B) return;
  uint64_t best = 0;
  constexpr int U = 16;
  for (int i0 = lane; i0 < nblk; i0 += 64 * U) {
    uint64_t k[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + 64 * u;
      k[u] = i < nblk ? keys[static_cast<size_t>(i) * MAXB + b] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) best = umax64(best, k[u]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) best = umax64(best, shfl_xor_u64(best, o));
  if (lane == 0) cand[b] = static_cast<int32_t>(~static_cast<uint32_t>(best));
}

// accepted = longest prefix with cand == target; all loads issued at once.
// With `state` (the device-resident positions {p, anchor, n_commit}), the
// cycle advances: the accepted cells and the continuation token's position
// are committed by the next pass, p += a + 1, anchor = next, n_commit = a + 1.
__global__ void k_verify(const int32_t* cand, const int32_t* target, int kmax,
                         const int32_t* k_dev, int32_t* out, int64_t* state) {
  const int lane = threadIdx.x;
  // k from a device word (the confidence gate's count), clamped to [0, kmax]
  const int kd = k_dev ? *k_dev : kmax;
  const int k = kd < 0 ? 0 : (kd > kmax ? kmax : kd);
  const int c = lane < k ? cand[lane] : 0;
  const int t = lane <= k ? target[lane] : 0;
  const bool miss = lane < k && c != t;
  const uint64_t m = __ballot(miss || lane == k);
  const int a = __ffsll(static_cast<unsigned long long>(m)) - 1;  // first mismatch or k
  const int nxt = __shfl(t, a, 64);
  if (lane == 0) {
    out[0] = a;
    out[1] = nxt;
    if (state) {
      state[0] += a + 1;
      state[1] = nxt;
      state[2] = a + 1;
    }
  }
}

template <int NW, int KBW>
hipError_t launch_gemv_nw(const GemvArgs& a, hipStream_t st) {
  const dim3 grid(a.N / 16, a.S), block(NW * 64);
  if (a.packed) {
    switch (a.fmt) {
      case W_BF16: hipLaunchKernelGGL((k_gemv<W_BF16, NW, KBW, true>), grid, block, 0, st, a); break;
      case W_Q8_0: hipLaunchKernelGGL((k_gemv<W_Q8_0, NW, KBW, true>), grid, block, 0, st, a); break;
      case W_Q4_0: hipLaunchKernelGGL((k_gemv<W_Q4_0, NW, KBW, true>), grid, block, 0, st, a); break;
      case W_Q5_0: hipLaunchKernelGGL((k_gemv<W_Q5_0, NW, KBW, true>), grid, block, 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.fmt) {
      case W_BF16: hipLaunchKernelGGL((k_gemv<W_BF16, NW, KBW, false>), grid, block, 0, st, a); break;
      case W_Q8_0: hipLaunchKernelGGL((k_gemv<W_Q8_0, NW, KBW, false>), grid, block, 0, st, a); break;
      case W_Q4_0: hipLaunchKernelGGL((k_gemv<W_Q4_0, NW, KBW, false>), grid, block, 0, st, a); break;
      case W_Q5_0: hipLaunchKernelGGL((k_gemv<W_Q5_0, NW, KBW, false>), grid, block, 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const GemvArgs& a, hipStream_t st) {
  if (a.B < 1 || a.B > GEMV_ROWS || a.N % 16 || a.K % 128) return hipErrorInvalidValue;
  // Each wave takes 256 k and a block 5 waves (1280 k per block and split):
  // the fc GEMV runs in 10 k splits (1600 blocks), the Wk / Wv GEMV in 2 (640
  // blocks for 256 CUs).  On an 8-row commit, 10 waves in 5 splits were 1 us
  // slower for fc, and 4 waves x 640 k 2 us; one split of 10 waves was 1.2 us
  // slower for Wk / Wv.
  constexpr int NW = 5, KBW = 2;
  if (a.S < 1 || a.K != a.S * 128 * NW * KBW) return hipErrorInvalidValue;
  return launch_gemv_nw<NW, KBW>(a, st);
}

hipError_t launch_dequant_bf16(const void* src, int fmt, int rows, int K, uint16_t* dst, int row0,
                               bool packed, hipStream_t st) {
  if (rows < 0 || K % 32 || rows % 16 || row0 % 16 || row0 < 0) return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  const size_t n8 = static_cast<size_t>(rows) * K / 8;
  const int grid = static_cast<int>(n8 / 256 < 4096 ? (n8 + 255) / 256 : 4096);
  const uint8_t* s8 = static_cast<const uint8_t*>(src);
  if (packed && (K % (fmt == W_Q8_0 ? 64 : 128))) return hipErrorInvalidValue;
  if (fmt == W_Q8_0 && packed)
    hipLaunchKernelGGL((k_dequant_bf16<W_Q8_0, true>), dim3(grid), dim3(256), 0, st, s8, rows, K, dst, row0);
  else if (fmt == W_Q8_0)
    hipLaunchKernelGGL((k_dequant_bf16<W_Q8_0, false>), dim3(grid), dim3(256), 0, st, s8, rows, K, dst, row0);
  else if (fmt == W_Q4_0 && packed)
    hipLaunchKernelGGL((k_dequant_bf16<W_Q4_0, true>), dim3(grid), dim3(256), 0, st, s8, rows, K, dst, row0);
  else if (fmt == W_Q4_0)
    hipLaunchKernelGGL((k_dequant_bf16<W_Q4_0, false>), dim3(grid), dim3(256), 0, st, s8, rows, K, dst, row0);
  else if (fmt == W_Q5_0 && packed)
    hipLaunchKernelGGL((k_dequant_bf16<W_Q5_0, true>), dim3(grid), dim3(256), 0, st, s8, rows, K, dst, row0);
  else if (fmt == W_Q5_0)
    hipLaunchKernelGGL((k_dequant_bf16<W_Q5_0, false>), dim3(grid), dim3(256), 0, st, s8, rows, K, dst, row0);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_lmhead_argmax(const void* lm, int fmt, bool packed, int vocab, const uint16_t* z,
                                int B, uint64_t* keys, int grid, uint16_t* logits_opt,
                                int32_t* cand, hipStream_t st) {
  if (B < 1 || B > MAXB || vocab % 16) return hipErrorInvalidValue;
  const int ntiles = vocab / 16;
  if (grid > ntiles) grid = ntiles;
  const uint16_t* l16 = static_cast<const uint16_t*>(lm);
  const uint8_t* l8 = static_cast<const uint8_t*>(lm);
  if (fmt == W_BF16 && packed)
    hipLaunchKernelGGL((k_lmhead_bf16<4, 5, true>), dim3(grid), dim3(256), 0, st, l16, ntiles, vocab,
                       z, B, keys, logits_opt);
  else if (fmt == W_BF16)
    hipLaunchKernelGGL((k_lmhead_bf16<4, 5, false>), dim3(grid), dim3(256), 0, st, l16, ntiles, vocab,
                       z, B, keys, logits_opt);
  else if (fmt == W_Q8_0 && packed)
    hipLaunchKernelGGL((k_lmhead_q8<4, 5, true>), dim3(grid), dim3(256), 0, st, l8, ntiles, vocab,
                       z, B, keys, logits_opt);
  else if (fmt == W_Q8_0)
    hipLaunchKernelGGL((k_lmhead_q8<4, 5, false>), dim3(grid), dim3(256), 0, st, l8, ntiles, vocab,
                       z, B, keys, logits_opt);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_argmax_reduce, dim3(1), dim3(MAXB * 64), 0, st, keys, grid, B, cand);
  return hipGetLastError();
}

hipError_t launch_verify(const int32_t* cand, const int32_t* target, int k, const int32_t* k_dev,
                         int32_t* out, int64_t* state, hipStream_t st) {
  hipLaunchKernelGGL(k_verify, dim3(1), dim3(64), 0, st, cand, target, k, k_dev, out, state);
  return hipGetLastError();
}

}  // namespace dfl
