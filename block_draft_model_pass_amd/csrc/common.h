// Device helpers and internal launch interfaces of the DFlash HIP library.
// gfx950 (CDNA4) only: 64-lane wavefronts, MFMA 16x16x32 bf16/fp16.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dfl {

// Fixed geometry (Strata PR #1426 page, "Drafter runtime").
constexpr int H = 2560;          // hidden
constexpr int L = 5;             // layers
constexpr int NQ = 24;           // query heads
constexpr int NKV = 2;           // key/value heads
constexpr int G = NQ / NKV;      // query heads per KV head (12)
constexpr int D = 256;           // head dim
constexpr int F = 7680;          // MLP width
constexpr int T = 5;             // target taps
constexpr int QKV_N = NQ * D + 2 * NKV * D;  // 7168 fused q|k|v rows
constexpr int KV_N = L * 2 * NKV * D;        // 5120 rows of [Wk_l; Wv_l] x 5
constexpr int MAXB = 8;          // max block rows
constexpr int GEMV_ROWS = 16;    // max activation rows of one skinny GEMV
constexpr int BLK_CELLS = 32;    // cells of the block-key buffer

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- numbers

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = static_cast<_Float16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// Order-preserving map of a finite fp32 to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t f32_order_key(float v) {
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// argmax key: value in the high word, inverted index in the low word, so
// that an unsigned max picks the largest value and, among equal values, the
// lowest index.
__device__ __forceinline__ uint64_t argmax_key(float v, uint32_t idx) {
  return (static_cast<uint64_t>(f32_order_key(v)) << 32) | static_cast<uint64_t>(~idx);
}

// ---------------------------------------------------------------- MFMA

// D[16][16] += A[16][32] * B[32][16].  Lane l supplies row (l % 16) of A and
// column (l % 16) of B, 8 consecutive k values each (the same k slots for A
// and B); it receives D rows 4*(l/16) .. 4*(l/16)+3 of column l % 16.
__device__ __forceinline__ f32x4 mfma_bf16(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// D[16][16] += A[16][16] * B[16][16]: the same lane layout with 4 k values
// per lane (k slots 4*(l/16) .. +3).
__device__ __forceinline__ f32x4 mfma_f16_k16(const uint2& a, const uint2& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c,
                                               0, 0, 0);
}

// ---------------------------------------------------------------- reductions

// Cross-lane reductions without LDS traffic (a lane shuffle is an LDS
// instruction, ~100 cycles per step).  v_permlane32_swap and
// v_permlane16_swap exchange the wave's halves / the rows of each row pair:
// their two results combined give op(v(l), v(l ^ 32)) and op(v(l), v(l ^ 16))
// in every lane.  DPP row rotations by 8, 4, 2 and 1 take the lane bits
// below 16: once the higher bits are reduced, lane (l +- 2^k) mod 16 holds
// the same bits as lane l ^ 2^k.  Every step therefore combines the same two
// values, in the same order of steps, as an xor-shuffle reduction over
// 32, 16, 8, 4, 2, 1 -- the results are bit-identical to it.  All 64 lanes
// must be active.
__device__ __forceinline__ uint2 swap32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return make_uint2(r[0], r[1]);
}
__device__ __forceinline__ uint2 swap16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return make_uint2(r[0], r[1]);
}
template <int CTRL>
__device__ __forceinline__ float dpp_rot(float v) {  // CTRL: row_ror by 1, 2, 4, 8 = 0x121, 0x122, 0x124, 0x128
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v) {
  uint2 p = swap32(v);
  v = __uint_as_float(p.x) + __uint_as_float(p.y);
  p = swap16(v);
  v = __uint_as_float(p.x) + __uint_as_float(p.y);
  v += dpp_rot<0x128>(v);
  v += dpp_rot<0x124>(v);
  v += dpp_rot<0x122>(v);
  v += dpp_rot<0x121>(v);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  uint2 p = swap32(v);
  v = fmaxf(__uint_as_float(p.x), __uint_as_float(p.y));
  p = swap16(v);
  v = fmaxf(__uint_as_float(p.x), __uint_as_float(p.y));
  v = fmaxf(v, dpp_rot<0x128>(v));
  v = fmaxf(v, dpp_rot<0x124>(v));
  v = fmaxf(v, dpp_rot<0x122>(v));
  v = fmaxf(v, dpp_rot<0x121>(v));
  return v;
}

// Sum over the 4 lanes l, l^16, l^32, l^48 (the four k-groups of an MFMA column).
__device__ __forceinline__ float group4_sum(float v) {
  uint2 p = swap16(v);
  v = __uint_as_float(p.x) + __uint_as_float(p.y);
  p = swap32(v);
  return __uint_as_float(p.x) + __uint_as_float(p.y);
}

__device__ __forceinline__ float group4_max(float v) {
  uint2 p = swap16(v);
  v = fmaxf(__uint_as_float(p.x), __uint_as_float(p.y));
  p = swap32(v);
  return fmaxf(__uint_as_float(p.x), __uint_as_float(p.y));
}

// Block-wide sum for blockDim.x == NT (multiple of 64); all threads get it.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* scratch /* [NT/64] */) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) scratch[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += scratch[i];
  __syncthreads();
  return s;
}

// ---------------------------------------------------------------- launches

// Row segments of one logical weight matrix stored in several buffers,
// concatenated along the output dimension.  Every segment's row count is a
// multiple of 128, so a 16- or 128-row tile never straddles two segments.
struct SegTable {
  const void* ptr[10];
  int row_end[10];   // cumulative
  int nseg;
};

enum WFormat { W_BF16 = 0, W_Q8_0 = 1, W_Q4_0 = 2, W_Q5_0 = 3 };

// Formats whose 64-byte quant pieces cover 128 k (nibbles).
constexpr bool nibble_fmt(int fmt) { return fmt == W_Q4_0 || fmt == W_Q5_0; }

// ---------------------------------------------------------------- quantized weights
// Q8_0 / Q4_0 / Q5_0 blocks (32 consecutive input-dim weights of one output
// row share an fp16 scale) are decoded to fp16 in registers.  The integer
// (q, nibble - 8, or 5-bit code - 16) is exact in fp16; the only rounding is
// that of q * scale (relative 2^-11).  A decoded group is the 8
// fp16 values one lane feeds to one MFMA 16x16x32 f16.

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Bytes 2j, 2j+1 of x as the fp16 pair (1024 + byte): 0x64 is the high byte
// of fp16 1024, so a byte in the low mantissa bits is added exactly.  One
// byte permute: selector bytes 0-3 pick from x, 4 picks 0x64.
__device__ __forceinline__ uint32_t u8pair_f16(uint32_t x, int j) {
  return __builtin_amdgcn_perm(0x64646464u, x, j ? 0x04030402u : 0x04010400u);
}

__device__ __forceinline__ uint32_t dq_pair(uint32_t t, h2 off, h2 s) {
  h2 v = __builtin_bit_cast(h2, t) - off;  // exact small integers
  v = v * s;                               // one rounding
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ h2 scale_h2(uint32_t s16) {
  return __builtin_bit_cast(h2, (s16 & 0xffffu) | (s16 << 16));
}

// Q8_0: 8 int8 (w0 bytes then w1 bytes, element order kept) times s.
__device__ __forceinline__ uint4 dq8(uint32_t w0, uint32_t w1, h2 s) {
  const h2 off = {static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
  const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;  // q + 128
  return make_uint4(dq_pair(u8pair_f16(u0, 0), off, s), dq_pair(u8pair_f16(u0, 1), off, s),
                    dq_pair(u8pair_f16(u1, 0), off, s), dq_pair(u8pair_f16(u1, 1), off, s));
}

// Q4_0: the low (hi = false) or high nibbles of the 8 bytes w0, w1 times s.
// Byte j of a block holds element j (low nibble) and element j + 16 (high).
__device__ __forceinline__ uint4 dq4(uint32_t w0, uint32_t w1, bool hi, h2 s) {
  const h2 off = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
  const uint32_t n0 = (hi ? w0 >> 4 : w0) & 0x0f0f0f0fu;
  const uint32_t n1 = (hi ? w1 >> 4 : w1) & 0x0f0f0f0fu;
  return make_uint4(dq_pair(u8pair_f16(n0, 0), off, s), dq_pair(u8pair_f16(n0, 1), off, s),
                    dq_pair(u8pair_f16(n1, 0), off, s), dq_pair(u8pair_f16(n1, 1), off, s));
}

// Q5_0: the low (hi = false) or high nibbles of the 8 bytes w0, w1 with
// their fifth bits hb0 / hb1 already at bits 4, 12, 20, 28 (one per byte),
// minus 16, times s.
__device__ __forceinline__ uint4 dq5(uint32_t w0, uint32_t w1, bool hi, uint32_t hb0, uint32_t hb1,
                                     h2 s) {
  const h2 off = {static_cast<_Float16>(1040.0f), static_cast<_Float16>(1040.0f)};
  const uint32_t n0 = ((hi ? w0 >> 4 : w0) & 0x0f0f0f0fu) | hb0;
  const uint32_t n1 = ((hi ? w1 >> 4 : w1) & 0x0f0f0f0fu) | hb1;
  return make_uint4(dq_pair(u8pair_f16(n0, 0), off, s), dq_pair(u8pair_f16(n0, 1), off, s),
                    dq_pair(u8pair_f16(n1, 0), off, s), dq_pair(u8pair_f16(n1, 1), off, s));
}

// Fifth bits of elements 4 C .. 4 C + 3 of a Q5_0 block at bits 4, 12, 20,
// 28, from the block's word in the streaming copy, where the bit of element
// 4 C + c sits at bit C + 8 c (one shift and a mask) ...
template <int C>
__device__ __forceinline__ uint32_t q5_bits_packed(uint32_t hw) {
  if constexpr (C <= 4) return (hw << (4 - C)) & 0x10101010u;
  else return (hw >> (C - 4)) & 0x10101010u;
}

// ... or from the row-major word (bit j = element j): the nibble t of bits
// 4 C .. 4 C + 3 spread to one bit per byte (t * 0x204081 puts bit i of t at
// bit 8 i, no carries since the four copies do not overlap).
template <int C>
__device__ __forceinline__ uint32_t q5_bits_rowmajor(uint32_t hw) {
  const uint32_t t = (hw >> (4 * C)) & 0xfu;
  return ((t * 0x00204081u) & 0x01010101u) << 4;
}

// Activation element in the MFMA input format of a weight format: bf16 next
// to bf16 weights, fp16 next to decoded quantized weights.
template <int FMT>
__device__ __forceinline__ uint16_t act16(float v) {
  if constexpr (FMT == W_BF16) return f32_to_bf16(v);
  else return f32_to_f16_bits(v);
}

// y[s][b][n] = sum over split s of k of W[n][k] * x[b][k]   (b < B <= 16)
struct GemvArgs {
  SegTable w;
  int fmt;               // WFormat
  int N, K;
  const uint16_t* x;     // bf16 [B][x_stride]
  int x_stride;
  int B;
  float* out;            // fp32 [S][B][N]
  int S;
  int packed;            // segments are streaming copies (16-row tiles, lane order)
};

hipError_t launch_gemv(const GemvArgs& a, hipStream_t st);

// bf16 [N][K] -> streaming copy (16-row tiles, 32-wide k blocks, MFMA lane
// order, 16 bytes per lane); element (r, k) lands at
// ((r/16 * K/32 + k/32) * 64 + r%16 + 16 * (k%32 / 8)) * 8 + k%8.
hipError_t launch_pack_bf16(const void* src, int N, int K, void* dst, hipStream_t st);
// Units of `unit` (4 or 8) bytes of an [N][per_row] array regrouped as 16-row
// tiles x per_row x 16 rows (the block scales of a packed quantized matrix).
hipError_t launch_pack_units(const void* src, int N, int per_row, int unit, void* dst,
                             hipStream_t st);
// Q5_0 high-bit words of an [N][per_row * 4] array (one word per 32-element
// block, bit j = element j) regrouped as 16-row tiles x per_row x 16 rows of
// 16-byte units, each word's bits reordered: element 8 a + 4 b + c at bit
// 2 a + b + 8 c.
hipError_t launch_pack_q5_bits(const void* src, int N, int per_row, void* dst, hipStream_t st);

// Quantized [rows][K] matrix (fmt Q8_0 / Q4_0 / Q5_0) -> rows row0 .. row0+rows-1
// of a bf16 [.][K] matrix in the streaming layout (rows, row0 multiples of 16).
// src: row-major blocks, or the matrix's streaming copy when `packed`.
hipError_t launch_dequant_bf16(const void* src, int fmt, int rows, int K, uint16_t* dst, int row0,
                               bool packed, hipStream_t st);

// LM head + greedy argmax over the vocabulary.
// lm: [vocab][2560] in format fmt (bf16 or Q8_0 blocks), row-major or its
// streaming copy when `packed`.
hipError_t launch_lmhead_argmax(const void* lm, int fmt, bool packed, int vocab, const uint16_t* z,
                                int B, uint64_t* keys, int grid, uint16_t* logits_opt,
                                int32_t* cand, hipStream_t st);

// Row RMSNorm: v = (h ? h[b] : 0) + sum_s part[s][b]; if h, h[b] = v;
// out[b] = bf16(v * rsqrt(mean(v^2) + eps) * gain); out2 (optional) the same.
hipError_t launch_rownorm(float* h, const float* part, int S, size_t part_split_stride,
                          int part_row_stride, int rows, const uint16_t* gain, float eps,
                          uint16_t* out, int out_stride, uint16_t* out2, hipStream_t st);

// Context K/V epilogue: y [n][KV_N] (row stride ldy; nsplit = 2: the sum of
// two k-split partials, the second split_stride floats after the first) ->
// k-norm + RoPE + fp16 into the ring.
hipError_t launch_kv_post(const float* y, int ldy, int nsplit, size_t split_stride, int n,
                          int64_t pos0, const void* const* k_norms, float eps, double theta,
                          uint16_t* ring_k, uint16_t* ring_vt, int capacity, hipStream_t st);

// C[M][N] (fp32, ldc) = A[M][K] (bf16, lda) * W[N][K]^T
// w_packed: the segments point at streaming copies of the bf16 matrices
// (16-row tiles x 32-wide k blocks in MFMA lane order) instead of row-major ones.
hipError_t launch_gemm_bf16(const uint16_t* A, int lda, int M, const SegTable& w, bool w_packed, int K,
                            float* C, int ldc, int N, int nsplit, size_t c_split, hipStream_t st);

// RoPE table of n consecutive positions pos0 ..: tab[row][i] = (cos, sin) of
// (pos0 + row) * theta^(-2i/256), i < 128, computed in fp64 and rounded to
// fp32 (the angles of the context keys).
hipError_t launch_rope_rows(float2* tab, int64_t pos0, int n, double theta, hipStream_t st);

// Context K/V projection with the cells as the GEMM's epilogue: for the
// [Wk_0; Wv_0; ...; Wk_4; Wv_4] weights (N = 5120, K = 2560) each 256-column
// tile is one head of one layer; key tiles get the per-head k-norm and RoPE
// (rope: launch_rope_rows of pos0), value tiles are transposed into the
// ring's 32-cell blocks; both in fp16, row m into cell (pos0 + m) % capacity.
struct KvEpi {
  uint16_t* ring_k;
  uint16_t* ring_vt;
  int cap;
  int64_t pos0;
  const float2* rope;
  const uint16_t* kg[L];   // k-norm gains (bf16)
  float eps;
};
hipError_t launch_gemm_kv_bf16(const uint16_t* A, int lda, int M, const SegTable& w, bool w_packed,
                               const KvEpi& kv, hipStream_t st);

// Finite check: *status = 0, then `code` if any of x[0..count) (dtype 0 bf16,
// 1 fp16, 2 fp32; 16-byte aligned) is NaN or infinite.
hipError_t launch_check_finite(const void* x, int64_t count, int dtype, int32_t* status, int32_t code,
                               hipStream_t st);

// The whole proposal pass as one persistent kernel (plus a small init kernel).
struct PassLaunch {
  int fmt;                 // WFormat of the layer matrices (bytes behind the pointers)
  int lm_fmt = W_BF16;     // WFormat of the LM head's streaming copy (bf16 or Q8_0)
  const uint16_t* wq[L];
  const uint16_t* wk[L];
  const uint16_t* wv[L];
  const uint16_t* wo[L];
  const uint16_t* wg[L];
  const uint16_t* wu[L];
  const uint16_t* wd[L];
  const uint16_t* in_norm[L];
  const uint16_t* q_norm[L];
  const uint16_t* k_norm[L];
  const uint16_t* post_norm[L];
  const uint16_t* final_norm;
  const uint16_t* embed;
  const uint16_t* lm;
  int vocab;
  float eps, scale_log2;
  double theta;
  const uint16_t* ring_k;    // layer 0 of the ring
  const uint16_t* ring_vt;
  int cap;
  int64_t lo, hi, p0;        // visible positions [lo, hi); first block position
  int nb, cb, nch;           // 32-cell blocks, blocks per chunk, chunks
  int B;
  int64_t p;
  int anchor, mask;
  float* h;
  uint16_t* h16;
  float* ss;
  uint16_t* qkv;           // fp16 [5][8][7168]
  float2* rope;             // [16][128]
  uint16_t* po;            // chunk outputs, fp16, normalised by the chunk sum
  float* pm;
  float* pl;
  uint16_t* o16;
  uint16_t* u16;
  uint64_t* keys;
  uint64_t* lse;             // [grid][8] softmax (max, sum) pairs
  unsigned* bar;
  void* tab;                 // workspace room for the per-layer pointer table
  uint64_t wait_ticks;       // grid-barrier wait bound in constant-clock ticks
  int grid;
  int32_t* cand;
  uint16_t* logits;
  uint16_t* hidden;
  // fused draft-commit cycle: nc commit rows of taps at positions pos0..pos0+nc-1
  const uint16_t* taps = nullptr;
  const void* fc = nullptr;  // streaming copy of fc (backbone format)
  const uint16_t* hidden_norm = nullptr;
  int nc = 0;
  int64_t pos0 = 0;
  float* yc = nullptr;       // [8][2560] fp32
  float* fcp = nullptr;      // FC-phase tile partials (pass_fcp_bytes)
  uint16_t* cn = nullptr;    // [8][2560] the commit rows' fused context (MFMA input format)
  float* ckv = nullptr;      // [5][8][1024] fp32
  float* conf = nullptr;     // [B-1] candidate probabilities, or null
  int32_t* nkeep = nullptr;  // confidence-gated candidate count, or null
  float min_p = 0.f;
  // Positions from device memory: with dstate set, p, the anchor and nc are
  // read from dstate[0..2] by the kernels and the fields above that derive
  // from them (lo, hi, p0, nb, cb, nch, pos0, taps) are ignored; the commit
  // taps are rows of taps_base, row r holding position taps_pos0 + r.
  const int64_t* dstate = nullptr;
  const uint16_t* taps_base = nullptr;
  int64_t taps_pos0 = 0, taps_rows = 0;
  int64_t window = 0;
  int maxch = 0;             // most chunks per KV head
};

hipError_t launch_draft_pass(const PassLaunch& q, hipStream_t st);
// Largest co-resident grid of the pass kernel on `device` (0 if it cannot run).
hipError_t draft_pass_max_grid(int device, int* grid);
size_t pass_po_bytes();   // attention chunk outputs, all layers
size_t pass_pml_bytes();  // chunk maxima (or sums), all layers
size_t pass_smem_bytes();
size_t pass_tab_bytes();
size_t pass_bar_bytes();
size_t pass_fcp_bytes();  // FC-phase tile partials of the fused draft-commit pass

// Greedy verify of k candidates, or of min(max(*k_dev, 0), k) when k_dev is
// set; with `state` ({p, anchor, n_commit}, int64) it also advances the
// device-resident positions.
hipError_t launch_verify(const int32_t* cand, const int32_t* target, int k, const int32_t* k_dev,
                         int32_t* out, int64_t* state, hipStream_t st);
// *status = timeout_code if the barrier words `bar` of the last pass record
// a wait that gave up, invalid_code if the pass found its device-resident
// positions invalid and did nothing, else 0.
hipError_t launch_pass_status(const unsigned* bar, int32_t* status, int32_t timeout_code,
                              int32_t invalid_code, hipStream_t st);
// Constant-clock ticks per microsecond on `device` (the counter the pass's
// barrier bound reads).
hipError_t wall_clock_ticks_per_us(int device, double* ticks);

}  // namespace dfl
