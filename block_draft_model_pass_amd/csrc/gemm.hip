// bf16 "NT" GEMM on MFMA for the long-context steps: context fusion
// (taps [n][12800] x fc^T) and the context K/V projection
// (ctx [n][2560] x [Wk_0; Wv_0; ...; Wk_4; Wv_4]^T).  Both operands are
// k-contiguous, which is the native operand layout of MFMA 16x16x32: a lane
// reads 8 consecutive k of one row of A and of one row of W.
//
// Block tile 256 x 256, 512 threads: 8 waves as 2 (m) x 4 (n), each owning a
// 128 x 64 sub-tile (8 x 4 MFMA tiles, 128 accumulators held in AGPRs).  Per
// 32-wide k step a wave reads 12 operand fragments (12 KiB) from LDS for 32
// MFMAs.
//
// k advances in 32-wide stages through a 5-deep LDS ring (32 KiB per stage,
// all 160 KiB of the CU's LDS) filled by direct buffer -> LDS loads (16 bytes
// per lane, no registers).  The fragments of a stage are read into one of two
// register sets while the MFMAs of the previous stage run from the other, so
// a stage's slot is free as soon as the rendezvous after its reads has
// passed and five stages are in flight while one is multiplied.  The MFMAs
// of a step start right after its rendezvous; the next stage's reads and the
// refill loads go out in two halves between groups of 16 MFMAs.  Stage rows
// are 64 bytes (32 bf16); 16-byte chunk c of row r sits at chunk
// c ^ ((r >> 1) & 3), which keeps the 16-row fragment reads free of bank
// conflicts (measured); each load instruction fills 1 KiB of LDS (16 rows) in
// lane order, so a lane fetches the global chunk that the swizzle places at
// its slot.
//
// With the streaming copies of the bf16 weights present, W comes from them:
// each W load is one contiguous 1 KiB block (8 cache lines instead of 16
// row pieces of 64 bytes) and W fragments are read without a swizzle
// (measured: fusion 1.85 -> 1.75 ms, projection 1.02 -> 0.98 ms).
//
// Tiles are dealt to the XCDs in contiguous runs (the hardware deals blocks
// round robin), so the blocks on one XCD share A panels in its L2.  With
// fewer tiles than CUs the k range can be split S ways (partial outputs S
// apart, summed by the consumer).
#include "common.h"
#include "fuse.h"

namespace dfl {

namespace {

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int NT = 512;
constexpr int STAGES = 5;
constexpr int STAGE_ELEMS = (BM + BN) * BK;  // bf16 per stage: A rows then W rows

// Measured on gfx950 (SQ_LDS_BANK_CONFLICT of single-wave ds_read_b128
// patterns): with 64-byte rows, 16 rows x one chunk per lane group read
// conflict-free when chunk c of row r sits at c ^ ((r >> 1) & 3); the same
// read is 2-way conflicted unswizzled or with c ^ (r & 3).
__device__ __forceinline__ int kswz(int row) { return (row >> 1) & 3; }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// LDS byte address of a __shared__ element.
__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint16_t*)p));
}

// Fragment read issued as its own instruction, at a byte offset the
// instruction carries: the compiler's wait-count pass cannot tell which stage
// a plain LDS read touches and would wait for every direct-to-LDS load in
// flight, serialising the stages.  The caller waits with lds_wait_all before
// using the value.
template <int OFF>
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF) : "memory");
  return v;
}

// Wait for all of this wave's LDS reads; the 12 fragments pass through the
// statement, so nothing that uses them is scheduled before the wait and no
// copy of a register still being loaded is taken.
__device__ __forceinline__ void lds_wait_all(u32x4 (&w)[4], u32x4 (&a)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(a[0]), "+v"(a[1]),
                 "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]), "+v"(a[7])
               :
               : "memory");
}

// Stage base + lane offset, computed where it is used (a plain add would be
// hoisted out of the loop as ten live registers, one per stage and operand).
__device__ __forceinline__ uint32_t lds_base(uint32_t stage, uint32_t lane_off) {
  uint32_t a;
  asm volatile("v_add_u32 %0, %1, %2" : "=v"(a) : "s"(stage), "v"(lane_off));
  return a;
}

__device__ __forceinline__ uint4 as_uint4(u32x4 v) { return __builtin_bit_cast(uint4, v); }

// LDS element offset of chunk c of stage row `row` (A rows 0..255, W rows 256..511).
__device__ __forceinline__ int lds_off(int row, int c) { return row * BK + ((c ^ kswz(row)) << 3); }

// ---------------------------------------------------------------- K/V epilogue
//
// A tile of the K/V projection is 256 positions x one head (256 dims) of one
// layer: columns n0 .. n0+255 of [Wk_0; Wv_0; ...] are layer n0 / 1024, keys
// for (n0 % 1024) < 512, head (n0 % 512) / 256.  Once the k loop is done the
// stage ring is free: each half of the tile (the 128 rows of the waves with
// wm = h) goes through four stage arrays as fp32 [32 rows][256] each (16-float
// groups XOR-swizzled by (row / 4) % 4, so the accumulator writes of the four
// lane groups hit different banks), then
//  - keys: 32 threads per row, thread p holding the NeoX pairs 4p .. 4p+3
//    (dims 4p.. and 128 + 4p..): sum of squares, 32-lane reduction, scale
//    with the k gain, rotation by the row's (cos, sin) from the table, fp16;
//    the same operations in the same order as the stand-alone K/V epilogue
//    kernel, with the fused multiply-adds written out in both, so the cells
//    are the same bits;
//  - values: thread (dim d, group) reads the 32 cells of an aligned 32-cell
//    group and writes the group's 64 contiguous bytes of the ring's value
//    block (cells of groups that straddle a half or the tile one by one).
// Every row of A is one position, pos0 + row; rows past M are not stored.

// Row `row` (0..127) of the staged half: array row / 32, row row % 32.
__device__ __forceinline__ float* half_row(uint16_t* s0, uint16_t* s1, uint16_t* s2, uint16_t* s3,
                                           int row) {
  const int q = row >> 5;
  uint16_t* a = q == 0 ? s0 : (q == 1 ? s1 : (q == 2 ? s2 : s3));
  return reinterpret_cast<float*>(a) + (row & 31) * 256;
}
__device__ __forceinline__ int half_col(int row, int col) { return col ^ (((row >> 2) & 3) << 4); }

__device__ __forceinline__ void kv_epilogue(const f32x4 (&acc)[8][4], uint16_t* st0, uint16_t* st1,
                                            uint16_t* st2, uint16_t* st3, int m0, int n0, int M,
                                            int wm, int wn, int r, int g, int tid, const KvEpi& kv) {
  constexpr int LW = 2 * NKV * D;  // 1024 columns per layer
  const int l = n0 / LW, kind = (n0 % LW) / (NKV * D), j = (n0 % (NKV * D)) / D;
  const size_t head = static_cast<size_t>(l) * NKV + j;
  __syncthreads();  // no wave reads the stage ring any more
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = i * 16 + 4 * g + e;
          float* pr = half_row(st0, st1, st2, st3, row);
#pragma unroll
          for (int jn = 0; jn < 4; ++jn) pr[half_col(row, wn * 64 + jn * 16 + r)] = acc[i][jn][e];
        }
    }
    __syncthreads();
    const int r0 = m0 + h * 128;                       // row of A of the half's row 0
    const int nvalid = M - r0 < 128 ? M - r0 : 128;    // rows of A in this half
    if (kind == 0) {
      const int p = tid & 31, rs = tid >> 5;           // 16 rows per round
      const uint16_t* gk = kv.kg[l];
      const uint2 gl = *reinterpret_cast<const uint2*>(gk + 4 * p);
      const uint2 gh = *reinterpret_cast<const uint2*>(gk + D / 2 + 4 * p);
      const float ga[4] = {bf16_to_f32(static_cast<uint16_t>(gl.x)), bf16_to_f32(static_cast<uint16_t>(gl.x >> 16)),
                           bf16_to_f32(static_cast<uint16_t>(gl.y)), bf16_to_f32(static_cast<uint16_t>(gl.y >> 16))};
      const float gc[4] = {bf16_to_f32(static_cast<uint16_t>(gh.x)), bf16_to_f32(static_cast<uint16_t>(gh.x >> 16)),
                           bf16_to_f32(static_cast<uint16_t>(gh.y)), bf16_to_f32(static_cast<uint16_t>(gh.y >> 16))};
#pragma unroll 4
      for (int it = 0; it < 8; ++it) {
        const int row = it * 16 + rs;
        const bool valid = row < nvalid;
        const int ra = valid ? r0 + row : 0;           // in-bounds table row for unused rows
        const float4 cs01 = *reinterpret_cast<const float4*>(kv.rope + static_cast<size_t>(ra) * (D / 2) + 4 * p);
        const float4 cs23 = *reinterpret_cast<const float4*>(kv.rope + static_cast<size_t>(ra) * (D / 2) + 4 * p + 2);
        const float fc[4] = {cs01.x, cs01.z, cs23.x, cs23.z}, fs[4] = {cs01.y, cs01.w, cs23.y, cs23.w};
        const float* pr = half_row(st0, st1, st2, st3, row);
        const f32x4 lo = *reinterpret_cast<const f32x4*>(pr + half_col(row, 4 * p));
        const f32x4 hi = *reinterpret_cast<const f32x4*>(pr + half_col(row, D / 2 + 4 * p));
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) ss += fmaf(hi[k], hi[k], lo[k] * lo[k]);
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        ss += __shfl_xor(ss, 4);
        ss += __shfl_xor(ss, 8);
        ss += __shfl_xor(ss, 16);
        const float sc = 1.0f / sqrtf(ss / static_cast<float>(D) + kv.eps);
        uint32_t olo[2], ohi[2];
#pragma unroll
        for (int k = 0; k < 4; k += 2) {
          float a[2], cc[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float x = lo[k + e] * (sc * ga[k + e]), z = hi[k + e] * (sc * gc[k + e]);
            a[e] = fmaf(x, fc[k + e], -(z * fs[k + e]));
            cc[e] = fmaf(z, fc[k + e], x * fs[k + e]);
          }
          olo[k / 2] = f32_to_f16_bits(a[0]) | (static_cast<uint32_t>(f32_to_f16_bits(a[1])) << 16);
          ohi[k / 2] = f32_to_f16_bits(cc[0]) | (static_cast<uint32_t>(f32_to_f16_bits(cc[1])) << 16);
        }
        if (valid) {
          const size_t cell = static_cast<size_t>((kv.pos0 + r0 + row) % kv.cap);
          uint16_t* k = kv.ring_k + (head * kv.cap + cell) * D + 4 * p;
          *reinterpret_cast<uint2*>(k) = make_uint2(olo[0], olo[1]);
          *reinterpret_cast<uint2*>(k + D / 2) = make_uint2(ohi[0], ohi[1]);
        }
      }
    } else if (nvalid > 0) {
      const int d = tid & (D - 1), gsel = tid >> 8;    // 2 groups per round
      const int64_t P0 = kv.pos0 + r0;                 // position of the half's row 0
      const int64_t g0 = P0 / BLK_CELLS;
      const int ngr = static_cast<int>((P0 + nvalid - 1) / BLK_CELLS - g0 + 1);
      uint16_t* vcol = kv.ring_vt + head * D * kv.cap + static_cast<size_t>(d) * BLK_CELLS;
      for (int gi = gsel; gi < ngr; gi += 2) {
        const int64_t gp = (g0 + gi) * BLK_CELLS;      // position of the group's cell 0
        const int rb = static_cast<int>(gp - P0);      // its row in the half (may be < 0)
        uint16_t* v = vcol + static_cast<size_t>((gp % kv.cap) / BLK_CELLS) * (D * BLK_CELLS);
        if (rb >= 0 && rb + BLK_CELLS <= nvalid) {
          uint32_t o[BLK_CELLS / 2];
#pragma unroll
          for (int c = 0; c < BLK_CELLS; c += 2) {
            const int ra = rb + c, rc = rb + c + 1;
            const float v0 = half_row(st0, st1, st2, st3, ra)[half_col(ra, d)];
            const float v1 = half_row(st0, st1, st2, st3, rc)[half_col(rc, d)];
            o[c / 2] = f32_to_f16_bits(v0) | (static_cast<uint32_t>(f32_to_f16_bits(v1)) << 16);
          }
          uint4* v4 = reinterpret_cast<uint4*>(v);
#pragma unroll
          for (int q = 0; q < 4; ++q) v4[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
        } else {
          for (int c = 0; c < BLK_CELLS; ++c) {
            const int row = rb + c;
            if (row >= 0 && row < nvalid) v[c] = f32_to_f16_bits(half_row(st0, st1, st2, st3, row)[half_col(row, d)]);
          }
        }
      }
    }
    __syncthreads();  // the half's stage arrays are free again
  }
}

// Fused context rows (EPI = 2): the two 128-row halves of the tile go
// through the stage ring as fp32, as in kv_epilogue; then each wave takes one
// row per round: its 64 lanes read the row's 256 values (16 bytes each; the
// swizzle keeps a lane's 4 columns together), write them as bf16 (512
// contiguous bytes) and reduce the row's sum of squares over the tile, from
// the fp32 values, into ss[row][n0 / 256].  Rows past M are not stored.
__device__ __forceinline__ void fuse_epilogue(const f32x4 (&acc)[8][4], uint16_t* st0, uint16_t* st1,
                                              uint16_t* st2, uint16_t* st3, int m0, int n0, int M,
                                              int wm, int wave, int lane, int r, int g, const FuseEpi& fe) {
  const int wn = wave & 3;
  __syncthreads();  // no wave reads the stage ring any more
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = i * 16 + 4 * g + e;
          float* pr = half_row(st0, st1, st2, st3, row);
#pragma unroll
          for (int jn = 0; jn < 4; ++jn) pr[half_col(row, wn * 64 + jn * 16 + r)] = acc[i][jn][e];
        }
    }
    __syncthreads();
    const int r0 = m0 + h * 128;                       // row of A of the half's row 0
    const int nvalid = M - r0 < 128 ? M - r0 : 128;    // rows of A in this half
    for (int row = wave; row < nvalid; row += NT / 64) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(half_row(st0, st1, st2, st3, row) +
                                                       half_col(row, 4 * lane));
      const float ss = wave_sum(v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]);
      const size_t gr = static_cast<size_t>(r0 + row);
      *reinterpret_cast<uint2*>(fe.y + gr * H + n0 + 4 * lane) =
          make_uint2(f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16),
                     f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16));
      if (lane == 0) fe.ss[gr * (H / BN) + n0 / BN] = ss;
    }
    __syncthreads();  // the half's stage arrays are free again
  }
}

// Split-K: block q of the tiles x S grid computes the k range
// [s K, (s+1) K) of tile t (t' = s tiles + t) into C + s c_split; W rows are
// ldw elements apart (S K).
//
// WP: the W matrices are their streaming copies (16-row tiles, 32-wide k
// blocks, the 64 MFMA lanes of 16 bytes each): a W load is one contiguous
// 1 KiB block, written to LDS in lane order, and a W fragment read is that
// block at lane x 16 bytes -- the same lanes/k slots as the swizzled
// row-major path.
// EPI = 0: fp32 C.  EPI = 1: the context K/V cells (kv_epilogue).  EPI = 2:
// the fused context rows in bf16 and their tile sums of squares
// (fuse_epilogue).
template <bool WP, int EPI>
__global__ __launch_bounds__(NT) void k_gemm_bf16_nt(const uint16_t* __restrict__ A, int lda,
                                                     int M, SegTable w, int K, int ldw,
                                                     float* __restrict__ C, int ldc, int nN,
                                                     int tiles, size_t c_split, KvEpi kv, FuseEpi fe) {
  // Five separate stage arrays (not one indexed ring): every access names its
  // stage statically, so the compiler can tell a stage being read from the
  // stages still being filled and does not wait for those loads.
  __shared__ __attribute__((aligned(16))) uint16_t st0[STAGE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t st1[STAGE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t st2[STAGE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t st3[STAGE_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t st4[STAGE_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // block b runs on XCD b % 8; XCD x owns the contiguous tile run
  // [x q + min(x, r), ...) of the nb = 8 q + r tiles (n fastest).
  const int nb = gridDim.x;
  const int x = blockIdx.x & 7, jb = blockIdx.x >> 3;
  const int q = nb >> 3, rem = nb & 7;
  const int tq = x * q + (x < rem ? x : rem) + jb;
  const int split = tq / tiles, t = tq - split * tiles;
  const int m0 = (t / nN) * BM, n0 = (t % nN) * BN;
  const size_t k0 = static_cast<size_t>(split) * K;
  C += split * c_split;

  int seg = 0, base = 0;
  for (int i = 0; i + 1 < w.nseg; ++i)
    if (n0 >= w.row_end[i]) { seg = i + 1; base = w.row_end[i]; }
  // row-major: row n0 - base, column k0; packed: row tile (n0 - base) / 16,
  // k block k0 / 32 (512 elements per block)
  const uint16_t* wb = static_cast<const uint16_t*>(w.ptr[seg]) +
                       (WP ? (static_cast<size_t>(n0 - base) / 16 * (ldw / BK) + k0 / BK) * 512
                           : static_cast<size_t>(n0 - base) * ldw + k0);

  // The stages are written only by direct-to-LDS loads; ordinary stores keep
  // the compiler from treating their contents as undefined.
  st0[tid] = 0;
  st1[tid] = 0;
  st2[tid] = 0;
  st3[tid] = 0;
  st4[tid] = 0;
  __syncthreads();

  // Loader: stage rows are 32 blocks of 16 (A blocks 0..15, W blocks 16..31);
  // wave v fills blocks 4v .. 4v+3, so waves 0-3 load A and waves 4-7 load W.
  // Lane L writes stage row 16 b + L/4, slot L%4, and fetches global chunk
  // slot ^ kswz(row).  A rows past M re-read row M-1 (their C rows are never
  // stored).  The loads go through a buffer resource over the rows this block
  // reads (scalar registers, exact byte extent), a constant per-lane byte
  // offset and the stage's k offset as the scalar offset, so no per-lane
  // address arithmetic is repeated per stage.
  const bool loads_a = wave < 4;
  const int last_a = (m0 + BM <= M ? m0 + BM : M) - 1;
  const char* rbase = loads_a ? reinterpret_cast<const char*>(A + static_cast<size_t>(m0) * lda + k0)
                              : reinterpret_cast<const char*>(wb);
  const uint32_t extent =
      loads_a ? 2u * static_cast<uint32_t>((last_a - m0) * lda + K)
              : (WP ? 1024u * static_cast<uint32_t>((BN / 16 - 1) * (ldw / BK) + K / BK)
                    : 2u * static_cast<uint32_t>((BN - 1) * ldw + K));
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(rbase), 0, static_cast<int>(extent), 0x00020000);
  uint32_t voff[4];
  int ldst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = 4 * wave + i, row = 16 * blk + (lane >> 2), c = (lane & 3) ^ kswz(row);
    if (loads_a) {
      const int gm = m0 + row < M ? m0 + row : M - 1;
      voff[i] = 2u * static_cast<uint32_t>((gm - m0) * lda + 8 * c);
    } else if (WP) {  // row tile blk - 16 of the tile, lane's 16 bytes of the block
      voff[i] = 1024u * static_cast<uint32_t>((blk - BM / 16) * (ldw / BK)) + 16u * lane;
    } else {
      voff[i] = 2u * static_cast<uint32_t>((row - BM) * ldw + 8 * c);
    }
    ldst[i] = blk * 16 * BK;  // element offset of the block inside a stage
  }
  const int kstep = loads_a || !WP ? 2 * BK : 1024;  // bytes between consecutive k stages
  auto issue_one = [&](uint16_t* st, int kt, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(st + ldst[i]),
                                             16, static_cast<int>(voff[i]), kt * kstep, 0, 0);
  };
  auto issue = [&](uint16_t* st, int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_one(st, kt, i);
  };

  // An (empty) statement naming an accumulation register lets the register
  // allocator place the 128 accumulators in AGPRs, leaving the VGPRs to the
  // two fragment sets.
  asm volatile("" ::"a"(0));
  const int wm = wave >> 2, wn = wave & 3;
  const int r = lane & 15, g = lane >> 4;
  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) acc[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Fragment rows start at multiples of 16, so the swizzle of every row a
  // lane reads is that of its row r, and the 12 fragment addresses of a
  // stage are two per-wave bases plus 1 KiB steps (instruction offsets).
  const uint32_t lane_w = WP ? 2 * BM * BK + wn * 4096 + 16 * lane : 2 * lds_off(BM + wn * 64 + r, g);
  const uint32_t lane_a = 2 * lds_off(wm * 128 + r, g);

  // Two register sets of the 12 fragments of a stage: the MFMAs of stage kt
  // run from one set while the reads of stage kt+1 fill the other.  Reads go
  // out in three-fragment groups q = 0..3 (W 0-2; W 3, A 0-1; A 2-4; A 5-7).
  u32x4 wfa[4], afa[8], wfb[4], afb[8];
  auto read_group = [&](const uint16_t* st, u32x4 (&wf)[4], u32x4 (&af)[8], int q) {
    if (q == 0) {
      const uint32_t bw = lds_base(lds_addr(st), lane_w);
      wf[0] = lds_read16<0>(bw);
      wf[1] = lds_read16<1024>(bw);
      wf[2] = lds_read16<2048>(bw);
    } else if (q == 1) {
      const uint32_t bw = lds_base(lds_addr(st), lane_w), ba = lds_base(lds_addr(st), lane_a);
      wf[3] = lds_read16<3072>(bw);
      af[0] = lds_read16<0>(ba);
      af[1] = lds_read16<1024>(ba);
    } else if (q == 2) {
      const uint32_t ba = lds_base(lds_addr(st), lane_a);
      af[2] = lds_read16<2048>(ba);
      af[3] = lds_read16<3072>(ba);
      af[4] = lds_read16<4096>(ba);
    } else {
      const uint32_t ba = lds_base(lds_addr(st), lane_a);
      af[5] = lds_read16<5120>(ba);
      af[6] = lds_read16<6144>(ba);
      af[7] = lds_read16<7168>(ba);
    }
  };
  auto read_frags = [&](const uint16_t* st, u32x4 (&wf)[4], u32x4 (&af)[8]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) read_group(st, wf, af, q);
  };

  // Step kt: wait for this wave's loads of stage kt+1 (the loads of the three
  // later stages, 4 each, may still be in flight) and for its reads of stage
  // kt; rendezvous (stage kt+1 has landed for every wave and no wave reads
  // stage kt's slot any more); multiply stage kt while reading stage kt+1
  // into the other register set and refilling stage kt's slot with stage
  // kt+5.
  auto step = [&](const uint16_t* nxt, uint16_t* refill, u32x4 (&wc)[4], u32x4 (&ac)[8],
                  u32x4 (&wn_)[4], u32x4 (&an)[8], int kt, int nk) {
    asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    lds_wait_all(wc, ac);
    // Plain rendezvous (no fence: a fence would also wait for the stages
    // still in flight).
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // The MFMAs start right after the rendezvous: stage kt+1's fragment
    // reads and the refill's loads go out in two halves, each after a group
    // of 16 MFMAs (issued together by all eight waves at the rendezvous, the
    // loads filled the address queue of the vector memory unit and held the
    // MFMAs back; measured: groups of 16 beat groups of 8, 4 and 32).
    // Both are unconditional: after the last stage the reads hit a slot no
    // load fills and are never used (a conditional read would keep the
    // set's previous contents live as well, a third set of registers), and
    // the refill loads the last stage again (in bounds, into a slot nothing
    // reads any more), so every step has the same loads in flight.
    const int ks = kt + STAGES < nk ? kt + STAGES : nk - 1;
    // Raised wave priority while this wave issues its MFMAs (measured: ~0.5%).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 4 * h; i < 4 * h + 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) acc[i][jn] = mfma_bf16(as_uint4(ac[i]), as_uint4(wc[jn]), acc[i][jn]);
      __builtin_amdgcn_sched_barrier(0);
      read_group(nxt, wn_, an, 2 * h);
      read_group(nxt, wn_, an, 2 * h + 1);
      issue_one(refill, ks, 2 * h);
      issue_one(refill, ks, 2 * h + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  const int nk = K / BK;  // a multiple of 10
  issue(st0, 0);
  issue(st1, 1);
  issue(st2, 2);
  issue(st3, 3);
  issue(st4, 4);
  asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  read_frags(st0, wfa, afa);
  for (int kt = 0; kt < nk; kt += 2 * STAGES) {
    step(st1, st0, wfa, afa, wfb, afb, kt, nk);
    step(st2, st1, wfb, afb, wfa, afa, kt + 1, nk);
    step(st3, st2, wfa, afa, wfb, afb, kt + 2, nk);
    step(st4, st3, wfb, afb, wfa, afa, kt + 3, nk);
    step(st0, st4, wfa, afa, wfb, afb, kt + 4, nk);
    step(st1, st0, wfb, afb, wfa, afa, kt + 5, nk);
    step(st2, st1, wfa, afa, wfb, afb, kt + 6, nk);
    step(st3, st2, wfb, afb, wfa, afa, kt + 7, nk);
    step(st4, st3, wfa, afa, wfb, afb, kt + 8, nk);
    step(st0, st4, wfb, afb, wfa, afa, kt + 9, nk);
  }
  // The last step's reads land before their registers can be reused, and
  // the repeated loads of the last stage land before the block's LDS is
  // released.
  lds_wait_all(wfa, afa);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if constexpr (EPI == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm * 128 + i * 16 + 4 * g + e;
        if (row < M) {
          float* cr = C + static_cast<size_t>(row) * ldc + n0 + wn * 64 + r;
#pragma unroll
          for (int jn = 0; jn < 4; ++jn) cr[jn * 16] = acc[i][jn][e];
        }
      }
  } else if constexpr (EPI == 1) {
    kv_epilogue(acc, st0, st1, st2, st3, m0, n0, M, wm, wn, r, g, tid, kv);
  } else {
    fuse_epilogue(acc, st0, st1, st2, st3, m0, n0, M, wm, wave, lane, r, g, fe);
  }
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* A, int lda, int M, const SegTable& w, bool w_packed, int K,
                            float* C, int ldc, int N, int nsplit, size_t c_split, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (nsplit < 1 || K % nsplit) return hipErrorInvalidValue;
  const int Ks = K / nsplit;
  if (N % BN || Ks % (2 * STAGES * BK) || lda % 8) return hipErrorInvalidValue;  // 12800: 40 x 10 x 32
  for (int i = 0; i < w.nseg; ++i)  // a block's 256 rows never straddle two matrices
    if (w.row_end[i] % BN) return hipErrorInvalidValue;
  const int nN = N / BN, nM = (M + BM - 1) / BM;
  const long long tiles = static_cast<long long>(nN) * nM;
  if (tiles * nsplit > 0x7fffffff) return hipErrorInvalidValue;
  const KvEpi none{};
  const FuseEpi fnone{};
  if (w_packed)
    hipLaunchKernelGGL((k_gemm_bf16_nt<true, 0>), dim3(static_cast<unsigned>(tiles * nsplit)), dim3(NT), 0, st, A,
                       lda, M, w, Ks, K, C, ldc, nN, static_cast<int>(tiles), c_split, none, fnone);
  else
    hipLaunchKernelGGL((k_gemm_bf16_nt<false, 0>), dim3(static_cast<unsigned>(tiles * nsplit)), dim3(NT), 0, st, A,
                       lda, M, w, Ks, K, C, ldc, nN, static_cast<int>(tiles), c_split, none, fnone);
  return hipGetLastError();
}

hipError_t launch_gemm_kv_bf16(const uint16_t* A, int lda, int M, const SegTable& w, bool w_packed,
                               const KvEpi& kv, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  constexpr int N = KV_N, K = H;
  if (lda % 8 || kv.cap <= 0 || kv.cap % BLK_CELLS || kv.pos0 < 0 || !kv.rope) return hipErrorInvalidValue;
  for (int i = 0; i < w.nseg; ++i)
    if (w.row_end[i] % BN) return hipErrorInvalidValue;
  if (w.nseg < 1 || w.row_end[w.nseg - 1] != N) return hipErrorInvalidValue;
  const int nN = N / BN, nM = (M + BM - 1) / BM;
  const long long tiles = static_cast<long long>(nN) * nM;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  const FuseEpi fnone{};
  if (w_packed)
    hipLaunchKernelGGL((k_gemm_bf16_nt<true, 1>), dim3(static_cast<unsigned>(tiles)), dim3(NT), 0, st, A, lda,
                       M, w, K, K, nullptr, 0, nN, static_cast<int>(tiles), size_t{0}, kv, fnone);
  else
    hipLaunchKernelGGL((k_gemm_bf16_nt<false, 1>), dim3(static_cast<unsigned>(tiles)), dim3(NT), 0, st, A, lda,
                       M, w, K, K, nullptr, 0, nN, static_cast<int>(tiles), size_t{0}, kv, fnone);
  return hipGetLastError();
}

hipError_t launch_gemm_fuse_bf16(const uint16_t* A, int lda, int M, const SegTable& w, bool w_packed,
                                 int K, const FuseEpi& fe, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  constexpr int N = H;
  if (K % (2 * STAGES * BK) || lda % 8 || !fe.y || !fe.ss) return hipErrorInvalidValue;
  for (int i = 0; i < w.nseg; ++i)
    if (w.row_end[i] % BN) return hipErrorInvalidValue;
  if (w.nseg < 1 || w.row_end[w.nseg - 1] != N) return hipErrorInvalidValue;
  const int nN = N / BN, nM = (M + BM - 1) / BM;
  const long long tiles = static_cast<long long>(nN) * nM;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  const KvEpi none{};
  if (w_packed)
    hipLaunchKernelGGL((k_gemm_bf16_nt<true, 2>), dim3(static_cast<unsigned>(tiles)), dim3(NT), 0, st, A, lda,
                       M, w, K, K, nullptr, 0, nN, static_cast<int>(tiles), size_t{0}, none, fe);
  else
    hipLaunchKernelGGL((k_gemm_bf16_nt<false, 2>), dim3(static_cast<unsigned>(tiles)), dim3(NT), 0, st, A, lda,
                       M, w, K, K, nullptr, 0, nN, static_cast<int>(tiles), size_t{0}, none, fe);
  return hipGetLastError();
}

}  // namespace dfl
