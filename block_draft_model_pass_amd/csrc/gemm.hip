// bf16 "NT" GEMM on MFMA for the long-context steps: context fusion
// (taps [n][12800] x fc^T) and the context K/V projection
// (ctx [n][2560] x [Wk_0; Wv_0; ...; Wk_4; Wv_4]^T).  Both operands are
// k-contiguous, which is the native operand layout of MFMA 16x16x32: a lane
// reads 8 consecutive k of one row of A and of one row of W.
//
// Block tile 256 x 256, 512 threads: 8 waves as 2 (m) x 4 (n), each owning a
// 128 x 64 sub-tile (8 x 4 MFMA tiles, 128 accumulator registers).  Per
// 32-wide k step a wave reads 12 operand fragments (12 KiB) from LDS for 32
// MFMAs, 384 bytes per 16-cycle MFMA, below what the four SIMDs of a CU need
// at full MFMA rate.
//
// k advances in 32-wide stages through a 5-deep LDS ring (32 KiB per stage,
// all 160 KiB of the CU's LDS) filled by direct global -> LDS loads (16 bytes
// per lane, no registers), so four stages are in flight while one is
// multiplied.  Stage rows are 64
// bytes (32 bf16); 16-byte chunk c of row r sits at chunk c ^ ((r >> 1) & 3),
// which keeps the 16-row fragment reads free of bank conflicts (measured);
// each load instruction fills 1 KiB of LDS (16 rows) in
// lane order, so a lane fetches the global chunk that the swizzle places at
// its slot.
//
// Tiles are dealt to the XCDs in contiguous runs (the hardware deals blocks
// round robin), so the blocks on one XCD share A panels in its L2.
#include "common.h"

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

// Fragment read issued as its own instruction: the compiler's wait-count
// pass cannot tell which stage a plain LDS read touches and would wait for
// every direct-to-LDS load in flight, serialising the stages.  The caller
// waits with lds_wait* before using the value.
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

// Wait until at most N of this wave's LDS reads are outstanding (they
// complete in order); the value passes through the statement so that nothing
// using it is scheduled before the wait.
template <int N>
__device__ __forceinline__ void lds_wait(u32x4& a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N) : "memory");
}

__device__ __forceinline__ uint4 as_uint4(u32x4 v) { return __builtin_bit_cast(uint4, v); }

// LDS element offset of chunk c of stage row `row` (A rows 0..255, W rows 256..511).
__device__ __forceinline__ int lds_off(int row, int c) { return row * BK + ((c ^ kswz(row)) << 3); }

__global__ __launch_bounds__(NT) void k_gemm_bf16_nt(const uint16_t* __restrict__ A, int lda,
                                                     int M, SegTable w, int K,
                                                     float* __restrict__ C, int ldc, int nN) {
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
  const int t = x * q + (x < rem ? x : rem) + jb;
  const int m0 = (t / nN) * BM, n0 = (t % nN) * BN;

  int seg = 0, base = 0;
  for (int i = 0; i + 1 < w.nseg; ++i)
    if (n0 >= w.row_end[i]) { seg = i + 1; base = w.row_end[i]; }
  const uint16_t* wb = static_cast<const uint16_t*>(w.ptr[seg]) + static_cast<size_t>(n0 - base) * K;

  // The stages are written only by direct-to-LDS loads; ordinary stores keep
  // the compiler from treating their contents as undefined.
  st0[tid] = 0;
  st1[tid] = 0;
  st2[tid] = 0;
  st3[tid] = 0;
  st4[tid] = 0;
  __syncthreads();

  // Loader: stage rows are 32 blocks of 16 (A blocks 0..15, W blocks 16..31);
  // wave v fills blocks 4v .. 4v+3.  Lane L writes stage row 16 b + L/4,
  // slot L%4, and fetches global chunk slot ^ kswz(row).  A rows past M
  // re-read row M-1 (their C rows are never stored).
  // Each block's 16 rows: a wave-uniform base pointer (scalar registers) and
  // a small per-lane element offset, to keep vector registers for the tile.
  const uint16_t* gbase[4];
  int goff[4];
  int ldst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = 4 * wave + i, row = 16 * blk + (lane >> 2), c = (lane & 3) ^ kswz(row);
    if (blk < BM / 16) {
      gbase[i] = A + static_cast<size_t>(m0 + 16 * blk) * lda;
      const int gm = m0 + row < M ? m0 + row : M - 1;
      goff[i] = (gm - (m0 + 16 * blk)) * lda + 8 * c;
    } else {
      gbase[i] = wb + static_cast<size_t>(16 * blk - BM) * K;
      goff[i] = (lane >> 2) * K + 8 * c;
    }
    ldst[i] = blk * 16 * BK;  // element offset of the block inside a stage
  }
  auto issue = [&](uint16_t* st, int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_global_load_lds(gbase[i] + goff[i] + kt * BK, st + ldst[i], 16, 0, 0);
  };

  const int wm = wave >> 2, wn = wave & 3;
  const int r = lane & 15, g = lane >> 4;
  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) acc[i][jn] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One k stage: wait for this wave's loads of stage kt (at most the later
  // stages' loads, 4 per stage, still outstanding), rendezvous, refill the
  // slot freed by stage kt-1 with stage kt+4, multiply stage kt.
  auto step = [&](const uint16_t* cur, uint16_t* refill, int kt, int nk) {
    const int later = nk - 1 - kt;
    if (later >= 3) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else if (later == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if (later == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // Plain rendezvous (no fence: a fence would also wait for the stages
    // still in flight); LDS reads of the previous stage were consumed by the
    // MFMAs before this point.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + STAGES - 1 < nk) issue(refill, kt + STAGES - 1);
    // All 12 fragment reads go out at once; row i of MFMAs waits only for
    // the reads up to its own A fragment.
    const uint32_t cb = lds_addr(cur);
    u32x4 wf[4], af[8];
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) wf[jn] = lds_read16(cb + 2 * lds_off(BM + wn * 64 + jn * 16 + r, g));
#pragma unroll
    for (int i = 0; i < 8; ++i) af[i] = lds_read16(cb + 2 * lds_off(wm * 128 + i * 16 + r, g));
    lds_wait<7>(wf[0]);
    lds_wait<7>(wf[1]);
    lds_wait<7>(wf[2]);
    lds_wait<7>(wf[3]);
#define GEMM_ROW(I, N)                                                                   \
    lds_wait<N>(af[I]);                                                                  \
    _Pragma("unroll") for (int jn = 0; jn < 4; ++jn)                                     \
        acc[I][jn] = mfma_bf16(as_uint4(af[I]), as_uint4(wf[jn]), acc[I][jn]);           \
    __builtin_amdgcn_sched_barrier(0);  /* keep this row between its wait and the next */
    GEMM_ROW(0, 7)
    GEMM_ROW(1, 6)
    GEMM_ROW(2, 5)
    GEMM_ROW(3, 4)
    GEMM_ROW(4, 3)
    GEMM_ROW(5, 2)
    GEMM_ROW(6, 1)
    GEMM_ROW(7, 0)
#undef GEMM_ROW
  };

  const int nk = K / BK;  // a multiple of 5
  issue(st0, 0);
  issue(st1, 1);
  issue(st2, 2);
  issue(st3, 3);
  for (int kt = 0; kt < nk; kt += STAGES) {
    step(st0, st4, kt, nk);
    step(st1, st0, kt + 1, nk);
    step(st2, st1, kt + 2, nk);
    step(st3, st2, kt + 3, nk);
    step(st4, st3, kt + 4, nk);
  }

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
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* A, int lda, int M, const SegTable& w, int K, float* C,
                            int ldc, int N, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (N % BN || K % (STAGES * BK) || lda % 8) return hipErrorInvalidValue;  // 12800: 80 x 5 x 32
  for (int i = 0; i < w.nseg; ++i)  // a block's 256 rows never straddle two matrices
    if (w.row_end[i] % BN) return hipErrorInvalidValue;
  const int nN = N / BN, nM = (M + BM - 1) / BM;
  const long long tiles = static_cast<long long>(nN) * nM;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gemm_bf16_nt, dim3(static_cast<unsigned>(tiles)), dim3(NT), 0, st, A, lda, M,
                     w, K, C, ldc, nN);
  return hipGetLastError();
}

}  // namespace dfl
