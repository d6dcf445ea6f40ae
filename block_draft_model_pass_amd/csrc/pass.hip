// The whole proposal pass as one persistent kernel (Strata PR #1426 page:
// "Drafter runtime" -- five dense layers, shared LM head, greedy proposals;
// "Target feature taps" -- anchor and mask rows, non-causal block attention,
// scale 1/16; "Parity validation" -- stage order).
//
// One 8-wave block per CU (a plain launch of at most as many blocks as the
// device has CUs; every block is resident while the device runs nothing
// else).  Phases are separated by a grid barrier (monotonic arrival counters,
// bounded spin: a wait that gives up sets a status word and the pass reports
// cand = -1):
//
//   per layer: QKV  -> ATTN (q/k norm + RoPE + partials) -> MERGE
//              -> O (+ residual, row sums of squares) -> GATE/UP -> DOWN (+ residual)
//   then:      LM head + greedy argmax -> final reduction by block 0
//
// Weights never depend on activations, so every wave issues the loads of its
// next weight slice while its block waits at a barrier (right after the
// block's arrival, so that a full load queue never delays the arrival); HBM
// keeps streaming while the grid synchronises and while activations are
// rebuilt in LDS.
//
// The L2 caches of the eight XCDs are not coherent with each other, and an
// agent-scope fence (L2 writeback or invalidate) costs about 2 us per
// barrier.  Instead, every value that one block writes and another block
// reads inside the kernel is written with device-coherent stores (agent-scope
// relaxed atomic stores, which write through to memory), and a wave waits for
// its own stores to complete before it arrives at a barrier.  Activations are
// single-assignment: each version of h, its row sums, qkv, the attention
// output and the MLP product has its own region, written once and only read
// after the barrier that follows, so no L2 can hold an older copy of a line
// (kernel launches start with invalidated L2s) and readers use ordinary cached
// loads -- the 80-120 KB every block reads comes from its XCD's L2.  Buffers
// that are rewritten within one pass (attention partials, argmax keys) are
// read with device-coherent loads.  The barrier is two-level (one counter per
// XCD, then one across XCDs) so that no single address takes 256 atomics.
//
// GEMV phases read bf16 activations from LDS (built once per phase; RMSNorm
// is folded into that build from fp32 h and per-tile sums of squares) and
// stream 16-row weight tiles through MFMA 16x16x32 bf16 exactly as the
// skinny GEMV kernels do (same k slots for weights and activations).
#include "common.h"

namespace dfl {

namespace {

constexpr int NWAVE = 8;
constexpr int ACT_WAVE = NWAVE - 1;  // the activation-staging wave (see "staged activations")
constexpr int NTHR = NWAVE * 64;
constexpr int XS_PAD = 8;                 // bf16 padding of an LDS activation row
constexpr int XS_MAX = F + XS_PAD;        // widest activation row (down projection)
constexpr int NT_H = H / 16;              // 160 row tiles of the hidden size
constexpr float NEG_INF = -__builtin_huge_valf();
// Versions: h_0 from the embedding, then after O(l) -> h_{2l+1}, after
// DOWN(l) -> h_{2l+2}.
constexpr int HV = 2 * L + 1;
constexpr size_t HSTRIDE = static_cast<size_t>(MAXB) * H;        // floats per h version
constexpr size_t SSTRIDE = static_cast<size_t>(H / 16) * MAXB;   // floats per ss version
constexpr size_t QSTRIDE = static_cast<size_t>(MAXB) * QKV_N;
constexpr size_t OSTRIDE = static_cast<size_t>(MAXB) * NQ * D;
constexpr size_t USTRIDE = static_cast<size_t>(MAXB) * F;
// Attention partials are single-assignment per layer too (chunk outputs fp16,
// chunk max / sum fp32); at most 128 chunks per KV head and 6 query tiles.
constexpr int NCH_PASS = 128, NQT_MAX = (G * MAXB + 15) / 16;
constexpr size_t PMSTRIDE = static_cast<size_t>(NKV) * NCH_PASS * NQT_MAX * 16;
constexpr size_t POSTRIDE = PMSTRIDE * D;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Global-address-space views of pointers the compiler cannot classify
// (pointers read from memory are generic): generic accesses would compile to
// flat instructions, which also count against the LDS wait counter and so
// would make every LDS rendezvous wait for the in-flight weight prefetch.
#define GA __attribute__((address_space(1)))

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <class T>
__device__ __forceinline__ T gld(const void* p) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if constexpr (sizeof(T) == 16) {
    return __builtin_bit_cast(T, *reinterpret_cast<const GA u32x4*>(a));
  } else if constexpr (sizeof(T) == 8) {
    return __builtin_bit_cast(T, *reinterpret_cast<const GA u32x2*>(a));
  } else if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, *reinterpret_cast<const GA uint32_t*>(a));
  } else {
    static_assert(sizeof(T) == 2, "gld: 2, 4, 8 or 16 bytes");
    return __builtin_bit_cast(T, *reinterpret_cast<const GA uint16_t*>(a));
  }
}

__device__ __forceinline__ void gst16(uint16_t* p, uint16_t v) {
  *reinterpret_cast<GA uint16_t*>(reinterpret_cast<uintptr_t>(p)) = v;
}

__device__ __forceinline__ uint4 ldw(const uint16_t* p) {
  return __builtin_bit_cast(
      uint4, __builtin_nontemporal_load(reinterpret_cast<const GA u32x4*>(reinterpret_cast<uintptr_t>(p))));
}

// LDS-only rendezvous: waits for this wave's LDS operations, not for its
// outstanding global loads (the weight prefetch stays in flight).
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// threadIdx.x as a value the compiler cannot see through: address math is
// then recomputed inside each phase instead of being hoisted out of the layer
// loop (which would keep hundreds of addresses alive and spill them).
__device__ __forceinline__ int otid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Wave index as a wave-uniform (scalar) value: conditions on it become scalar
// branches, and pointers chosen by it come from scalar loads.
__device__ __forceinline__ int wid() { return __builtin_amdgcn_readfirstlane(otid() >> 6); }

// Per-layer weight pointers; the init kernel copies them into the workspace
// so the pass kernel can index them by layer with plain global loads.
struct LayerTab {
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
};

struct PassArgs {
  const LayerTab* tab;   // in the workspace, written by the init kernel
  const uint16_t* final_norm;
  const uint16_t* lm;
  int vocab;
  float eps, scale_log2;
  // context ring of layer 0 (layer l adds l * layer stride)
  const uint16_t* ring_k;
  const uint16_t* ring_vt;
  int cap;
  int64_t lo, hi, p0;
  int nb, cb, nch;
  int B, nqt;
  // workspace
  // Single-assignment buffers: every version of a shared tensor has its own
  // region, written once (coherent stores) and read after a barrier with
  // ordinary cached loads -- no cache can hold an older value of it.
  float* h;          // [HV][8][H] residual stream versions
  uint16_t* h16;     // [HV][8][H] fp16 copies: the input of the RMSNorm builds
  float* ss;         // [HV][NT_H][8] per-tile sums of squares of each h version
  uint16_t* qkv;     // [L][8][QKV_N] fp16 (raw q, k, v before the head norms)
  const float2* rope;  // [16][128] (cos, sin): block rows, then commit rows at 8 + t
  uint16_t* po;
  float* pm;
  float* pl;
  uint16_t* o16;     // [L][8][NQ*D]
  uint16_t* u16;     // [L][8][F]
  uint64_t* keys;    // [grid][8]
  uint64_t* lse;     // [grid][8] per-block (max, sum) pairs of the softmax sweep
  unsigned* bar;     // barrier words (BAR_*)
  uint64_t wait_ticks;  // barrier wait bound, constant-clock ticks
  // Commit rows of the fused draft-commit cycle: nc (0..8) rows of target taps
  // for positions pos0 .. pos0+nc-1 (= p-nc .. p-1), fused and projected
  // inside this pass (their cells are written to the ring and attended to
  // from the workspace; the ring is read at [lo, hi) with hi = pos0).
  const uint16_t* taps;   // bf16 [nc][5][2560]
  const void* fc;         // streaming copy of fc, in the backbone's format
  const uint16_t* hidden_norm;
  int nc;
  int64_t pos0;
  float* yc;              // [8][H] fc outputs of the commit rows (fp32)
  float* fcp;             // [160][4][64][4] the FC phase's per-block tile partials
  uint16_t* cn;           // [8][H] their fused context rows in the MFMA input format,
                          // built in layer 0 and staged from here by later layers
  float* ckv;             // [L][8][1024] raw Wk | Wv outputs of the commit rows (fp32)
  // outputs
  int32_t* cand;
  uint16_t* logits;
  uint16_t* hidden;
  float* conf;       // [B-1] or null: softmax probability of each candidate
  int32_t* nkeep;    // or null: leading candidates whose conf >= min_p
  float min_p;
  // Device-resident positions (the decode cycle with no host round trip):
  // when dstate is set, p, the anchor and nc come from dstate[0..2] and lo,
  // hi, p0, nb, cb, nch, nc, pos0 and taps are derived from them at the start
  // of the pass (resolve_positions), exactly as the host derives them
  // otherwise; the commit taps are rows of taps_base (row r = position
  // taps_pos0 + r).
  const int64_t* dstate;
  const uint16_t* taps_base;
  int64_t taps_pos0, taps_rows, window;
  int maxch;
};

struct Smem {
  uint16_t x[MAXB * XS_MAX];   // activations (GEMV phases) / K/V blocks, rows buffer, staged constants (ATTN)
  uint16_t gain[H];            // RMSNorm gain of the phase (staged)
  float ssb[NT_H * MAXB];      // per-tile sums of squares of the phase's h version (staged)
  f32x4 red[NWAVE][64];        // cross-wave reduction
  float scal[64];              // per-row scales / merge weights
  float mw[4 * 256];           // merge: chunk weights and partial sums
  uint64_t best[2][64];
  float2 lse[2][64];
  float cf[MAXB];
};

// The layer table through the constant address space: indexed by the
// (uniform) layer, its pointers arrive by scalar loads, which never make the
// vector memory counter wait -- a vector load of a pointer would make the
// loads that use it wait for every weight load still in flight.
typedef const __attribute__((address_space(4))) LayerTab CLayerTab;
__device__ __forceinline__ CLayerTab* ctab(const PassArgs& a) {
  return reinterpret_cast<CLayerTab*>(reinterpret_cast<uintptr_t>(a.tab));
}

// ---------------------------------------------------------------- coherence

__device__ __forceinline__ GA uint64_t* g64(const void* p) {
  return reinterpret_cast<GA uint64_t*>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ GA uint32_t* g32(const void* p) {
  return reinterpret_cast<GA uint32_t*>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ uint64_t ld_coh64(const void* p) {
  return __hip_atomic_load(g64(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh64(void* p, uint64_t v) {
  __hip_atomic_store(g64(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_cohf(float* p, float v) {
  __hip_atomic_store(g32(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coh32(const void* p) {
  return __hip_atomic_load(g32(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint4 ld_coh128(const void* p) {
  const uint64_t a = ld_coh64(p), b = ld_coh64(static_cast<const char*>(p) + 8);
  return make_uint4(static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32),
                    static_cast<uint32_t>(b), static_cast<uint32_t>(b >> 32));
}
__device__ __forceinline__ void st_coh128(void* p, uint4 v) {
  st_coh64(p, static_cast<uint64_t>(v.x) | (static_cast<uint64_t>(v.y) << 32));
  st_coh64(static_cast<char*>(p) + 8, static_cast<uint64_t>(v.z) | (static_cast<uint64_t>(v.w) << 32));
}
__device__ __forceinline__ void st_coh_f4(float* p, f32x4 v) {
  st_coh128(p, make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                          __float_as_uint(v[3])));
}

// ---------------------------------------------------------------- barrier

// Barrier words (unsigned): status at [0], per-XCD arrival counters at
// [128 + 64 x], per-XCD release lines at [640 + 32 x] -- each in its own
// cache line.  The counters only grow during a pass (the init kernel zeroes
// them), so barrier k (1-based, counted by every block itself) is complete
// on XCD x once x's counter reaches k * (blocks on x); the arrival that
// completes it writes k into byte x of every XCD's 8-byte release word, and
// each XCD's waiters poll their own word until all its bytes reach k (32
// pollers per word instead of all 256 on one: measured 9 us less per pass).
// No resets and no second-level counter: the critical path is one atomic,
// the byte stores and the waiters' next poll, which matters because every
// memory round trip is slow while the weight stream saturates HBM (measured
// 2.3 us per pass less than a cross-XCD counter whose last arrival wrote the
// release words; 32-bit flags read by four loads per poll were 8.5 us
// slower).  The FC phase
// (fused draft-commit cycle) adds an arrival counter per fc output tile at
// [1024 + t] and the count of written tiles at [1184].
constexpr int BAR_STATUS = 0, BAR_XCD = 128, BAR_REL = 640, BAR_FC = 1024,
              BAR_FCDONE = BAR_FC + NT_H, BAR_WORDS = 1024 + 256;
static_assert(BAR_FCDONE < BAR_WORDS, "the FC words fit the barrier words");
// BAR_STATUS values: a barrier wait gave up, or the device-resident positions
// were invalid (the pass then did nothing but report it)
constexpr unsigned ST_TIMEOUT = 1u, ST_INVALID = 2u;

__device__ __forceinline__ unsigned ald(unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barrier state of one block: barriers passed, and (thread 0) whether this
// pass has given up waiting.
struct BarState {
  unsigned k = 0;
  bool quit = false;
};

// Grid barrier during which the waves issue the next phase's first loads
// (`prefetch`: each wave's weight slice; before the attention phase, the
// K/V and constants loads of waves 6 and 7 into LDS), after thread 0's
// arrival atomics (and, for the last arrival, the release): an s_barrier
// holds waves 1..7 until then.  The
// arrival atomics thus never queue behind the prefetch -- a wave's loads
// complete in order, and a CU whose load queue is full stalls further issue
// -- while the loads still stream during the wait.  (Issuing the prefetch of
// waves 1..7 before the arrival instead delayed arrivals by their issue
// stalls: measured 467 -> 445 us per pass at ctx 8192, block 8, with every
// barrier contributing.)
//
// The release is polled by one lane whose wave issued no prefetch at this
// barrier when there is one (`quiet_poller`: the staging wave, ACT_WAVE) --
// the poll loads of a wave that just issued its prefetch return only after
// that prefetch, in issue order, so such a block saw the release late --
// else by thread 0.
//
// The wait is bounded in wall-clock time (the constant-rate counter read by
// s_memrealtime): a wait longer than a.wait_ticks (plus 16 polls) sets the
// status word and gives up.  A block that gave up, or that finds the status word set (checked
// every 64 polls), waits at no later barrier of the pass, so a pass whose
// blocks cannot all be resident ends after about one bound instead of
// hanging the stream.
// Whether every XCD with blocks (the first nx) has completed barrier k, read
// from XCD x's release word: one byte per XCD (a pass has fewer than 256
// barriers), so a poll is one 8-byte load.
__device__ __forceinline__ bool released(const PassArgs& a, unsigned x, unsigned k, unsigned nx) {
  const uint64_t w = ld_coh64(a.bar + BAR_REL + 32 * x);
  bool ok = true;
#pragma unroll
  for (unsigned y = 0; y < 8; ++y) ok = ok && (y >= nx || ((w >> (8 * y)) & 0xffu) >= (k & 0xffu));
  return ok;
}

template <bool quiet_poller = false, class Pf>
__device__ __forceinline__ void grid_sync_pf(const PassArgs& a, BarState& b, Pf&& prefetch) {
  lds_sync();
  const unsigned k = ++b.k;
  const unsigned nx = gridDim.x < 8 ? gridDim.x : 8;
  const unsigned x = blockIdx.x & 7;  // blocks are dealt to the XCDs round robin
  if (otid() == 0) {
    unsigned* bar = a.bar;
    const unsigned per = (gridDim.x + 7 - x) / 8;
    if (__hip_atomic_fetch_add(bar + BAR_XCD + 64 * x, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT) == k * per - 1) {
      // the XCD's last arrival: its word in every XCD's release line
      for (unsigned xx = 0; xx < 8; ++xx)
        __hip_atomic_store(reinterpret_cast<uint8_t*>(bar + BAR_REL + 32 * xx) + x,
                           static_cast<uint8_t>(k), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_s_barrier();  // thread 0's arrival has gone out
  prefetch();
  const bool poller = quiet_poller ? otid() == ACT_WAVE * 64 : otid() == 0;
  if (poller && !b.quit) {
    // The clock and the status word are read every 16 and 64 polls only (a
    // counter read per poll would delay seeing the release); the clock starts
    // at the 16th poll, so a wait gives up after the bound plus 16 polls.
    uint64_t t0 = 0;
    unsigned n = 0;
    while (!released(a, x, k, nx)) {
      __builtin_amdgcn_s_sleep(2);
      if ((++n & 15) != 0) continue;
      if ((n & 63) == 0 && ald(a.bar + BAR_STATUS) != 0u) {  // another block gave up
        b.quit = true;
        break;
      }
      const uint64_t now = __builtin_amdgcn_s_memrealtime();
      if (n == 16) {
        t0 = now;
      } else if (now - t0 > a.wait_ticks) {  // bounded: never hang
        __hip_atomic_store(a.bar + BAR_STATUS, ST_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        b.quit = true;
        break;
      }
    }
  }
  lds_sync();
}

__device__ __forceinline__ void grid_sync(const PassArgs& a, BarState& b) {
  grid_sync_pf(a, b, [] {});
}

// ---------------------------------------------------------------- GEMV pieces

// bf16 matrices (the LM head and the layer matrices) are read from their
// streaming copies: 16-row tiles, then 32-wide k blocks, then the 64 MFMA
// lanes (lane = row % 16 + 16 g), 16 bytes each, so a wave's load of one k
// block is 1 KiB of contiguous memory -- about 1.5x the streaming rate of 64
// bytes from each of 16 rows (measured: 7.2 vs 4.6 TB/s).  Element offset of
// lane (row % 16, g)'s 8 values of k block kb:
__device__ __forceinline__ size_t packed_off(int K, int row, int kb, int g) {
  return ((static_cast<size_t>(row >> 4) * (K >> 5) + kb) * 64 + (row & 15) + 16 * g) * 8;
}

// nw weight uint4 of one lane: k = kbeg + 32 i + 8 g, i < nw, of row `row`
// of the packed bf16 matrix m (K columns).
// Every element is defined on every path (zero when !valid or i >= nw) so
// that no stale register value stays live across phases.
template <int NMAX>
__device__ __forceinline__ void load_tile(uint4 (&w)[NMAX], const uint16_t* m, int K, int row,
                                          int kbeg, int g, int nw, bool valid) {
  if (valid) {
#pragma unroll
    for (int i = 0; i < NMAX; ++i)
      w[i] = i < nw ? ldw(m + packed_off(K, row, (kbeg >> 5) + i, g)) : make_uint4(0, 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < NMAX; ++i) w[i] = make_uint4(0, 0, 0, 0);
  }
}

// acc over the same k slots, activations from LDS row xr.  MFMA column n
// only depends on the activation lanes of column n, so lanes past the
// block's rows read a valid row (see xrow) and their columns are ignored.
template <int NMAX>
__device__ __forceinline__ f32x4 mma_tile(const uint4 (&w)[NMAX], const uint16_t* xr, int kbeg,
                                          int g, int nw) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NMAX; ++i)
    if (i < nw) acc = mfma_bf16(w[i], *reinterpret_cast<const uint4*>(xr + kbeg + 32 * i + 8 * g), acc);
  return acc;
}

// LDS activation row fed to MFMA column r: r itself for the block's rows,
// else row 0 (a finite stand-in whose output column is never used).
__device__ __forceinline__ int xrow(int r, int B) { return r < B ? r : 0; }

// ---------------------------------------------------------------- weight formats

// One lane's share of a weight tile: N 16-byte loads.
//   bf16 : load i holds k = kbeg + 32 i + 8 g .. +8 (one MFMA bf16), from the
//          matrix's streaming copy (packed_off).
//   Q8_0 : load i holds 16 int8 at k = kbeg + 64 i + 16 g (two MFMAs, slots
//          + 8 m), all inside quant block kbeg/32 + 2 i + g/2.
//   Q4_0 : load i is the whole quant block kbeg/32 + 4 i + g (four MFMAs:
//          elements 8 m .. 8 m + 7 of the block).
//   Q5_0 : as Q4_0, plus the block's 32-bit word of fifth bits.
// Every format is read from the matrix's streaming copy, where the 64 lanes'
// 16 bytes of one load are 1 KiB of contiguous memory (and the quantized
// formats' scales of that load 64 or 128 contiguous bytes).
// A quantized load carries its block's fp16 scale (raw bits, splatted at use
// so that the load stays asynchronous); activations use the same k slots.
template <int FMT> struct KPerLoad;  // k covered by one load of all four lane groups
template <> struct KPerLoad<W_BF16> { static constexpr int v = 32; };
template <> struct KPerLoad<W_Q8_0> { static constexpr int v = 64; };
template <> struct KPerLoad<W_Q4_0> { static constexpr int v = 128; };
template <> struct KPerLoad<W_Q5_0> { static constexpr int v = 128; };

template <int FMT, int N>
struct WTile {
  uint4 q[N];
  uint32_t s[FMT == W_BF16 ? 1 : N];
  uint32_t h[FMT == W_Q5_0 ? N : 1];  // Q5_0 fifth bits (streaming-copy bit order)
};

struct WMat {
  const void* base;  // the matrix buffer in its storage format
  int rows, K;       // [rows][K]
};

__device__ __forceinline__ uint4 ldb(const uint8_t* p) {
  return __builtin_bit_cast(
      uint4, __builtin_nontemporal_load(reinterpret_cast<const GA u32x4*>(reinterpret_cast<uintptr_t>(p))));
}

// nl loads of row `row` from kbeg (loads i >= nl repeat load 0 and are never
// used).  One branch around the whole tile and straight-line loads inside:
// per-load branches leave join points at which the compiler's wait-count
// pass has to assume any load may still be in flight, and it then drains
// the whole queue (weight prefetch included) before reusing a register.
template <int FMT, int N>
__device__ __forceinline__ void load_wt(WTile<FMT, N>& t, WMat m, int row, int kbeg, int g, int nl,
                                        bool valid) {
  const uint8_t* b = static_cast<const uint8_t*>(m.base);
  if (valid) {
#pragma unroll
    for (int i0 = 0; i0 < N; ++i0) {
      const int i = i0 < nl ? i0 : 0;
      if constexpr (FMT == W_BF16) {
        t.q[i0] = ldb(b + 2 * packed_off(m.K, row, (kbeg >> 5) + i, g));
      } else if constexpr (FMT == W_Q8_0) {  // piece = 64 k: 1 KiB of quants, 64 B of scales
        const size_t pc = static_cast<size_t>(row >> 4) * (m.K >> 6) + (kbeg >> 6) + i;
        t.q[i0] = ldb(b + (pc * 64 + (row & 15) + 16 * g) * 16);
        t.s[i0] = gld<uint16_t>(b + static_cast<size_t>(m.rows) * m.K +
                                2 * (pc * 32 + (row & 15) * 2 + (g >> 1)));
      } else {  // piece = 128 k: 1 KiB of quants, 128 B of scales (Q5_0: 256 B of bits)
        const size_t pc = static_cast<size_t>(row >> 4) * (m.K >> 7) + (kbeg >> 7) + i;
        const size_t sq = static_cast<size_t>(m.rows) * m.K / 2;
        t.q[i0] = ldb(b + (pc * 64 + (row & 15) + 16 * g) * 16);
        t.s[i0] = gld<uint16_t>(b + sq + 2 * (pc * 64 + (row & 15) * 4 + g));
        if constexpr (FMT == W_Q5_0)
          t.h[i0] = gld<uint32_t>(b + sq + sq / 8 + 4 * (pc * 64 + (row & 15) * 4 + g));
      }
    }
  } else {
#pragma unroll
    for (int i0 = 0; i0 < N; ++i0) {
      t.q[i0] = make_uint4(0, 0, 0, 0);
      if constexpr (FMT != W_BF16) t.s[i0] = 0u;
      if constexpr (FMT == W_Q5_0) t.h[i0] = 0u;
    }
  }
  if constexpr (FMT == W_BF16) t.s[0] = 0u;
  if constexpr (FMT != W_Q5_0) t.h[0] = 0u;
}

template <int FMT, int N>
__device__ __forceinline__ f32x4 mma_wt(const WTile<FMT, N>& t, const uint16_t* xr, int kbeg, int g,
                                        int nl) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i < nl) {
      if constexpr (FMT == W_BF16) {
        acc = mfma_bf16(t.q[i], *reinterpret_cast<const uint4*>(xr + kbeg + 32 * i + 8 * g), acc);
      } else if constexpr (FMT == W_Q8_0) {
        const h2 sc = scale_h2(t.s[i]);
        const uint16_t* xp = xr + kbeg + 64 * i + 16 * g;
        const uint4 x0 = *reinterpret_cast<const uint4*>(xp);
        const uint4 x1 = *reinterpret_cast<const uint4*>(xp + 8);
        acc = mfma_f16(dq8(t.q[i].x, t.q[i].y, sc), x0, acc);
        acc = mfma_f16(dq8(t.q[i].z, t.q[i].w, sc), x1, acc);
      } else if constexpr (FMT == W_Q4_0) {
        const h2 sc = scale_h2(t.s[i]);
        const uint16_t* xp = xr + kbeg + 128 * i + 32 * g;
        const uint4 x0 = *reinterpret_cast<const uint4*>(xp);
        const uint4 x1 = *reinterpret_cast<const uint4*>(xp + 8);
        const uint4 x2 = *reinterpret_cast<const uint4*>(xp + 16);
        const uint4 x3 = *reinterpret_cast<const uint4*>(xp + 24);
        acc = mfma_f16(dq4(t.q[i].x, t.q[i].y, false, sc), x0, acc);
        acc = mfma_f16(dq4(t.q[i].z, t.q[i].w, false, sc), x1, acc);
        acc = mfma_f16(dq4(t.q[i].x, t.q[i].y, true, sc), x2, acc);
        acc = mfma_f16(dq4(t.q[i].z, t.q[i].w, true, sc), x3, acc);
      } else {  // Q5_0: elements 4 C .. 4 C + 3 take the fifth bits of group C
        const h2 sc = scale_h2(t.s[i]);
        const uint32_t hw = t.h[i];
        const uint16_t* xp = xr + kbeg + 128 * i + 32 * g;
        const uint4 x0 = *reinterpret_cast<const uint4*>(xp);
        const uint4 x1 = *reinterpret_cast<const uint4*>(xp + 8);
        const uint4 x2 = *reinterpret_cast<const uint4*>(xp + 16);
        const uint4 x3 = *reinterpret_cast<const uint4*>(xp + 24);
        acc = mfma_f16(dq5(t.q[i].x, t.q[i].y, false, q5_bits_packed<0>(hw), q5_bits_packed<1>(hw), sc),
                       x0, acc);
        acc = mfma_f16(dq5(t.q[i].z, t.q[i].w, false, q5_bits_packed<2>(hw), q5_bits_packed<3>(hw), sc),
                       x1, acc);
        acc = mfma_f16(dq5(t.q[i].x, t.q[i].y, true, q5_bits_packed<4>(hw), q5_bits_packed<5>(hw), sc),
                       x2, acc);
        acc = mfma_f16(dq5(t.q[i].z, t.q[i].w, true, q5_bits_packed<6>(hw), q5_bits_packed<7>(hw), sc),
                       x3, acc);
      }
    }
  }
  return acc;
}

// Sum of red[w0 .. w0+n) for this lane (after lds_sync).
__device__ __forceinline__ f32x4 group_sum(Smem& s, int w0, int n, int lane) {
  f32x4 acc = s.red[w0][lane];
  for (int w = 1; w < n; ++w) acc += s.red[w0 + w][lane];
  return acc;
}

// ---------------------------------------------------------------- staged activations
//
// A wave's loads complete in issue order, so an activation read issued after
// a wave's weight prefetch waits for the whole prefetch.  In the QKV, O, DOWN
// and LM phases the activations are therefore read by one wave that
// prefetches no weights at the barrier (ACT_WAVE): right after the release it
// copies them straight into LDS (buffer loads with an LDS destination, no
// registers), waits for them, then issues its own weight slice; the other
// waves' slices were issued during the barrier.  (ATTN and GU keep the
// register path: there the late slice of ACT_WAVE -- a K/V block share, or
// two gate/up pairs -- costs more than the earlier activations save.)
__device__ __forceinline__ bool act_wave() { return wid() == ACT_WAVE; }

// Cache-policy operand of the buffer builtins: sc1, as on the agent-scope
// stores (write-through, visible to the other XCDs once acknowledged).
constexpr int CPOL_SC1 = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// 64 lanes x 16 bytes from the resource (lane byte offset voff; bytes past its
// extent read as zeros) into 1 KiB of LDS at dst (lane i -> dst + 16 i).
__device__ __forceinline__ void g2lds(__amdgpu_buffer_rsrc_t rs, void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16,
                                           static_cast<int>(voff), 0, 0, 0);
}

// Rows 0..B-1 of a global [rows][K] fp16/bf16 matrix (K * 2 a multiple of
// 1 KiB) into LDS rows of stride K + XS_PAD, by the calling wave.
template <int K>
__device__ __forceinline__ void stage_rows(const PassArgs& a, Smem& s, const uint16_t* src) {
  static_assert((K * 2) % 1024 == 0, "rows are whole KiB");
  constexpr int XS = K + XS_PAD, C = K * 2 / 1024;
  const int lane = otid() & 63;
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc(src, static_cast<uint32_t>(a.B) * K * 2);
  for (int b = 0; b < a.B; ++b)
#pragma unroll
    for (int c = 0; c < C; ++c)
      g2lds(rs, s.x + b * XS + 512 * c, static_cast<uint32_t>(b * K * 2 + 1024 * c + 16 * lane));
}

// Wait for this wave's LDS-destination loads (and everything before them).
__device__ __forceinline__ void staged_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// x[b][k] = h[b][k] * rsqrt(mean_k h^2 + eps) * gain[k] for b < B, rounded to
// the activation format XF (bf16, or fp16 beside quantized weights), into
// LDS rows of stride H + pad.  np per-tile sums of squares are reduced in a
// fixed order.  Split in two so that a phase can issue its own weight loads
// between them: xn_load issues every load (h, the gains and the sums) in one
// round, xn_finish reduces, scales and stores.
constexpr int XN8 = MAXB * (H / 8) / NTHR;  // 8-element fp16 groups of h per thread (5)

struct XnRegs {
  uint4 h[XN8], g[XN8];
  float sv[3];
};

__device__ __forceinline__ void xn_load(const PassArgs& a, XnRegs& x, int ver, int np,
                                        const uint16_t* gain) {
  const int tid = otid(), wave = wid(), lane = tid & 63;
  const int n8 = a.B * (H / 8);
  const uint16_t* hsrc = a.h16 + ver * HSTRIDE;
  const float* ssrc = a.ss + ver * SSTRIDE;
#pragma unroll
  for (int u = 0; u < XN8; ++u) {
    const int e = tid + u * NTHR;
    // e >= n8 re-reads group 0 (never stored): no branch around the loads
    x.h[u] = gld<uint4>(hsrc + 8 * (e < n8 ? e : 0));
    x.g[u] = gld<uint4>(gain + (e % (H / 8)) * 8);
  }
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const int i = lane + 64 * q;
    const float v = gld<float>(ssrc + (i < np ? i : 0) * MAXB + (wave < MAXB ? wave : 0));
    x.sv[q] = wave < a.B && i < np ? v : 0.f;
  }
}

template <int XF>
__device__ __forceinline__ void xn_finish(const PassArgs& a, Smem& s, const XnRegs& x) {
  const int tid = otid(), wave = wid(), lane = tid & 63;
  const int n8 = a.B * (H / 8);
  if (wave < a.B) {
    const float v = wave_sum(x.sv[0] + x.sv[1] + x.sv[2]);
    if (lane == 0) s.scal[wave] = 1.0f / sqrtf(v / static_cast<float>(H) + a.eps);
  }
  lds_sync();
  constexpr int XS = H + XS_PAD;
#pragma unroll
  for (int u = 0; u < XN8; ++u) {
    const int e = tid + u * NTHR;
    if (e < n8) {
      const int b = e / (H / 8), k = (e % (H / 8)) * 8;
      const float sc = s.scal[b];
      const uint32_t hw[4] = {x.h[u].x, x.h[u].y, x.h[u].z, x.h[u].w};
      const uint32_t gw[4] = {x.g[u].x, x.g[u].y, x.g[u].z, x.g[u].w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t y0 = act16<XF>(f16_bits_to_f32(static_cast<uint16_t>(hw[i])) * sc *
                                      bf16_to_f32(static_cast<uint16_t>(gw[i])));
        const uint16_t y1 = act16<XF>(f16_bits_to_f32(static_cast<uint16_t>(hw[i] >> 16)) * sc *
                                      bf16_to_f32(static_cast<uint16_t>(gw[i] >> 16)));
        o[i] = y0 | (static_cast<uint32_t>(y1) << 16);
      }
      *reinterpret_cast<uint4*>(s.x + b * XS + k) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  lds_sync();
}

// x rows = act(h[ver] * rsqrt(mean h^2 + eps) * gain) from a staged copy:
// ACT_WAVE copies the fp16 h rows into the LDS x rows, the gain and the np
// per-tile sums of squares; wave b < B then reduces row b's sums (fixed
// order) and every thread normalises its groups in place.  `after` runs on
// ACT_WAVE once its copies have landed (its weight slice).
template <int XF, class Pre, class After>
__device__ __forceinline__ void build_x_norm_staged(const PassArgs& a, Smem& s, int ver, int np,
                                                    const uint16_t* gain, Pre&& pre,
                                                    After&& after) {
  const int tid = otid(), wave = wid(), lane = tid & 63;
  if (act_wave()) {
    stage_rows<H>(a, s, a.h16 + ver * HSTRIDE);
    const __amdgpu_buffer_rsrc_t rg = buf_rsrc(gain, H * 2);
#pragma unroll
    for (int c = 0; c < H * 2 / 1024; ++c) g2lds(rg, s.gain + 512 * c, 1024 * c + 16 * lane);
    const __amdgpu_buffer_rsrc_t rq =
        buf_rsrc(a.ss + ver * SSTRIDE, static_cast<uint32_t>(np) * MAXB * 4);
    for (int c = 0; c * 1024 < np * MAXB * 4; ++c) g2lds(rq, s.ssb + 256 * c, 1024 * c + 16 * lane);
    pre();  // more rows staged in the same round
    staged_wait();
    after();
  }
  lds_sync();
  if (wave < a.B) {
    float v = 0.f;
    for (int i = lane; i < np; i += 64) v += s.ssb[i * MAXB + wave];
    v = wave_sum(v);
    if (lane == 0) s.scal[wave] = 1.0f / sqrtf(v / static_cast<float>(H) + a.eps);
  }
  lds_sync();
  constexpr int XS = H + XS_PAD;
  const int n8 = a.B * (H / 8);
#pragma unroll
  for (int u = 0; u < XN8; ++u) {
    const int e = tid + u * NTHR;
    if (e < n8) {
      const int b = e / (H / 8), k = (e % (H / 8)) * 8;
      const float sc = s.scal[b];
      uint4* px = reinterpret_cast<uint4*>(s.x + b * XS + k);
      const uint4 hv = *px;
      const uint4 gv = *reinterpret_cast<const uint4*>(s.gain + k);
      const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
      const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t y0 = act16<XF>(f16_bits_to_f32(static_cast<uint16_t>(hw[i])) * sc *
                                      bf16_to_f32(static_cast<uint16_t>(gw[i])));
        const uint16_t y1 = act16<XF>(f16_bits_to_f32(static_cast<uint16_t>(hw[i] >> 16)) * sc *
                                      bf16_to_f32(static_cast<uint16_t>(gw[i] >> 16)));
        o[i] = y0 | (static_cast<uint32_t>(y1) << 16);
      }
      *px = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  lds_sync();
}

template <int XF, class After>
__device__ __forceinline__ void build_x_norm_staged(const PassArgs& a, Smem& s, int ver, int np,
                                                    const uint16_t* gain, After&& after) {
  build_x_norm_staged<XF>(a, s, ver, np, gain, [] {}, after);
}

template <int XF>
__device__ __forceinline__ void build_x_norm(const PassArgs& a, Smem& s, int ver, int np,
                                             const uint16_t* gain) {
  build_x_norm_staged<XF>(a, s, ver, np, gain, [] {}, [] {});
}

// The residual rows this lane updates (tile's 16 columns, row r), loaded at
// the start of a phase so that the epilogue does not wait for them.
__device__ __forceinline__ float4 residual_load(const PassArgs& a, int tile, int r, int g, int vin) {
  // rows past the block re-read row 0 (never used): no branch around the load
  return gld<float4>(a.h + vin * HSTRIDE + static_cast<size_t>(r < a.B ? r : 0) * H + tile * 16 + 4 * g);
}

// h rows (this tile's 16 columns) += acc, hv = residual_load(...); per-tile
// sums of squares.  Runs on the lanes of one wave holding the reduced tile.
__device__ __forceinline__ void residual_epilogue(const PassArgs& a, f32x4 acc, float4 hv,
                                                  int tile, int r, int g, int vin) {
  float sq = 0.f;
  if (r < a.B) {
    const size_t off = static_cast<size_t>(r) * H + tile * 16 + 4 * g;
    const f32x4 hn = {hv.x + acc[0], hv.y + acc[1], hv.z + acc[2], hv.w + acc[3]};
    st_coh_f4(a.h + (vin + 1) * HSTRIDE + off, hn);
    st_coh64(a.h16 + (vin + 1) * HSTRIDE + off,
             static_cast<uint64_t>(f32_to_f16_bits(hn[0])) |
                 (static_cast<uint64_t>(f32_to_f16_bits(hn[1])) << 16) |
                 (static_cast<uint64_t>(f32_to_f16_bits(hn[2])) << 32) |
                 (static_cast<uint64_t>(f32_to_f16_bits(hn[3])) << 48));
    sq = hn[0] * hn[0] + hn[1] * hn[1] + hn[2] * hn[2] + hn[3] * hn[3];
  }
  sq = group4_sum(sq);
  if (g == 0 && r < MAXB)
    st_cohf(a.ss + (vin + 1) * SSTRIDE + tile * MAXB + r, r < a.B ? sq : 0.f);
}

// ---------------------------------------------------------------- phases

// ---------------------------------------------------------------- commit rows
//
// Fused draft-commit cycle: the nc commit rows (the cells the last verify
// accepted) are fused (fc, then RMSNorm) and projected (each layer's Wk / Wv)
// inside the pass.  Their K/V projection rides the QKV phase's Wk / Wv tiles
// as MFMA columns 8..15 (the block rows use columns 0..7), so it streams no
// extra weight bytes; only fc (65.5 MB bf16) is added, in an FC phase at the
// start of the pass.
//
// FC phase: fc's 160 output tiles (16 of the 2560 rows) x 50 k slices of 256
// (of the 12800 = 5 taps x 2560) are 8000 work items dealt to the grid in
// contiguous runs (block b: items [8000 b / G, 8000 (b+1) / G), 31 or 32 at
// G = 256, spanning at most two tiles), so every block streams ~1/G of fc.
// Each wave takes every 8th item of its block's run: the item's weights
// (its 16 rows x 256 k) and the commit rows' taps at the same k slots, both
// straight into registers (lanes of MFMA columns 8..15 load no taps), with
// the next item's loads in flight while the current one runs; per tile it
// keeps one accumulator.  The block's waves are summed in LDS into one
// partial per tile it touched (16 rows x 8 commit rows, fp32), written to
// the workspace; the last of a tile's 2-3 contributing blocks (an arrival
// counter per tile) sums the tile's partials in contributor order -- the
// result does not depend on which block finishes last -- and writes the
// tile's 16 columns of the fc outputs.
constexpr int FC_SLICE = 256, FC_SLICES = T * H / FC_SLICE, FC_ITEMS = NT_H * FC_SLICES;
constexpr int FC_CONTRIB = 4;  // most blocks sharing a tile: 3 at 224 <= G <= 256, 4 up to G = 384
constexpr int FC_GRID_MAX = 384;
template <int FMT> using FcTile = WTile<FMT, FC_SLICE / KPerLoad<FMT>::v>;

__device__ __forceinline__ int fc_lo(int b, int G) { return b * FC_ITEMS / G; }
__device__ __forceinline__ int fc_owner(int item, int G) { return ((item + 1) * G - 1) / FC_ITEMS; }

// k offset (from the item's first k) of the 8-element activation group j of
// lane group g, matching the weight slots of each format (see load_wt).
template <int FMT>
__device__ __forceinline__ int fc_xslot(int j, int g) {
  if constexpr (FMT == W_BF16) return 32 * j + 8 * g;
  else if constexpr (FMT == W_Q8_0) return 64 * (j >> 1) + 16 * g + 8 * (j & 1);
  else return 128 * (j >> 2) + 32 * g + 8 * (j & 3);
}

// One item's loads: weights of rows 16 t.. at k = 256 s.., and taps of commit
// row n (lanes n < 8 that hold a commit row; the others get zeros).
template <int FMT>
__device__ __forceinline__ void fc_item_load(const PassArgs& a, int item, bool valid, FcTile<FMT>& W,
                                             uint4 (&x)[8]) {
  const int lane = otid() & 63, n = lane & 15, g = lane >> 4;
  const int it = valid ? item : 0;
  const int t = it / FC_SLICES, k0 = (it % FC_SLICES) * FC_SLICE;
  constexpr int N = FC_SLICE / KPerLoad<FMT>::v;
  load_wt<FMT, N>(W, WMat{a.fc, H, T * H}, t * 16 + n, k0, g, N, valid);
  const bool xv = valid && n < a.nc;
  const uint16_t* xr = a.taps + static_cast<size_t>(xv ? n : 0) * (T * H) + k0;
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = xv ? gld<uint4>(xr + fc_xslot<FMT>(j, g)) : make_uint4(0, 0, 0, 0);
}

__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 v) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = static_cast<uint32_t>(f32_to_f16_bits(bf16_to_f32(static_cast<uint16_t>(w[i])))) |
           (static_cast<uint32_t>(f32_to_f16_bits(bf16_to_f32(static_cast<uint16_t>(w[i] >> 16)))) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int FMT>
__device__ __forceinline__ f32x4 fc_item_mma(const FcTile<FMT>& W, const uint4 (&x)[8], f32x4 acc) {
  constexpr int N = FC_SLICE / KPerLoad<FMT>::v;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if constexpr (FMT == W_BF16) {
      acc = mfma_bf16(W.q[i], x[i], acc);
    } else if constexpr (FMT == W_Q8_0) {
      const h2 sc = scale_h2(W.s[i]);
      acc = mfma_f16(dq8(W.q[i].x, W.q[i].y, sc), bf16x8_to_f16x8(x[2 * i]), acc);
      acc = mfma_f16(dq8(W.q[i].z, W.q[i].w, sc), bf16x8_to_f16x8(x[2 * i + 1]), acc);
    } else if constexpr (FMT == W_Q4_0) {
      const h2 sc = scale_h2(W.s[i]);
      acc = mfma_f16(dq4(W.q[i].x, W.q[i].y, false, sc), bf16x8_to_f16x8(x[4 * i]), acc);
      acc = mfma_f16(dq4(W.q[i].z, W.q[i].w, false, sc), bf16x8_to_f16x8(x[4 * i + 1]), acc);
      acc = mfma_f16(dq4(W.q[i].x, W.q[i].y, true, sc), bf16x8_to_f16x8(x[4 * i + 2]), acc);
      acc = mfma_f16(dq4(W.q[i].z, W.q[i].w, true, sc), bf16x8_to_f16x8(x[4 * i + 3]), acc);
    } else {
      const h2 sc = scale_h2(W.s[i]);
      const uint32_t hw = W.h[i];
      acc = mfma_f16(dq5(W.q[i].x, W.q[i].y, false, q5_bits_packed<0>(hw), q5_bits_packed<1>(hw), sc),
                     bf16x8_to_f16x8(x[4 * i]), acc);
      acc = mfma_f16(dq5(W.q[i].z, W.q[i].w, false, q5_bits_packed<2>(hw), q5_bits_packed<3>(hw), sc),
                     bf16x8_to_f16x8(x[4 * i + 1]), acc);
      acc = mfma_f16(dq5(W.q[i].x, W.q[i].y, true, q5_bits_packed<4>(hw), q5_bits_packed<5>(hw), sc),
                     bf16x8_to_f16x8(x[4 * i + 2]), acc);
      acc = mfma_f16(dq5(W.q[i].z, W.q[i].w, true, q5_bits_packed<6>(hw), q5_bits_packed<7>(hw), sc),
                     bf16x8_to_f16x8(x[4 * i + 3]), acc);
    }
  }
  return acc;
}

template <int FMT>
__device__ __forceinline__ void fc_phase(const PassArgs& a, Smem& s) {
  if (a.nc == 0) return;
  const int G = static_cast<int>(gridDim.x), b = blockIdx.x;
  const int wave = wid(), lane = otid() & 63, n = lane & 15, g = lane >> 4;
  const int lo = fc_lo(b, G), hi = fc_lo(b + 1, G);
  const int t0 = lo / FC_SLICES;          // first tile of the run
  const int nt = (hi - 1) / FC_SLICES - t0 + 1;  // 1 or 2 tiles
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  // two register sets, alternating (rounds unrolled in pairs: no dynamic
  // indexing of register arrays)
  FcTile<FMT> W0, W1;
  uint4 x0[8], x1[8];
  auto run = [&](int cur, const FcTile<FMT>& W, const uint4 (&x)[8]) {
    if (cur < hi) {
      if (cur / FC_SLICES == t0) acc0 = fc_item_mma<FMT>(W, x, acc0);
      else acc1 = fc_item_mma<FMT>(W, x, acc1);
    }
  };
  const int rounds = (hi - lo + NWAVE - 1) / NWAVE;
  fc_item_load<FMT>(a, lo + wave, lo + wave < hi, W0, x0);
  for (int r = 0; r < rounds; r += 2) {
    const int c0 = lo + wave + NWAVE * r, c1 = c0 + NWAVE, c2 = c1 + NWAVE;
    if (r + 1 < rounds) fc_item_load<FMT>(a, c1, c1 < hi, W1, x1);
    run(c0, W0, x0);
    if (r + 1 < rounds) {
      if (r + 2 < rounds) fc_item_load<FMT>(a, c2, c2 < hi, W0, x0);
      run(c1, W1, x1);
    }
  }
  // the block's partial of each tile it touched: waves summed in LDS (fixed order)
  float* part = a.fcp;
  for (int ti = 0; ti < nt; ++ti) {
    s.red[wave][lane] = ti == 0 ? acc0 : acc1;
    lds_sync();
    if (wave == 0) {
      const f32x4 v = group_sum(s, 0, NWAVE, lane);
      const int t = t0 + ti, q = b - fc_owner(t * FC_SLICES, G);  // contributor index
      st_coh_f4(part + ((static_cast<size_t>(t) * FC_CONTRIB + q) * 64 + lane) * 4, v);
    }
    lds_sync();
  }
  wait_stores();
  // arrival per tile; the last contributor sums the partials in contributor order
  if (otid() == 0) {
    for (int ti = 0; ti < nt; ++ti) {
      const int t = t0 + ti;
      const int q0 = fc_owner(t * FC_SLICES, G), q1 = fc_owner(t * FC_SLICES + FC_SLICES - 1, G);
      const unsigned prev = __hip_atomic_fetch_add(a.bar + BAR_FC + t, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      s.scal[ti] = prev == static_cast<unsigned>(q1 - q0) ? 1.f : 0.f;
    }
  }
  lds_sync();
  if (wave == 0) {
    for (int ti = 0; ti < nt; ++ti) {
      if (s.scal[ti] != 0.f) {
        const int t = t0 + ti;
        const int q0 = fc_owner(t * FC_SLICES, G), q1 = fc_owner(t * FC_SLICES + FC_SLICES - 1, G);
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q <= q1 - q0; ++q) {
          const uint4 u = ld_coh128(part + ((static_cast<size_t>(t) * FC_CONTRIB + q) * 64 + lane) * 4);
          sum += f32x4{__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                       __uint_as_float(u.w)};
        }
        // lane (n, g) holds rows 4g..4g+3 of the tile for commit row n
        if (n < a.nc) st_coh_f4(a.yc + static_cast<size_t>(n) * H + t * 16 + 4 * g, sum);
      }
    }
    wait_stores();
    // the tiles this block completed are announced once their outputs are out
    if (lane == 0)
      for (int ti = 0; ti < nt; ++ti)
        if (s.scal[ti] != 0.f)
          __hip_atomic_fetch_add(a.bar + BAR_FCDONE, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Wait (thread 0, bounded in wall-clock time like a barrier) until every fc
// output tile is written: only the blocks that build the commit rows wait,
// so the pass needs no grid barrier after the FC phase.
__device__ __forceinline__ void fc_wait(const PassArgs& a) {
  uint64_t t0 = 0;
  unsigned n = 0;
  while (ald(a.bar + BAR_FCDONE) < static_cast<unsigned>(NT_H)) {
    __builtin_amdgcn_s_sleep(2);
    if ((++n & 15) != 0) continue;
    if ((n & 63) == 0 && ald(a.bar + BAR_STATUS) != 0u) break;  // the pass gave up
    const uint64_t now = __builtin_amdgcn_s_memrealtime();
    if (n == 16) {
      t0 = now;
    } else if (now - t0 > a.wait_ticks) {
      __hip_atomic_store(a.bar + BAR_STATUS, ST_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
  }
}

// Commit rows into LDS rows 8 .. 8+nc-1 for the Wk / Wv tiles of the QKV
// phase: c = bf16(rmsnorm(y) * hidden_norm) (the fused context row, in bf16
// as the fusion hands it to the projection), in the MFMA input format.  Wave
// t builds row t; rows past nc are zeros.
template <int FMT>
__device__ __forceinline__ void commit_rows_build(const PassArgs& a, Smem& s) {
  constexpr int XS = H + XS_PAD;
  const int wave = wid(), lane = otid() & 63;
  const int t = wave < a.nc ? wave : 0;
  float4 v[10];
  uint2 gn[10];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    v[i] = gld<float4>(a.yc + static_cast<size_t>(t) * H + 4 * (lane + 64 * i));
    gn[i] = gld<uint2>(a.hidden_norm + 4 * (lane + 64 * i));
  }
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < 10; ++i) sq += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
  sq = wave_sum(sq);
  const float sc = 1.0f / sqrtf(sq / static_cast<float>(H) + a.eps);
  const bool live = wave < a.nc;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const float y4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    const uint32_t gw[2] = {gn[i].x, gn[i].y};
    uint16_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t c = f32_to_bf16(y4[e] * sc * bf16_to_f32(static_cast<uint16_t>(gw[e >> 1] >> (16 * (e & 1)))));
      o[e] = live ? (FMT == W_BF16 ? c : f32_to_f16_bits(bf16_to_f32(c))) : 0;
    }
    *reinterpret_cast<uint2*>(s.x + (MAXB + wave) * XS + 4 * (lane + 64 * i)) =
        make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
  }
}

// Work of one block for the QKV phase: tiles 2w and 2w+1 of the 448 fused
// q|k|v row tiles; wave v takes tile 2w + v/4 and k quarter v%4 (640 k).
// Tiles never straddle the q / k / v matrices (6144 and 512 rows).
__device__ __forceinline__ WMat qkv_mat(const PassArgs& a, int l, int tile, int& row0) {
  const int r0 = tile * 16;
  if (r0 < NQ * D) { row0 = r0; return WMat{ctab(a)->wq[l], NQ * D, H}; }
  if (r0 < NQ * D + NKV * D) { row0 = r0 - NQ * D; return WMat{ctab(a)->wk[l], NKV * D, H}; }
  row0 = r0 - NQ * D - NKV * D;
  return WMat{ctab(a)->wv[l], NKV * D, H};
}

__device__ __forceinline__ bool qkv_has(int w) { return w < QKV_N / 32; }

template <int FMT> using QkvTile = WTile<FMT, 640 / KPerLoad<FMT>::v>;

template <int FMT>
__device__ __forceinline__ void qkv_prefetch(const PassArgs& a, int l, QkvTile<FMT>& W, bool go) {
  const int w = blockIdx.x, wave = wid(), lane = otid() & 63;
  const bool has = qkv_has(w);
  int row0;
  const WMat m = qkv_mat(a, l, has ? 2 * w + (wave >> 2) : 0, row0);
  constexpr int N = 640 / KPerLoad<FMT>::v;
  load_wt<FMT, N>(W, m, row0 + (lane & 15), (wave & 3) * 640, lane >> 4, N, go && has);
}

// Blocks whose two tiles are Wk / Wv rows (the ctx K/V projection's rows).
__device__ __forceinline__ bool qkv_kv_block(int w) { return 2 * w * 16 >= NQ * D && qkv_has(w); }
constexpr int QKV_KV_FIRST = NQ * D / 32;  // the first block with Wk / Wv tiles

// The commit rows built in LDS rows 8..15 (layer 0) into a.cn for the later
// layers' QKV phases (read there after several barriers: coherent stores).
__device__ __forceinline__ void commit_rows_keep(const PassArgs& a, Smem& s) {
  constexpr int XS = H + XS_PAD, U = MAXB * (H / 8) / NTHR;
  static_assert(MAXB * (H / 8) % NTHR == 0, "whole 16-byte groups per thread");
  const int tid = otid();
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int e = tid + u * NTHR, t = e / (H / 8), k8 = e % (H / 8);
    st_coh128(a.cn + static_cast<size_t>(t) * H + 8 * k8,
              *reinterpret_cast<const uint4*>(s.x + (MAXB + t) * XS + 8 * k8));
  }
}

template <int FMT>
__device__ __forceinline__ void qkv_phase(const PassArgs& a, Smem& s, int l, int np, QkvTile<FMT>& W) {
  const int w = blockIdx.x, wave = wid(), lane = otid() & 63;
  const int r = lane & 15, g = lane >> 4;
  const bool has = qkv_has(w);
  // commit rows ride the Wk / Wv tiles as MFMA columns 8..15: built from the
  // fc outputs in layer 0 (and kept in a.cn by the first such block), staged
  // from a.cn with the activations in later layers
  const bool cm = a.nc > 0 && qkv_kv_block(w);
  // activations staged by ACT_WAVE, which then issues its weight slice
  if (has)
    build_x_norm_staged<FMT>(
        a, s, 2 * l, np, ctab(a)->in_norm[l],
        [&] {
          if (cm && l > 0) {
            constexpr int XS = H + XS_PAD;
            const int lane = otid() & 63;
            const __amdgpu_buffer_rsrc_t rc = buf_rsrc(a.cn, MAXB * H * 2);
            for (int t = 0; t < MAXB; ++t)
#pragma unroll
              for (int c = 0; c < H * 2 / 1024; ++c)
                g2lds(rc, s.x + (MAXB + t) * XS + 512 * c,
                      static_cast<uint32_t>(t * H * 2 + 1024 * c + 16 * lane));
          }
        },
        [&] { qkv_prefetch<FMT>(a, l, W, true); });
  if (cm && l == 0) {
    if (otid() == 0) fc_wait(a);
    lds_sync();
    commit_rows_build<FMT>(a, s);
    lds_sync();
    if (w == QKV_KV_FIRST) commit_rows_keep(a, s);
  }
  if (has) {
    const int tile = 2 * w + (wave >> 2);
    constexpr int XS = H + XS_PAD;
    constexpr int N = 640 / KPerLoad<FMT>::v;
    const int xr = r < MAXB ? xrow(r, a.B) : (cm ? r : 0);
    f32x4 acc = mma_wt<FMT, N>(W, s.x + xr * XS, (wave & 3) * 640, g, N);
    s.red[wave][lane] = acc;
    lds_sync();
    if ((wave & 3) == 0) {
      acc = group_sum(s, wave, 4, lane);
      if (r < a.B)
        st_coh64(a.qkv + l * QSTRIDE + static_cast<size_t>(r) * QKV_N + tile * 16 + 4 * g,
                 static_cast<uint64_t>(f32_to_f16_bits(acc[0])) |
                     (static_cast<uint64_t>(f32_to_f16_bits(acc[1])) << 16) |
                     (static_cast<uint64_t>(f32_to_f16_bits(acc[2])) << 32) |
                     (static_cast<uint64_t>(f32_to_f16_bits(acc[3])) << 48));
      else if (cm && r >= MAXB && r - MAXB < a.nc)  // raw K | V of commit row r - 8, fp32
        st_coh_f4(a.ckv + (static_cast<size_t>(l) * MAXB + (r - MAXB)) * (2 * NKV * D) +
                      tile * 16 - NQ * D + 4 * g,
                  acc);
    }
  }
  wait_stores();
}

// ---------------------------------------------------------------- attention
//
// Block w < 2 nch takes KV head j = w / nch and chunk c = w % nch of the
// visible context (cb blocks of 32 cells); the last chunk of each head also
// takes the block rows' own keys.  Context K/V never depends on this pass, so
// the chunk's first two 32-cell blocks (16 KiB of K and 16 KiB of V^T each)
// are loaded straight into LDS during the barrier that precedes the phase,
// with the layer's q / k norm gains and the RoPE rows (attn_stage); later
// pairs (long contexts) go through registers, each loaded once the previous
// pair has run (its registers are free then).  Waves t < nqt own 16 query
// rows each.  A chunk leaves
// its output normalised by its own softmax sum, in fp16, with its maximum
// and sum.

struct KVRegs {
  uint4 v[4];
};

__device__ __forceinline__ bool attn_block_src(const PassArgs& a, int l, int ib_global,
                                               const uint16_t*& kp, const uint16_t*& vp, int j) {
  if (ib_global >= a.nb) return false;
  const int64_t pb = a.p0 + 32 * static_cast<int64_t>(ib_global);
  const int cidx = static_cast<int>(pb % a.cap);
  kp = a.ring_k + ((static_cast<size_t>(l) * NKV + j) * a.cap + cidx) * D;
  vp = a.ring_vt + (static_cast<size_t>(l) * NKV + j) * D * a.cap + static_cast<size_t>(cidx) * D;
  return true;
}

// Thread's share of one block: K (1024 uint4) then V^T (1024 uint4).
__device__ __forceinline__ void attn_load(const PassArgs& a, int l, int ib_global, int j,
                                          KVRegs& R, bool go) {
  const uint16_t *kp = nullptr, *vp = nullptr;
  const bool ok = go && attn_block_src(a, l, ib_global, kp, vp, j);
  const int tid = otid();
  if (ok) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      R.v[u] = ldw(kp + 8 * (tid + u * NTHR));
      R.v[2 + u] = ldw(vp + 8 * (tid + u * NTHR));
    }
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) R.v[u] = make_uint4(0, 0, 0, 0);
  }
}

// LDS layouts of one 32-cell block, XOR-swizzled in 16-byte pieces, so that
// every MFMA operand read below touches each bank once and a piece can come
// straight from the ring by a 16-byte load with an LDS destination:
//   keys   [32 cells][256]: 16-byte piece c of cell r sits at piece c ^ kf(r)
//   values [256 dims][32] : 16-byte piece q of dim d (cells 8q..8q+7) sits at
//                           piece q ^ vf(d)
// Row n of a block's first 16-row score tile is cell kcell(n), of its second
// kcell(n) + 4: the lanes of group g then hold the scores of cells 8g..8g+7,
// which is one 16-byte piece of a value row -- the k slots of the P.V MFMA.
// (kf(kcell(n)) = kf(kcell(n) + 4) = n, so a key read by 16 rows at one piece
// hits 16 distinct pieces; vf gives 8 consecutive dims distinct (d & 1, vf)
// and 16 distinct (d & 3, vf).)  Offsets are in fp16 elements.
__device__ __forceinline__ int kf(int cell) { return (cell & 3) | ((cell >> 1) & 12); }
__device__ __forceinline__ int vf(int dim) { return (((dim >> 1) ^ (dim >> 3)) & 1) | ((dim >> 1) & 2); }
__device__ __forceinline__ int kcell(int n) { return 8 * (n >> 2) + (n & 3); }
__device__ __forceinline__ int kswz(int cell, int c16) { return cell * D + ((c16 ^ kf(cell)) << 3); }
__device__ __forceinline__ int vswz(int dim, int q) { return dim * BLK_CELLS + ((q ^ vf(dim)) << 3); }
__device__ __forceinline__ int vel(int dim, int cell) { return vswz(dim, cell >> 3) + (cell & 7); }

__device__ __forceinline__ void attn_store(const KVRegs& R, uint16_t* kbuf, uint16_t* vbuf) {
  const int tid = otid();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + u * NTHR;
    *reinterpret_cast<uint4*>(kbuf + kswz(e >> 5, e & 31)) = R.v[u];
    *reinterpret_cast<uint4*>(vbuf + vswz(e >> 2, e & 3)) = R.v[2 + u];
  }
}

// LDS of the attention phase, in fp16 elements of s.x: the two block
// buffers of a pair (keys of block b at 2 b x 8192, its values right after),
// the block rows' buffer (4 x 8192), and the staged per-layer constants: the
// q-norm and k-norm gains (bf16, 1 KiB slots) and the RoPE rows of the block
// rows (rows 0..B-1) and commit rows (rows MAXB..) at their table rows.
constexpr int ATT_QG = 6 * BLK_CELLS * D, ATT_KG = ATT_QG + 512, ATT_ROPE = ATT_QG + 1024;
static_assert(ATT_ROPE + 2 * MAXB * 2 * D <= MAXB * XS_MAX, "staged constants fit in s.x");  // 1 KiB rows
// Waves 6 and 7 load, with an LDS destination, at the barrier before the
// phase (the query waves t < nqt <= 6 load nothing there, so their query
// loads go out at the release): wave 7 first the per-layer constants, then
// both waves 32 KiB each of the chunk's first two K/V blocks -- exactly
// KV_DMA_LOADS loads each (an absent block reads as zeros), so that wave 7
// can wait for its constants alone.  Load i of a block's keys or values
// fills LDS bytes [1024 i, 1024 i + 1024) lane by lane, each lane reading
// the ring piece that belongs at its slot of the swizzled layout.
constexpr int KV_DMA_W0 = NWAVE - 2, KV_DMA_LOADS = 32;
static_assert(NQT_MAX <= KV_DMA_W0, "the K/V waves own no query rows");
static_assert(ACT_WAVE >= KV_DMA_W0, "the staging wave is a K/V wave");
__device__ __forceinline__ void attn_stage(const PassArgs& a, Smem& s, int l) {
  const int w = blockIdx.x, wave = wid();
  if (w >= NKV * a.nch || wave < KV_DMA_W0) return;
  const int lane = otid() & 63;
  if (wave == ACT_WAVE) {
    g2lds(buf_rsrc(ctab(a)->q_norm[l], D * 2), s.x + ATT_QG, 16 * lane);
    g2lds(buf_rsrc(ctab(a)->k_norm[l], D * 2), s.x + ATT_KG, 16 * lane);
    const __amdgpu_buffer_rsrc_t rr = buf_rsrc(a.rope, 2 * MAXB * D * 4);
    for (int r = 0; r < a.B; ++r) g2lds(rr, s.x + ATT_ROPE + r * 2 * D, r * D * 4 + 16 * lane);
    for (int r = MAXB; r < MAXB + a.nc; ++r) g2lds(rr, s.x + ATT_ROPE + r * 2 * D, r * D * 4 + 16 * lane);
  }
  const int j = w / a.nch, c = w % a.nch;
  const int blk0 = c * a.cb;
  const int nblk = a.nb > blk0 ? min(a.cb, a.nb - blk0) : 0;
  const int b = wave - KV_DMA_W0;  // this wave's block of the pair
  const uint16_t *kp = a.ring_k, *vp = a.ring_vt;
  const bool has = b < nblk && attn_block_src(a, l, blk0 + b, kp, vp, j);
  const uint32_t bytes = has ? BLK_CELLS * D * 2 : 0;
  const __amdgpu_buffer_rsrc_t rk = buf_rsrc(kp, bytes), rv = buf_rsrc(vp, bytes);
  uint16_t* kb = s.x + 2 * b * BLK_CELLS * D;
  uint16_t* vb = kb + BLK_CELLS * D;
  const int kcl = lane >> 5, kpc = lane & 31, vdl = lane >> 2, vq = lane & 3;
#pragma unroll
  for (int pc = 0; pc < 16; ++pc) {
    const int cell = 2 * pc + kcl;
    g2lds(rk, kb + 512 * pc, static_cast<uint32_t>(cell * D * 2 + 16 * (kpc ^ kf(cell))));
  }
#pragma unroll
  for (int pc = 0; pc < 16; ++pc) {
    const int dim = 16 * pc + vdl;
    g2lds(rv, vb + 512 * pc, static_cast<uint32_t>(dim * BLK_CELLS * 2 + 16 * (vq ^ vf(dim))));
  }
}

// One 32-cell block from LDS (keys [32][256], values [256][32]) for this
// wave's 16 query rows; cells at positions outside [lo, hi) are masked.
__device__ __forceinline__ void attn_block(const uint16_t* kb, const uint16_t* vb, int64_t pb,
                                           int64_t lo, int64_t hi, float scale_log2,
                                           const uint4 (&qf)[8], f32x4 (&o)[16], float& m,
                                           float& lsum, int n, int g) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int si = 0; si < 8; ++si) {
    s0 = mfma_f16(*reinterpret_cast<const uint4*>(kb + kswz(kcell(n), g + 4 * si)), qf[si], s0);
    s1 = mfma_f16(*reinterpret_cast<const uint4*>(kb + kswz(kcell(n) + 4, g + 4 * si)), qf[si], s1);
  }
  const bool full = pb >= lo && pb + 32 <= hi;
  float x[8];
  bool ok[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t q0 = pb + 8 * g + i, q1 = q0 + 4;  // cells of s0[i], s1[i]
    ok[i] = full || (q0 >= lo && q0 < hi);
    ok[4 + i] = full || (q1 >= lo && q1 < hi);
    x[i] = ok[i] ? s0[i] * scale_log2 : NEG_INF;
    x[4 + i] = ok[4 + i] ? s1[i] * scale_log2 : NEG_INF;
  }
  float bm = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) bm = fmaxf(bm, x[i]);
  bm = group4_max(bm);
  const float mnew = fmaxf(m, bm);
  const float muse = mnew == NEG_INF ? 0.f : mnew;
  const float alpha = __builtin_amdgcn_exp2f(m - muse);
  float pr[8], ps = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pr[i] = __builtin_amdgcn_exp2f(x[i] - muse);
    ps += pr[i];
  }
  lsum = lsum * alpha + ps;
  m = mnew;
  uint32_t pp[4], vm[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pp[i] = static_cast<uint32_t>(f32_to_f16_bits(pr[2 * i])) |
            (static_cast<uint32_t>(f32_to_f16_bits(pr[2 * i + 1])) << 16);
    vm[i] = (ok[2 * i] ? 0x0000ffffu : 0u) | (ok[2 * i + 1] ? 0xffff0000u : 0u);
  }
  const uint4 pf = make_uint4(pp[0], pp[1], pp[2], pp[3]);
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) {
    o[dt] *= alpha;
    const uint4 x = *reinterpret_cast<const uint4*>(vb + vswz(16 * dt + n, g));
    const uint4 v = make_uint4(x.x & vm[0], x.y & vm[1], x.z & vm[2], x.w & vm[3]);
    o[dt] = mfma_f16(v, pf, o[dt]);
  }
}

// Two 32-cell blocks that lie entirely inside the visible range: one
// softmax update for all 64 cells (one rescale of the outputs) and no
// masking of scores or values.
__device__ __forceinline__ void attn_pair_full(const uint16_t* kb0, const uint16_t* vb0,
                                               const uint16_t* kb1, const uint16_t* vb1,
                                               float scale_log2, const uint4 (&qf)[8],
                                               f32x4 (&o)[16], float& m, float& lsum, int n, int g) {
  f32x4 sc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) sc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int si = 0; si < 8; ++si) {
    const int c = g + 4 * si;
    const int c0 = kcell(n), c1 = c0 + 4;
    sc[0] = mfma_f16(*reinterpret_cast<const uint4*>(kb0 + kswz(c0, c)), qf[si], sc[0]);
    sc[1] = mfma_f16(*reinterpret_cast<const uint4*>(kb0 + kswz(c1, c)), qf[si], sc[1]);
    sc[2] = mfma_f16(*reinterpret_cast<const uint4*>(kb1 + kswz(c0, c)), qf[si], sc[2]);
    sc[3] = mfma_f16(*reinterpret_cast<const uint4*>(kb1 + kswz(c1, c)), qf[si], sc[3]);
  }
  float x[16];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[4 * q + i] = sc[q][i] * scale_log2;
  float bm = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) bm = fmaxf(bm, x[i]);
  bm = group4_max(bm);
  const float mnew = fmaxf(m, bm);
  const float alpha = __builtin_amdgcn_exp2f(m - mnew);
  float pr[16], ps = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    pr[i] = __builtin_amdgcn_exp2f(x[i] - mnew);
    ps += pr[i];
  }
  lsum = lsum * alpha + ps;
  m = mnew;
  uint32_t pp[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    pp[i] = static_cast<uint32_t>(f32_to_f16_bits(pr[2 * i])) |
            (static_cast<uint32_t>(f32_to_f16_bits(pr[2 * i + 1])) << 16);
  const uint4 pf0 = make_uint4(pp[0], pp[1], pp[2], pp[3]);
  const uint4 pf1 = make_uint4(pp[4], pp[5], pp[6], pp[7]);
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) {
    o[dt] *= alpha;
    const int d = 16 * dt + n;
    o[dt] = mfma_f16(*reinterpret_cast<const uint4*>(vb0 + vswz(d, g)), pf0, o[dt]);
    o[dt] = mfma_f16(*reinterpret_cast<const uint4*>(vb1 + vswz(d, g)), pf1, o[dt]);
  }
}

// The rows buffer: its nrows() <= 16 rows sit at cells kcell(r), so the
// first 16-row score tile alone covers them (the lanes of group g hold rows
// 4g .. 4g+3, cells 8g .. 8g+3: the first half of a value piece) and P.V
// takes 16-deep MFMAs; rows at or past nr are masked.
static_assert(2 * MAXB <= 16, "block and commit rows fit one score tile");
__device__ __forceinline__ void attn_rows16(const uint16_t* kb, const uint16_t* vb, int nr, float scale_log2,
                                            const uint4 (&qf)[8], f32x4 (&o)[16], float& m, float& lsum,
                                            int n, int g) {
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int si = 0; si < 8; ++si)
    s0 = mfma_f16(*reinterpret_cast<const uint4*>(kb + kswz(kcell(n), g + 4 * si)), qf[si], s0);
  float x[4];
  bool ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ok[i] = 4 * g + i < nr;
    x[i] = ok[i] ? s0[i] * scale_log2 : NEG_INF;
  }
  float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  bm = group4_max(bm);
  const float mnew = fmaxf(m, bm);
  const float muse = mnew == NEG_INF ? 0.f : mnew;
  const float alpha = __builtin_amdgcn_exp2f(m - muse);
  float pr[4], ps = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pr[i] = __builtin_amdgcn_exp2f(x[i] - muse);
    ps += pr[i];
  }
  lsum = lsum * alpha + ps;
  m = mnew;
  const uint2 pf = make_uint2(
      static_cast<uint32_t>(f32_to_f16_bits(pr[0])) | (static_cast<uint32_t>(f32_to_f16_bits(pr[1])) << 16),
      static_cast<uint32_t>(f32_to_f16_bits(pr[2])) | (static_cast<uint32_t>(f32_to_f16_bits(pr[3])) << 16));
  const uint32_t vm0 = (ok[0] ? 0x0000ffffu : 0u) | (ok[1] ? 0xffff0000u : 0u);
  const uint32_t vm1 = (ok[2] ? 0x0000ffffu : 0u) | (ok[3] ? 0xffff0000u : 0u);
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) {
    o[dt] *= alpha;
    const uint2 v = *reinterpret_cast<const uint2*>(vb + vswz(16 * dt + n, g));
    o[dt] = mfma_f16_k16(make_uint2(v.x & vm0, v.y & vm1), pf, o[dt]);
  }
}

// Query operand of this wave: qrow r = 16 t + n -> (row r / 12, head 12 j +
// r % 12); RMSNorm over the head (the lane holds 64 of its 256 values), then
// NeoX RoPE: dims 32 s + 8 g + e and 32 (s + 4) + 8 g + e form a pair.
__device__ __forceinline__ void attn_query_load(const PassArgs& a, int l, int j, int t, int n, int g,
                                                uint4 (&u)[8]) {
  const int r = t * 16 + n;
  const bool qv = r < G * a.B;
  const int bi = qv ? r / G : 0, hl = qv ? r % G : 0;
  const uint16_t* qraw = a.qkv + l * QSTRIDE + static_cast<size_t>(bi) * QKV_N + (j * G + hl) * D;
#pragma unroll
  for (int si = 0; si < 8; ++si) u[si] = gld<uint4>(qraw + 32 * si + 8 * g);
}

__device__ __forceinline__ void attn_query(const PassArgs& a, const Smem& s, int t, int n, int g,
                                           const uint4 (&u8)[8], uint4 (&qf)[8]) {
  const int r = t * 16 + n;
  const bool qv = r < G * a.B;
  const int bi = qv ? r / G : 0;
  float qv8[8][8];
#pragma unroll
  for (int si = 0; si < 8; ++si) {
    const uint4 u = u8[si];
    const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qv8[si][2 * i] = f16_bits_to_f32(static_cast<uint16_t>(uw[i]));
      qv8[si][2 * i + 1] = f16_bits_to_f32(static_cast<uint16_t>(uw[i] >> 16));
    }
  }
  float sq = 0.f;
#pragma unroll
  for (int si = 0; si < 8; ++si)
#pragma unroll
    for (int e = 0; e < 8; ++e) sq += qv8[si][e] * qv8[si][e];
  sq = group4_sum(sq);
  const float sc = 1.0f / sqrtf(sq / static_cast<float>(D) + a.eps);
  const uint16_t* gq = s.x + ATT_QG;
  const float2* rope = reinterpret_cast<const float2*>(s.x + ATT_ROPE);
  uint32_t pk[8][4];
#pragma unroll
  for (int si = 0; si < 4; ++si) {
    const uint4 ga = *reinterpret_cast<const uint4*>(gq + 32 * si + 8 * g);
    const uint4 gb = *reinterpret_cast<const uint4*>(gq + 32 * (si + 4) + 8 * g);
    const uint32_t gav[4] = {ga.x, ga.y, ga.z, ga.w}, gbv[4] = {gb.x, gb.y, gb.z, gb.w};
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      float lo2[2], hi2[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int ee = e + h2;
        const float ga_f = bf16_to_f32((gav[ee >> 1] >> (16 * (ee & 1))) & 0xffff);
        const float gb_f = bf16_to_f32((gbv[ee >> 1] >> (16 * (ee & 1))) & 0xffff);
        const float x0 = qv8[si][ee] * sc * ga_f, x1 = qv8[si + 4][ee] * sc * gb_f;
        const float2 cs = rope[bi * (D / 2) + 32 * si + 8 * g + ee];
        lo2[h2] = x0 * cs.x - x1 * cs.y;
        hi2[h2] = x1 * cs.x + x0 * cs.y;
      }
      pk[si][e >> 1] = static_cast<uint32_t>(f32_to_f16_bits(lo2[0])) |
                       (static_cast<uint32_t>(f32_to_f16_bits(lo2[1])) << 16);
      pk[si + 4][e >> 1] = static_cast<uint32_t>(f32_to_f16_bits(hi2[0])) |
                           (static_cast<uint32_t>(f32_to_f16_bits(hi2[1])) << 16);
    }
  }
#pragma unroll
  for (int si = 0; si < 8; ++si)
    qf[si] = qv ? make_uint4(pk[si][0], pk[si][1], pk[si][2], pk[si][3]) : make_uint4(0, 0, 0, 0);
}

// Block rows' keys and values of KV head j into LDS (the block layouts: keys
// [32][256], values [256][32]; row r of the rows buffer at cell kcell(r),
// where the first score tile reads it); wave b = row b.  With commit rows
// (the fused draft-commit cycle), wave t also finishes commit row t: k-norm
// and RoPE at pos0 + t on its raw fp32 projection, fp16 K and V written to
// the ring cell of that position (read by later passes), and -- when the
// position is inside the window -- the same fp16 key and value as row
// B + t - t0 of the rows buffer (t0 = the first visible commit row), so it
// holds nrows() rows.
__device__ __forceinline__ int commit_first_visible(const PassArgs& a) {
  const int64_t d = a.lo - a.pos0;
  return d <= 0 ? 0 : (d >= a.nc ? a.nc : static_cast<int>(d));
}
__device__ __forceinline__ int nrows(const PassArgs& a) {
  return a.B + a.nc - commit_first_visible(a);
}

__device__ __forceinline__ void attn_block_rows(const PassArgs& a, const Smem& s, int l, int j,
                                                uint16_t* kl, uint16_t* vl) {
  const int wave = wid(), lane = otid() & 63;
  const uint16_t* gn = s.x + ATT_KG;
  const float2* rope = reinterpret_cast<const float2*>(s.x + ATT_ROPE);
  float gk[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) gk[q] = bf16_to_f32(gn[lane + 64 * q]);
  if (wave < a.B) {
    const int b = wave;
    const uint16_t* kr = a.qkv + l * QSTRIDE + static_cast<size_t>(b) * QKV_N + NQ * D + j * D;
    const uint16_t* vr = kr + NKV * D;
    float k0 = f16_bits_to_f32(gld<uint16_t>(kr + lane)), k1 = f16_bits_to_f32(gld<uint16_t>(kr + lane + 64));
    float k2 = f16_bits_to_f32(gld<uint16_t>(kr + lane + 128)), k3 = f16_bits_to_f32(gld<uint16_t>(kr + lane + 192));
    float vv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) vv[q] = f16_bits_to_f32(gld<uint16_t>(vr + lane + 64 * q));
    const float sq = wave_sum(k0 * k0 + k1 * k1 + k2 * k2 + k3 * k3);
    const float sc = 1.0f / sqrtf(sq / static_cast<float>(D) + a.eps);
    k0 *= sc * gk[0];
    k1 *= sc * gk[1];
    k2 *= sc * gk[2];
    k3 *= sc * gk[3];
    const float2 c0 = rope[b * (D / 2) + lane];
    const float2 c1 = rope[b * (D / 2) + lane + 64];
    const float kv[4] = {k0 * c0.x - k2 * c0.y, k1 * c1.x - k3 * c1.y, k2 * c0.x + k0 * c0.y,
                         k3 * c1.x + k1 * c1.y};
    const int cell = kcell(b);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = lane + 64 * q;
      kl[kswz(cell, d >> 3) + (d & 7)] = f32_to_f16_bits(kv[q]);
      vl[vel(d, cell)] = f32_to_f16_bits(vv[q]);
    }
  }
  if (wave < a.nc) {
    const int t = wave;
    const float* kr = a.ckv + (static_cast<size_t>(l) * MAXB + t) * (2 * NKV * D) + j * D;
    const float* vr = kr + NKV * D;
    float k[4], vv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      k[q] = gld<float>(kr + lane + 64 * q);
      vv[q] = gld<float>(vr + lane + 64 * q);
    }
    const float sq = wave_sum(k[0] * k[0] + k[1] * k[1] + k[2] * k[2] + k[3] * k[3]);
    const float sc = 1.0f / sqrtf(sq / static_cast<float>(D) + a.eps);
#pragma unroll
    for (int q = 0; q < 4; ++q) k[q] *= sc * gk[q];
    const float2 c0 = rope[(MAXB + t) * (D / 2) + lane];
    const float2 c1 = rope[(MAXB + t) * (D / 2) + lane + 64];
    const float kv[4] = {k[0] * c0.x - k[2] * c0.y, k[1] * c1.x - k[3] * c1.y,
                         k[2] * c0.x + k[0] * c0.y, k[3] * c1.x + k[1] * c1.y};
    const int cell = static_cast<int>((a.pos0 + t) % a.cap);
    uint16_t* rk = const_cast<uint16_t*>(a.ring_k) + ((static_cast<size_t>(l) * NKV + j) * a.cap + cell) * D;
    uint16_t* rv = const_cast<uint16_t*>(a.ring_vt) + (static_cast<size_t>(l) * NKV + j) * D * a.cap +
                   static_cast<size_t>(cell / BLK_CELLS) * D * BLK_CELLS + cell % BLK_CELLS;
    const int t0 = commit_first_visible(a);
    const int c = kcell(a.B + t - t0);  // LDS cell of a visible commit row
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = lane + 64 * q;
      const uint16_t kb = f32_to_f16_bits(kv[q]), vb = f32_to_f16_bits(vv[q]);
      gst16(rk + d, kb);
      gst16(rv + static_cast<size_t>(d) * BLK_CELLS, vb);
      if (t >= t0) {
        kl[kswz(c, d >> 3) + (d & 7)] = kb;
        vl[vel(d, c)] = vb;
      }
    }
  }
}

__device__ __forceinline__ void attn_phase(const PassArgs& a, Smem& s, int l) {
  const int w = blockIdx.x;
  if (w < NKV * a.nch) {
    const int j = w / a.nch, c = w % a.nch;
    const int wave = wid(), lane = otid() & 63;
    const int n = lane & 15, g = lane >> 4;
    const int blk0 = c * a.cb;
    const int nblk = a.nb > blk0 ? min(a.cb, a.nb - blk0) : 0;
    const bool rows = c == a.nch - 1;  // this chunk also takes the block rows
    // LDS: block buffers (keys then values) at 0 and 2 x 8192, block rows at 4 x 8192
    uint16_t* kl = s.x + 4 * BLK_CELLS * D;
    uint16_t* vl = s.x + 5 * BLK_CELLS * D;
    uint4 qf[8];
    {
      uint4 u[8];
      if (wave < a.nqt) attn_query_load(a, l, j, wave, n, g, u);
      // the staged gains and RoPE rows -- wave 7's loads before its
      // KV_DMA_LOADS K/V loads -- are in LDS
      if (wave == ACT_WAVE) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KV_DMA_LOADS) : "memory");
      lds_sync();
      if (wave < a.nqt) attn_query(a, s, wave, n, g, u, qf);
    }
    // the first pair's K/V has landed once the K/V waves' loads are done
    if (wave >= KV_DMA_W0) wait_stores();
    if (rows) attn_block_rows(a, s, l, j, kl, vl);
    float m = NEG_INF, lsum = 0.f;
    f32x4 o[16];
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Blocks go through LDS in pairs (buffers at 0 and 2 x 8192; the first
    // pair is already there, later ones are stored from registers), run
    // together -- in one softmax update when both lie entirely inside the
    // visible range.
    KVRegs R0, R1;
    uint16_t* k0b = s.x;
    uint16_t* v0b = k0b + BLK_CELLS * D;
    uint16_t* k1b = s.x + 2 * BLK_CELLS * D;
    uint16_t* v1b = k1b + BLK_CELLS * D;
    for (int ib = 0; ib < nblk; ib += 2) {
      const bool two = ib + 1 < nblk;
      if (ib > 0) {
        lds_sync();  // every wave is done with the previous pair
        attn_store(R0, k0b, v0b);
        if (two) attn_store(R1, k1b, v1b);
      }
      lds_sync();
      if (wave < a.nqt) {
        const int64_t pb0 = a.p0 + 32 * static_cast<int64_t>(blk0 + ib), pb1 = pb0 + 32;
        const bool f0 = pb0 >= a.lo && pb0 + 32 <= a.hi;
        const bool f1 = two && pb1 >= a.lo && pb1 + 32 <= a.hi;
        if (f0 && f1) {
          attn_pair_full(k0b, v0b, k1b, v1b, a.scale_log2, qf, o, m, lsum, n, g);
        } else {
          attn_block(k0b, v0b, pb0, a.lo, a.hi, a.scale_log2, qf, o, m, lsum, n, g);
          if (two) attn_block(k1b, v1b, pb1, a.lo, a.hi, a.scale_log2, qf, o, m, lsum, n, g);
        }
      }
      // next pair (long contexts): loaded after this pair ran, so that the
      // register slots are free while it runs
      attn_load(a, l, blk0 + ib + 2, j, R0, ib + 2 < nblk);
      attn_load(a, l, blk0 + ib + 3, j, R1, ib + 3 < nblk);
    }
    if (rows) {
      lds_sync();
      if (wave < a.nqt) attn_rows16(kl, vl, nrows(a), a.scale_log2, qf, o, m, lsum, n, g);
    }
    if (wave < a.nqt) {
      lsum = group4_sum(lsum);
      if (g == 0) {
        // [head][query tile][row][chunk]: a group's chunks side by side for the merge
        const size_t mi = ((static_cast<size_t>(j) * a.nqt + wave) * 16 + n) * NCH_PASS + c;
        st_cohf(a.pm + l * PMSTRIDE + mi, m);
        st_cohf(a.pl + l * PMSTRIDE + mi, lsum);
      }
    }
    // The normalised chunk output leaves through LDS: a lane holds 4 dims of
    // one query row per 16-dim tile, so direct stores would write 32-byte
    // pieces of 16 rows per instruction; staged as rows (stride D + 8), each
    // store instruction writes two whole 512-byte rows, 16 bytes per lane.
    lds_sync();  // every wave is done with the K/V blocks in s.x
    if (wave < a.nqt) {
      constexpr int RS = D + 8;
      uint16_t* st = s.x + wave * 16 * RS;
      const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
#pragma unroll
      for (int dt = 0; dt < 16; ++dt) {
        const uint32_t lo = static_cast<uint32_t>(f32_to_f16_bits(o[dt][0] * inv)) |
                            (static_cast<uint32_t>(f32_to_f16_bits(o[dt][1] * inv)) << 16);
        const uint32_t hi = static_cast<uint32_t>(f32_to_f16_bits(o[dt][2] * inv)) |
                            (static_cast<uint32_t>(f32_to_f16_bits(o[dt][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(st + n * RS + 16 * dt + 4 * g) = make_uint2(lo, hi);
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // 16-byte stores with the agent-scope stores' cache policy (sc1:
      // visible to the other XCDs once acknowledged), through a buffer
      // resource over this wave's 16 rows
      const size_t base = (static_cast<size_t>(j) * a.nch + c) * a.nqt + wave;
      const __amdgpu_buffer_rsrc_t ro = buf_rsrc(a.po + l * POSTRIDE + base * 16 * D, 16 * D * 2);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int row = 2 * k + (lane >> 5), c8 = lane & 31;
        __builtin_amdgcn_raw_buffer_store_b128(
            *reinterpret_cast<const u32x4*>(st + row * RS + 8 * c8), ro,
            2 * (row * D + 8 * c8), 0, CPOL_SC1);
      }
    }
  }
  wait_stores();
}

// Merge of the chunks of one (KV head, query tile, query row) -- a group.
// The last `groups` blocks (192 at 8 block rows; the launch requires a grid
// at least that large) merge one group each.  32 threads cover the 256 head
// dims of one chunk (8 each) and 16 such slots take chunks slot, slot + 16,
// ... with 16-byte loads; wave 0 turns the chunks' maxima and sums into
// weights w_c = 2^(m_c - M) l_c (chunk outputs are already normalised by
// l_c).  The maxima and sums are loaded before the chunk outputs, so the
// weights wait only for them; they are laid out [head][query tile][row]
// [chunk], so a group's 128 maxima are 512 contiguous bytes (with the chunk
// outputs' layout they would sit 384 bytes apart, a cache line each).  Partials of this layer were written once, so
// plain loads read them.  (Two groups per block on the last 96 blocks, which
// left the first 160 free to start their O-projection prefetch at once, was
// 3 us per pass slower.)
constexpr int MRG_U = NCH_PASS / 16;  // chunks per slot (8)

template <int FMT>
__device__ __forceinline__ void merge_phase(const PassArgs& a, Smem& s, int l) {
  const int ngroup = NKV * a.nqt * 16;
  const int w0 = gridDim.x - ngroup;
  if (blockIdx.x >= w0) {
    const int tid = otid(), lane = tid & 63;
    const int grp = blockIdx.x - w0;
    const int gc = grp < ngroup ? grp : 0;  // addresses stay inside the partials
    const int n = gc & 15, t = (gc >> 4) % a.nqt, j = (gc >> 4) / a.nqt;
    const bool act = grp < ngroup && t * 16 + n < G * a.B;
    const int nc = a.nch;
    const size_t cstride = static_cast<size_t>(a.nqt) * 16;
    const size_t row0 = (static_cast<size_t>(j) * nc * a.nqt + t) * 16 + n;
    const size_t mrow = ((static_cast<size_t>(j) * a.nqt + t) * 16 + n) * NCH_PASS;
    const uint16_t* po = a.po + l * POSTRIDE;
    const float* pm = a.pm + l * PMSTRIDE;
    const float* pl = a.pl + l * PMSTRIDE;
    const int slot = tid >> 5, dp = tid & 31;
    float mraw[2], lraw[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = lane + 64 * q;
      mraw[q] = gld<float>(pm + mrow + (c < nc ? c : 0));
      lraw[q] = gld<float>(pl + mrow + (c < nc ? c : 0));
    }
    uint4 ov[MRG_U];
#pragma unroll
    for (int u = 0; u < MRG_U; ++u) {
      const int c = slot + 16 * u;
      ov[u] = gld<uint4>(po + (row0 + (c < nc ? c : 0) * cstride) * D + 8 * dp);  // c >= nc: unused
    }
    if (wid() == 0) {  // chunk weights
      float mv[2], lv[2];
      float M = NEG_INF;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int c = lane + 64 * q;
        mv[q] = act && c < nc ? mraw[q] : NEG_INF;
        lv[q] = act && c < nc ? lraw[q] : 0.f;
        M = fmaxf(M, mv[q]);
      }
      M = wave_max(M);
      float Ls = 0.f;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int c = lane + 64 * q;
        const float wt = act && c < nc ? exp2f(mv[q] - M) * lv[q] : 0.f;
        s.mw[c] = wt;
        Ls += wt;
      }
      Ls = wave_sum(Ls);
      if (lane == 0) s.scal[0] = Ls > 0.f ? 1.0f / Ls : 0.f;
    }
    lds_sync();
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int u = 0; u < MRG_U; ++u) {
      const int c = slot + 16 * u;
      if (c < nc) {
        const float wt = s.mw[c];
        const uint32_t wd[4] = {ov[u].x, ov[u].y, ov[u].z, ov[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += f16_bits_to_f32(static_cast<uint16_t>(wd[i])) * wt;
          acc[2 * i + 1] += f16_bits_to_f32(static_cast<uint16_t>(wd[i] >> 16)) * wt;
        }
      }
    }
    // slots 1..15 hand their sums to slot 0 (fixed order: deterministic)
    float* red = reinterpret_cast<float*>(s.x);  // [16][256]
    if (slot > 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) red[slot * D + 8 * dp + i] = acc[i];
    }
    lds_sync();
    if (slot == 0 && act) {
      for (int sl = 1; sl < 16; ++sl) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += red[sl * D + 8 * dp + i];
      }
      const float sc = s.scal[0];
      uint32_t pk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pk[i] = static_cast<uint32_t>(act16<FMT>(acc[2 * i] * sc)) |
                (static_cast<uint32_t>(act16<FMT>(acc[2 * i + 1] * sc)) << 16);
      const int r = t * 16 + n, bi = r / G, hl = r % G;
      st_coh128(a.o16 + l * OSTRIDE + static_cast<size_t>(bi) * NQ * D + (j * G + hl) * D + 8 * dp,
                make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }
  }
  wait_stores();
}

// O projection: block w < 160 owns row tile w; wave v takes k in
// [768 v, 768 v + 768) (6 k blocks).
template <int FMT> using OTile = WTile<FMT, 768 / KPerLoad<FMT>::v>;

template <int FMT>
__device__ __forceinline__ void o_prefetch(const PassArgs& a, int l, OTile<FMT>& W, bool go) {
  const int w = blockIdx.x, wave = wid(), lane = otid() & 63;
  const bool has = w < NT_H;
  constexpr int N = 768 / KPerLoad<FMT>::v;
  load_wt<FMT, N>(W, WMat{ctab(a)->wo[l], H, NQ * D}, (has ? w : 0) * 16 + (lane & 15), wave * 768,
                  lane >> 4, N, go && has);
}

template <int FMT>
__device__ __forceinline__ void o_phase(const PassArgs& a, Smem& s, int l, OTile<FMT>& W) {
  const int w = blockIdx.x, wave = wid(), lane = otid() & 63;
  const int r = lane & 15, g = lane >> 4;
  if (w < NT_H) {
    if (act_wave()) {  // attention output rows straight into LDS, then its weight slice
      stage_rows<NQ * D>(a, s, a.o16 + l * OSTRIDE);
      staged_wait();
      o_prefetch<FMT>(a, l, W, true);
    }
    const float4 hres = residual_load(a, w, r, g, 2 * l);  // used by wave 0
    lds_sync();
    constexpr int XS = NQ * D + XS_PAD;
    constexpr int N = 768 / KPerLoad<FMT>::v;
    f32x4 acc = mma_wt<FMT, N>(W, s.x + xrow(r, a.B) * XS, wave * 768, g, N);
    s.red[wave][lane] = acc;
    lds_sync();
    if (wave == 0) residual_epilogue(a, group_sum(s, 0, NWAVE, lane), hres, w, r, g, 2 * l);
  }
  wait_stores();
}

// Gate/up: 480 tile pairs; round q handles pair w + q * grid.  Waves 0-3 the
// gate tile's k quarters, waves 4-7 the up tile's.
template <int FMT> using GuTile = WTile<FMT, 640 / KPerLoad<FMT>::v>;

template <int FMT>
__device__ __forceinline__ void gu_prefetch(const PassArgs& a, int l, int pair, GuTile<FMT>& W,
                                            bool go) {
  const int wave = wid(), lane = otid() & 63;
  const bool has = pair < F / 16;
  constexpr int N = 640 / KPerLoad<FMT>::v;
  load_wt<FMT, N>(W, WMat{wave < 4 ? ctab(a)->wg[l] : ctab(a)->wu[l], F, H},
                  (has ? pair : 0) * 16 + (lane & 15), (wave & 3) * 640, lane >> 4, N, go && has);
}

// One gate/up tile pair from the weights in W: reduce the k quarters, write
// silu(gate) * up for the block rows.
template <int FMT>
__device__ __forceinline__ void gu_round(const PassArgs& a, Smem& s, int l, int pair,
                                         const GuTile<FMT>& W) {
  const int wave = wid(), lane = otid() & 63;
  const int r = lane & 15, g = lane >> 4;
  constexpr int XS = H + XS_PAD;
  constexpr int N = 640 / KPerLoad<FMT>::v;
  f32x4 acc = mma_wt<FMT, N>(W, s.x + xrow(r, a.B) * XS, (wave & 3) * 640, g, N);
  s.red[wave][lane] = acc;
  lds_sync();
  if (wave == 0) {
    const f32x4 ag = group_sum(s, 0, 4, lane);
    const f32x4 au = group_sum(s, 4, 4, lane);
    if (r < a.B) {
      uint16_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float z = ag[i];
        o[i] = act16<FMT>(z / (1.0f + __expf(-z)) * au[i]);
      }
      st_coh64(a.u16 + l * USTRIDE + static_cast<size_t>(r) * F + pair * 16 + 4 * g,
               static_cast<uint64_t>(o[0] | (static_cast<uint32_t>(o[1]) << 16)) |
                   (static_cast<uint64_t>(o[2] | (static_cast<uint32_t>(o[3]) << 16)) << 32));
    }
  }
  lds_sync();  // red[] reuse
}

// The first pair's tiles were prefetched before the barrier (wave 0: during
// it); the second pair's go out right behind the activation loads, into
// a second register tile, so that they stream while the first pair runs.
// Grids under 240 blocks take further pairs one at a time.
template <int FMT>
__device__ __forceinline__ void gu_phase(const PassArgs& a, Smem& s, int l, int np, GuTile<FMT>& W) {
  const int w = blockIdx.x, wave = wid();
  const bool has = w < F / 16;
  if (has) {
    XnRegs x;
    xn_load(a, x, 2 * l + 1, np, ctab(a)->post_norm[l]);
    // Unconditional: a block without a second pair re-reads its first (no
    // branch, so the norm below waits only for the activation loads).
    GuTile<FMT> W2;
    const int p2 = w + gridDim.x;
    {
      const int lane = otid() & 63;
      constexpr int N = 640 / KPerLoad<FMT>::v;
      load_wt<FMT, N>(W2, WMat{wave < 4 ? ctab(a)->wg[l] : ctab(a)->wu[l], F, H},
                      (p2 < F / 16 ? p2 : w) * 16 + (lane & 15), (wave & 3) * 640, lane >> 4, N,
                      true);
    }
    xn_finish<FMT>(a, s, x);
    gu_round<FMT>(a, s, l, w, W);
    if (p2 < F / 16) gu_round<FMT>(a, s, l, p2, W2);
    for (int pair = p2 + gridDim.x; pair < F / 16; pair += gridDim.x) {
      gu_prefetch<FMT>(a, l, pair, W, true);
      gu_round<FMT>(a, s, l, pair, W);
    }
  }
  wait_stores();
}

// Down projection: block w < 160 owns row tile w and wave v a k range: 960
// each for bf16 and Q8_0 (30 and 15 loads); Q4_0 / Q5_0 loads cover 128 k,
// so their waves 0-3 take 1024 (k < 4096) and waves 4-7 take 896.
template <int FMT>
__device__ __forceinline__ void down_range(int wave, int& kbeg, int& klen) {
  if constexpr (!nibble_fmt(FMT)) {
    kbeg = wave * (F / NWAVE);
    klen = F / NWAVE;
  } else if (wave < 4) {
    kbeg = wave * 1024;
    klen = 1024;
  } else {
    kbeg = 4096 + (wave - 4) * 896;
    klen = 896;
  }
}

template <int FMT>
using DownTile = WTile<FMT, (nibble_fmt(FMT) ? 1024 : F / NWAVE) / KPerLoad<FMT>::v>;

// Down projection tile w for blocks w < 160.  Only waves 0..DOWN_PRE_LAST
// load their k range at the barrier that ends the gate/up phase (which those
// blocks spend streaming two gate/up tile pairs); the others load theirs at
// the start of the phase, behind the activations.
constexpr int DOWN_PRE_LAST = 3;

__device__ __forceinline__ bool down_pre(int wave) { return wave <= DOWN_PRE_LAST; }

template <int FMT>
__device__ __forceinline__ void down_prefetch(const PassArgs& a, int l, DownTile<FMT>& W, bool go) {
  const int w = blockIdx.x, wave = wid(), lane = otid() & 63;
  const bool has = w < NT_H;
  int kbeg, klen;
  down_range<FMT>(wave, kbeg, klen);
  constexpr int N = sizeof(W.q) / sizeof(uint4);
  load_wt<FMT, N>(W, WMat{ctab(a)->wd[l], H, F}, (has ? w : 0) * 16 + (lane & 15), kbeg, lane >> 4,
                  klen / KPerLoad<FMT>::v, go && has);
}

template <int FMT>
__device__ __forceinline__ void down_phase(const PassArgs& a, Smem& s, int l, DownTile<FMT>& W) {
  const int w = blockIdx.x, wave = wid(), lane = otid() & 63;
  const int r = lane & 15, g = lane >> 4;
  const int tile = w;
  if (w < NT_H) {
    if (act_wave()) {  // MLP product rows straight into LDS
      stage_rows<F>(a, s, a.u16 + l * USTRIDE);
      staged_wait();
    }
    if (wave > DOWN_PRE_LAST) down_prefetch<FMT>(a, l, W, true);
    const float4 hres = residual_load(a, tile, r, g, 2 * l + 1);  // used by wave 0
    lds_sync();
    int kbeg, klen;
    down_range<FMT>(wave, kbeg, klen);
    constexpr int XS = F + XS_PAD;
    constexpr int N = sizeof(W.q) / sizeof(uint4);
    f32x4 acc = mma_wt<FMT, N>(W, s.x + xrow(r, a.B) * XS, kbeg, g, klen / KPerLoad<FMT>::v);
    s.red[wave][lane] = acc;
    lds_sync();
    if (wave == 0)
      residual_epilogue(a, group_sum(s, 0, NWAVE, lane), hres, tile, r, g, 2 * l + 1);
  }
  wait_stores();
}

// LM head: tile pairs p = w, w + grid, ...; wave v takes tile 2p + v/4 and k
// quarter v%4.  Activations: final-normed rows 1..B-1 (row b in LDS row b),
// bf16 next to a bf16 LM head, fp16 next to a Q8_0 one (decoded in registers
// like the quantized layer matrices: one load carries 64 k and its scale).
template <int LMF> using LmTile = WTile<LMF, 640 / KPerLoad<LMF>::v>;

template <int LMF>
__device__ __forceinline__ void lm_prefetch(const PassArgs& a, int pair, LmTile<LMF>& W, bool go) {
  const int wave = wid(), lane = otid() & 63;
  const int tile = 2 * pair + (wave >> 2);
  const bool has = tile < a.vocab / 16;
  const int row = (has ? tile : 0) * 16 + (lane & 15);
  if constexpr (LMF == W_BF16) {
    load_tile<20>(W.q, a.lm, H, row, (wave & 3) * 640, lane >> 4, 20, go && has);
    W.s[0] = 0u;
  } else {
    constexpr int N = 640 / KPerLoad<LMF>::v;
    load_wt<LMF, N>(W, WMat{a.lm, a.vocab, H}, row, (wave & 3) * 640, lane >> 4, N, go && has);
  }
}

template <int LMF>
__device__ __forceinline__ f32x4 lm_mma(const LmTile<LMF>& W, const uint16_t* xr, int g) {
  const int kbeg = (wid() & 3) * 640;
  if constexpr (LMF == W_BF16) return mma_tile<20>(W.q, xr, kbeg, g, 20);
  else return mma_wt<LMF, 640 / KPerLoad<LMF>::v>(W, xr, kbeg, g, 640 / KPerLoad<LMF>::v);
}

__device__ __forceinline__ uint64_t umax64(uint64_t x, uint64_t y) { return x > y ? x : y; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
  lo = __shfl_xor(lo, m, 64);
  hi = __shfl_xor(hi, m, 64);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Online log-sum-exp state (m, s) of a set of logits: m their maximum, s the
// sum of exp(l - m).  Merging two states rescales both sums to the larger
// maximum; an empty state is (-inf, 0).
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = s * expf(m - M) + s2 * expf(m2 - M);
  m = M;
}
// Adds one logit v to a state with a single exponential: the smaller of v
// and m is scaled by exp(-|v - m|), on the hardware exp2 (exp(x) =
// 2^(x log2 e); -inf -> 0, so the empty state takes its first value exactly).
__device__ __forceinline__ void lse_add(float& m, float& s, float v) {
  const float d = v - m;
  const float e = __builtin_amdgcn_exp2f(-fabsf(d) * 1.4426950408889634f);
  const bool up = d > 0.f;
  s = up ? fmaf(s, e, 1.f) : s + e;
  m = up ? v : m;
}
__device__ __forceinline__ uint64_t lse_pack(float m, float s) {
  return static_cast<uint64_t>(__float_as_uint(m)) |
         (static_cast<uint64_t>(__float_as_uint(s)) << 32);
}
__device__ __forceinline__ void lse_unpack(uint64_t v, float& m, float& s) {
  m = __uint_as_float(static_cast<uint32_t>(v));
  s = __uint_as_float(static_cast<uint32_t>(v >> 32));
}

// hidden_opt rows (bf16) from the final-normed LDS rows: copied when they
// are bf16, converted when they are fp16 (next to a Q8_0 LM head).
template <int XF>
__device__ __forceinline__ void write_hidden(const PassArgs& a, const Smem& s) {
  constexpr int XS = H + XS_PAD;
  for (int e = otid(); e < a.B * H; e += NTHR) {
    const uint16_t v = s.x[(e / H) * XS + (e % H)];
    a.hidden[e] = XF == W_BF16 ? v : f32_to_bf16(f16_bits_to_f32(v));
  }
}

template <int LMF>
__device__ __forceinline__ void lm_phase(const PassArgs& a, Smem& s, int np, LmTile<LMF>& W) {
  const int w = blockIdx.x, wave = wid(), lane = otid() & 63;
  const int r = lane & 15, g = lane >> 4;
  const int ntiles = a.vocab / 16, npairs = (ntiles + 1) / 2;
  build_x_norm_staged<LMF>(a, s, 2 * L, np, a.final_norm, [&] {
    if (a.B > 1) lm_prefetch<LMF>(a, w, W, true);
  });
  constexpr int XS = H + XS_PAD;
  if (w == 0 && a.hidden) write_hidden<LMF>(a, s);
  // mask row r + 1 of the block feeds MFMA column r
  const bool xv = r + 1 < a.B;
  const uint16_t* xr = s.x + (xv ? r + 1 : 1) * XS;
  uint64_t best = 0;
  float lm = -INFINITY, ls = 0.f;  // softmax state of this lane's logits
  LmTile<LMF> W2;
  int p = w;
  while (p < npairs) {
    // round with W, prefetch into W2
    const int pn = p + gridDim.x;
    lm_prefetch<LMF>(a, pn, W2, pn < npairs);
    const int tile = 2 * p + (wave >> 2);
    f32x4 acc = tile < ntiles ? lm_mma<LMF>(W, xr, g) : f32x4{0.f, 0.f, 0.f, 0.f};
    s.red[wave][lane] = acc;
    lds_sync();
    if ((wave & 3) == 0 && tile < ntiles) {
      acc = group_sum(s, wave, 4, lane);
      if (xv) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          best = umax64(best, argmax_key(acc[i], static_cast<uint32_t>(tile * 16 + 4 * g + i)));
        if (a.conf) {
#pragma unroll
          for (int i = 0; i < 4; ++i) lse_add(lm, ls, acc[i]);
        }
        if (a.logits) {
          uint16_t o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16(acc[i]);
          *reinterpret_cast<uint2*>(a.logits + static_cast<size_t>(r) * a.vocab + tile * 16 + 4 * g) =
              make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16),
                         o[2] | (static_cast<uint32_t>(o[3]) << 16));
        }
      }
    }
    lds_sync();
    p = pn;
    if (p >= npairs) break;
    // round with W2, prefetch into W
    const int pn2 = p + gridDim.x;
    lm_prefetch<LMF>(a, pn2, W, pn2 < npairs);
    const int tile2 = 2 * p + (wave >> 2);
    acc = tile2 < ntiles ? lm_mma<LMF>(W2, xr, g) : f32x4{0.f, 0.f, 0.f, 0.f};
    s.red[wave][lane] = acc;
    lds_sync();
    if ((wave & 3) == 0 && tile2 < ntiles) {
      acc = group_sum(s, wave, 4, lane);
      if (xv) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          best = umax64(best, argmax_key(acc[i], static_cast<uint32_t>(tile2 * 16 + 4 * g + i)));
        if (a.conf) {
#pragma unroll
          for (int i = 0; i < 4; ++i) lse_add(lm, ls, acc[i]);
        }
        if (a.logits) {
          uint16_t o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16(acc[i]);
          *reinterpret_cast<uint2*>(a.logits + static_cast<size_t>(r) * a.vocab + tile2 * 16 + 4 * g) =
              make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16),
                         o[2] | (static_cast<uint32_t>(o[3]) << 16));
        }
      }
    }
    lds_sync();
    p = pn2;
  }
  // per-block best of mask row r + 1: waves 0 and 4 hold candidates
  if ((wave & 3) == 0) {
    best = umax64(best, shfl_xor_u64(best, 16));
    best = umax64(best, shfl_xor_u64(best, 32));
    if (g == 0) s.best[wave >> 2][r] = best;
    if (a.conf) {
#pragma unroll
      for (int o = 16; o < 64; o <<= 1)
        lse_merge(lm, ls, __shfl_xor(lm, o, 64), __shfl_xor(ls, o, 64));
      if (g == 0) s.lse[wave >> 2][r] = make_float2(lm, ls);
    }
  }
  lds_sync();
  if (otid() < MAXB) {
    st_coh64(a.keys + static_cast<size_t>(w) * MAXB + otid(),
             umax64(s.best[0][otid()], s.best[1][otid()]));
    if (a.conf) {
      float m = s.lse[0][otid()].x, sm = s.lse[0][otid()].y;
      lse_merge(m, sm, s.lse[1][otid()].x, s.lse[1][otid()].y);
      st_coh64(a.lse + static_cast<size_t>(w) * MAXB + otid(), lse_pack(m, sm));
    }
  }
  wait_stores();
}

// ---------------------------------------------------------------- device-resident positions

// The pass's positions from dstate = {p, anchor, nc} and the derived split
// of the visible context, computed the way the host computes them for the
// host-argument entry points: the ring is read at [lo, hi) with lo = max(0,
// p - window), hi = p - nc; 32-cell blocks from p0 = lo rounded down to 32;
// at most maxch chunks per KV head.  ok = false when the state is outside
// what the host entry points accept (then nothing may be read from it).
struct PosState {
  int64_t p, lo, hi, p0, pos0;
  int nb, cb, nch, nc, anchor;
  bool ok;
};

__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint64_t u = static_cast<uint64_t>(v);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ PosState resolve_positions(const int64_t* st, int64_t window, int maxch,
                                                      int vocab, int64_t taps_pos0,
                                                      int64_t taps_rows) {
  PosState r;
  r.p = uni64(static_cast<int64_t>(ld_coh64(st)));
  const int64_t anchor = uni64(static_cast<int64_t>(ld_coh64(st + 1)));
  const int64_t nc = uni64(static_cast<int64_t>(ld_coh64(st + 2)));
  r.ok = r.p >= 0 && nc >= 0 && nc <= MAXB && r.p >= nc && anchor >= 0 && anchor < vocab &&
         (nc == 0 || (r.p - nc >= taps_pos0 && r.p <= taps_pos0 + taps_rows));
  r.nc = r.ok ? static_cast<int>(nc) : 0;
  r.anchor = r.ok ? static_cast<int>(anchor) : 0;
  r.lo = r.p - window > 0 ? r.p - window : 0;
  r.hi = r.p - r.nc;
  r.pos0 = r.hi;
  if (r.ok && r.hi > r.lo) {
    r.p0 = r.lo & ~static_cast<int64_t>(31);
    r.nb = static_cast<int>((r.hi - r.p0 + 31) / 32);
    r.cb = (r.nb + maxch - 1) / maxch;
    r.nch = (r.nb + r.cb - 1) / r.cb;
  } else {
    r.p0 = 0;
    r.nb = 0;
    r.cb = 1;
    r.nch = 1;
  }
  return r;
}

__device__ __forceinline__ void argmax_final(const PassArgs& a, Smem& s) {
  if (blockIdx.x != 0) return;
  const int wave = wid(), lane = otid() & 63;
  // a grid barrier that gave up waiting leaves the pass's results undefined:
  // report it through the candidates
  const bool timed_out = ld_coh32(a.bar + BAR_STATUS) != 0u;
  if (wave + 1 < a.B) {  // wave b reduces mask row b + 1
    uint64_t best = 0;
    for (int i = lane; i < static_cast<int>(gridDim.x); i += 64)
      best = umax64(best, ld_coh64(a.keys + static_cast<size_t>(i) * MAXB + wave));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) best = umax64(best, shfl_xor_u64(best, o));
    if (lane == 0) a.cand[wave] = timed_out ? -1 : static_cast<int32_t>(~static_cast<uint32_t>(best));
    if (a.conf) {
      // p(cand) = exp(l_max - logsumexp(l)) = 1 / sum_v exp(l_v - l_max):
      // the state's maximum is the candidate's own logit
      float m = -INFINITY, sm = 0.f;
      for (int i = lane; i < static_cast<int>(gridDim.x); i += 64) {
        float m2, s2;
        lse_unpack(ld_coh64(a.lse + static_cast<size_t>(i) * MAXB + wave), m2, s2);
        lse_merge(m, sm, m2, s2);
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1)
        lse_merge(m, sm, __shfl_xor(m, o, 64), __shfl_xor(sm, o, 64));
      const float c = timed_out ? __uint_as_float(0x7fc00000u) : 1.f / sm;
      if (lane == 0) {
        a.conf[wave] = c;
        s.cf[wave] = c;
      }
    }
  }
  if (a.nkeep) {
    // confidence gate: candidates are kept up to the first one below min_p
    lds_sync();
    if (otid() == 0) {
      int n = 0;
      while (n + 1 < a.B && s.cf[n] >= a.min_p) ++n;
      *a.nkeep = timed_out ? 0 : n;
    }
  }
}

template <int FMT, int LMF>
__global__ __launch_bounds__(NTHR) void k_draft_pass(PassArgs args) {
  __shared__ Smem s;
  PassArgs a = args;
  if (a.dstate) {  // positions from device memory (uniform: every block reads the same words)
    const PosState ps = resolve_positions(a.dstate, a.window, a.maxch, a.vocab, a.taps_pos0,
                                          a.taps_rows);
    if (!ps.ok) {  // nothing is read from an invalid state; report it
      if (blockIdx.x == 0 && otid() == 0) {
        __hip_atomic_store(a.bar + BAR_STATUS, ST_INVALID, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        for (int b = 0; b + 1 < a.B; ++b) a.cand[b] = -1;
        if (a.conf)
          for (int b = 0; b + 1 < a.B; ++b) a.conf[b] = __uint_as_float(0x7fc00000u);
        if (a.nkeep) *a.nkeep = 0;
      }
      return;
    }
    a.lo = ps.lo;
    a.hi = ps.hi;
    a.p0 = ps.p0;
    a.nb = ps.nb;
    a.cb = ps.cb;
    a.nch = ps.nch;
    a.nc = ps.nc;
    a.pos0 = ps.pos0;
    a.taps = ps.nc ? a.taps_base + static_cast<size_t>(ps.pos0 - a.taps_pos0) * T * H : nullptr;
  }
  BarState bk;      // barriers passed, give-up flag
  QkvTile<FMT> Wq;
  LmTile<LMF> Wl;   // LM head slice, prefetched after the last layer
  // Commit rows (fused draft-commit cycle) through fc first; then each block
  // goes straight on to layer 0's QKV phase (h, ss, the RoPE table and the
  // layer table come from the init kernel, visible from the start): only the
  // blocks that project the commit rows wait, there, until every fc output
  // tile is written (fc_wait) -- no grid barrier.
  fc_phase<FMT>(a, s);
  qkv_prefetch<FMT>(a, 0, Wq, !act_wave());
  int np = 1;    // sums of squares of h: one entry per row from the init kernel
  for (int l = 0; l < L; ++l) {
    qkv_phase<FMT>(a, s, l, np, Wq);
    grid_sync_pf(a, bk, [&] { attn_stage(a, s, l); });
    attn_phase(a, s, l);
    grid_sync(a, bk);
    merge_phase<FMT>(a, s, l);
    OTile<FMT> Wo;
    grid_sync_pf<true>(a, bk, [&] { o_prefetch<FMT>(a, l, Wo, !act_wave()); });
    o_phase<FMT>(a, s, l, Wo);
    GuTile<FMT> Wg;
    grid_sync_pf(a, bk, [&] { gu_prefetch<FMT>(a, l, blockIdx.x, Wg, true); });
    gu_phase<FMT>(a, s, l, NT_H, Wg);
    DownTile<FMT> Wd;
    grid_sync_pf<(ACT_WAVE > DOWN_PRE_LAST)>(a, bk,
                                           [&] { down_prefetch<FMT>(a, l, Wd, down_pre(wid())); });
    down_phase<FMT>(a, s, l, Wd);
    // Both prefetch targets are assigned on every iteration (zeros when
    // idle), so neither carries a value around the loop.
    const bool last = l + 1 == L;
    grid_sync_pf<true>(a, bk, [&] {
      qkv_prefetch<FMT>(a, last ? l : l + 1, Wq, !last && !act_wave());
      lm_prefetch<LMF>(a, blockIdx.x, Wl, last && a.B > 1 && !act_wave());
    });
    np = NT_H;
  }
  if (a.B > 1) {
    lm_phase<LMF>(a, s, np, Wl);
    grid_sync(a, bk);
    argmax_final(a, s);
  } else if (blockIdx.x == 0 && a.hidden) {
    build_x_norm<W_BF16>(a, s, 2 * L, np, a.final_norm);
    for (int e = otid(); e < H; e += NTHR) a.hidden[e] = s.x[e];
  }
}

// h[b] = E[token_b], per-row sum of squares, RoPE table of p .. p+B-1 (rows
// 0..B-1) and of the commit positions pos0 .. pos0+nc-1 (rows 8..8+nc-1), and
// the barrier words of the pass kernel.  grid max(B, nc), block 256.
// Positions read by the init kernel when they live in device memory (the
// same state and bounds the pass reads).
struct InitPos {
  const int64_t* dstate;
  int64_t window, taps_pos0, taps_rows;
  int maxch, vocab;
};

__global__ __launch_bounds__(256) void k_pass_init(LayerTab tab, LayerTab* tab_out,
                                                   const uint16_t* embed, int anchor, int mask,
                                                   int B, int64_t p, int nc, int64_t pos0,
                                                   double theta, float* h, uint16_t* h16,
                                                   float* ss, float2* rope, unsigned* bar,
                                                   InitPos dp) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  if (b == 0)
    for (int i = threadIdx.x; i < BAR_WORDS; i += 256) bar[i] = 0u;
  if (b == 0 && threadIdx.x == 0) *tab_out = tab;
  if (dp.dstate) {
    const PosState ps = resolve_positions(dp.dstate, dp.window, dp.maxch, dp.vocab, dp.taps_pos0,
                                          dp.taps_rows);
    if (!ps.ok) return;  // the pass reports it
    anchor = ps.anchor;
    p = ps.p;
    nc = ps.nc;
    pos0 = ps.pos0;
  }
  if (b < nc && threadIdx.x < D / 2) {
    const double inv = pow(theta, -2.0 * static_cast<double>(threadIdx.x) / static_cast<double>(D));
    double sn, cs;
    sincos(static_cast<double>(pos0 + b) * inv, &sn, &cs);
    rope[(MAXB + b) * (D / 2) + threadIdx.x] = make_float2(static_cast<float>(cs), static_cast<float>(sn));
  }
  if (b >= B) return;  // block-uniform
  const int tok = b == 0 ? anchor : mask;
  const uint16_t* row = embed + static_cast<size_t>(tok) * H;
  // All of the row's loads are issued before any store (a store could alias
  // the row, so a load after it would wait for it: one memory round trip per
  // element group), and the RoPE table is computed while they are in flight.
  constexpr int PER = H / 256;
  static_assert(H % 256 == 0, "embedding row split over 256 threads");
  uint16_t raw[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) raw[i] = row[threadIdx.x + 256 * i];
  if (threadIdx.x < D / 2) {
    const double inv = pow(theta, -2.0 * static_cast<double>(threadIdx.x) / static_cast<double>(D));
    double sn, cs;
    sincos(static_cast<double>(p + b) * inv, &sn, &cs);
    rope[b * (D / 2) + threadIdx.x] = make_float2(static_cast<float>(cs), static_cast<float>(sn));
  }
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = threadIdx.x + 256 * i;
    const float v = bf16_to_f32(raw[i]);
    h[static_cast<size_t>(b) * H + e] = v;
    h16[static_cast<size_t>(b) * H + e] = f32_to_f16_bits(v);
    sq += v * v;
  }
  sq = block_sum<256>(sq, red);
  if (threadIdx.x == 0) ss[b] = sq;
}

__global__ void k_pass_status(const unsigned* bar, int32_t* status, int32_t timeout_code,
                              int32_t invalid_code) {
  if (threadIdx.x == 0) {
    const uint32_t v = ld_coh32(bar + BAR_STATUS);
    *status = v == 0u ? 0 : (v == ST_INVALID ? invalid_code : timeout_code);
  }
}

}  // namespace

size_t pass_smem_bytes() { return sizeof(Smem); }
size_t pass_tab_bytes() { return sizeof(LayerTab); }
size_t pass_bar_bytes() { return sizeof(unsigned) * BAR_WORDS; }
size_t pass_fcp_bytes() { return sizeof(float) * NT_H * FC_CONTRIB * 64 * 4; }
size_t pass_po_bytes() { return sizeof(uint16_t) * L * POSTRIDE; }
size_t pass_pml_bytes() { return sizeof(float) * L * PMSTRIDE; }

namespace {
// The pass kernel for a backbone format and an LM-head format.
const void* pass_kernel(int fmt, int lm_fmt) {
  if (lm_fmt == W_BF16) {
    if (fmt == W_BF16) return reinterpret_cast<const void*>(k_draft_pass<W_BF16, W_BF16>);
    if (fmt == W_Q8_0) return reinterpret_cast<const void*>(k_draft_pass<W_Q8_0, W_BF16>);
    if (fmt == W_Q4_0) return reinterpret_cast<const void*>(k_draft_pass<W_Q4_0, W_BF16>);
    if (fmt == W_Q5_0) return reinterpret_cast<const void*>(k_draft_pass<W_Q5_0, W_BF16>);
  } else if (lm_fmt == W_Q8_0) {
    if (fmt == W_BF16) return reinterpret_cast<const void*>(k_draft_pass<W_BF16, W_Q8_0>);
    if (fmt == W_Q8_0) return reinterpret_cast<const void*>(k_draft_pass<W_Q8_0, W_Q8_0>);
    if (fmt == W_Q4_0) return reinterpret_cast<const void*>(k_draft_pass<W_Q4_0, W_Q8_0>);
    if (fmt == W_Q5_0) return reinterpret_cast<const void*>(k_draft_pass<W_Q5_0, W_Q8_0>);
  }
  return nullptr;
}
}  // namespace

hipError_t launch_draft_pass(const PassLaunch& q, hipStream_t st) {
  LayerTab tab;
  for (int l = 0; l < L; ++l) {
    tab.wq[l] = q.wq[l];
    tab.wk[l] = q.wk[l];
    tab.wv[l] = q.wv[l];
    tab.wo[l] = q.wo[l];
    tab.wg[l] = q.wg[l];
    tab.wu[l] = q.wu[l];
    tab.wd[l] = q.wd[l];
    tab.in_norm[l] = q.in_norm[l];
    tab.q_norm[l] = q.q_norm[l];
    tab.k_norm[l] = q.k_norm[l];
    tab.post_norm[l] = q.post_norm[l];
  }
  PassArgs a;
  a.tab = reinterpret_cast<const LayerTab*>(q.tab);
  a.final_norm = q.final_norm;
  a.lm = q.lm;
  a.vocab = q.vocab;
  a.eps = q.eps;
  a.scale_log2 = q.scale_log2;
  a.ring_k = q.ring_k;
  a.ring_vt = q.ring_vt;
  a.cap = q.cap;
  a.lo = q.lo;
  a.hi = q.hi;
  a.p0 = q.p0;
  a.nb = q.nb;
  a.cb = q.cb;
  a.nch = q.nch;
  a.B = q.B;
  a.nqt = (G * q.B + 15) / 16;
  a.h = q.h;
  a.h16 = q.h16;
  a.ss = q.ss;
  a.qkv = q.qkv;
  a.rope = q.rope;
  a.po = q.po;
  a.pm = q.pm;
  a.pl = q.pl;
  a.o16 = q.o16;
  a.u16 = q.u16;
  a.keys = q.keys;
  a.lse = q.lse;
  a.conf = q.conf;
  a.nkeep = q.nkeep;
  a.min_p = q.min_p;
  a.bar = q.bar;
  a.wait_ticks = q.wait_ticks;
  a.taps = q.taps;
  a.fc = q.fc;
  a.hidden_norm = q.hidden_norm;
  a.nc = q.nc;
  a.pos0 = q.pos0;
  a.yc = q.yc;
  a.fcp = q.fcp;
  a.cn = q.cn;
  a.ckv = q.ckv;
  a.cand = q.cand;
  a.logits = q.logits;
  a.hidden = q.hidden;
  a.dstate = q.dstate;
  a.taps_base = q.taps_base;
  a.taps_pos0 = q.taps_pos0;
  a.taps_rows = q.taps_rows;
  a.window = q.window;
  a.maxch = q.maxch;
  // every phase assumes at least one block per work item of its first round
  if (q.fmt < W_BF16 || q.fmt > W_Q5_0 || (q.lm_fmt != W_BF16 && q.lm_fmt != W_Q8_0))
    return hipErrorInvalidValue;
  if (q.nch < 1 || q.nch > 128 || q.grid < NKV * q.nch || q.grid < QKV_N / 32 ||
      q.grid < NKV * a.nqt * 16 || q.grid > 1024)
    return hipErrorInvalidValue;
  if (q.nc < 0 || q.nc > MAXB ||
      (q.nc > 0 && (!q.taps || !q.fc || !q.yc || !q.fcp || !q.cn || !q.ckv || q.grid < NT_H ||
                    q.grid > FC_GRID_MAX)))
    return hipErrorInvalidValue;
  // device-resident positions: up to MAXB commit rows, at most maxch chunks per head
  if (q.dstate && (!q.taps_base || !q.fc || !q.yc || !q.fcp || !q.cn || !q.ckv || q.grid < NT_H ||
                   q.grid > FC_GRID_MAX || q.maxch < 1 ||
                   q.maxch > 128 || q.grid < NKV * q.maxch || q.window < 1 || q.taps_pos0 < 0 ||
                   q.taps_rows < 0))
    return hipErrorInvalidValue;
  InitPos dp{q.dstate, q.window, q.taps_pos0, q.taps_rows, q.maxch, q.vocab};
  const int init_grid = q.dstate ? MAXB : (q.B > q.nc ? q.B : q.nc);
  hipLaunchKernelGGL(k_pass_init, dim3(init_grid), dim3(256), 0, st, tab,
                     reinterpret_cast<LayerTab*>(q.tab), q.embed, q.anchor, q.mask, q.B, q.p, q.nc,
                     q.pos0, q.theta, q.h, q.h16, q.ss, q.rope, q.bar, dp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const void* kern = pass_kernel(q.fmt, q.lm_fmt);
  if (!kern) return hipErrorInvalidValue;
  void* args[] = {&a};
  // A plain launch: the grid is at most one block per CU, the most the device
  // holds at once (draft_pass_max_grid), so every block is resident as soon
  // as the device is not busy with other work.  (A cooperative launch adds
  // about 20 us per pass on MI355X, measured.)  If other work keeps blocks
  // from becoming resident for longer than the barriers' bounded wait, the
  // pass reports it through cand = -1 instead of hanging.
  return hipLaunchKernel(kern, dim3(q.grid), dim3(NTHR), args, 0, st);
}

hipError_t launch_pass_status(const unsigned* bar, int32_t* status, int32_t timeout_code,
                              int32_t invalid_code, hipStream_t st) {
  hipLaunchKernelGGL(k_pass_status, dim3(1), dim3(64), 0, st, bar, status, timeout_code,
                     invalid_code);
  return hipGetLastError();
}

hipError_t wall_clock_ticks_per_us(int device, double* ticks) {
  int khz = 0;
  const hipError_t e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device);
  if (e != hipSuccess) return e;
  if (khz <= 0) return hipErrorInvalidValue;
  *ticks = static_cast<double>(khz) / 1000.0;
  return hipSuccess;
}

hipError_t draft_pass_max_grid(int device, int* grid) {
  int cus = 0, per = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return e;
  // one block per CU for every weight format's instantiation
  int ok = 1;
  for (int f = W_BF16; f <= W_Q5_0; ++f) {
    for (int lf : {static_cast<int>(W_BF16), static_cast<int>(W_Q8_0)}) {
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, pass_kernel(f, lf), NTHR, 0);
      if (e != hipSuccess) return e;
      ok = ok && per > 0;
    }
  }
  *grid = ok ? cus : 0;
  return hipSuccess;
}

}  // namespace dfl
