// C ABI entry points: argument validation, workspace carving and the launch
// sequence of each operation.  Everything is enqueued on the caller's stream;
// positions and sizes travel as kernel arguments (no host staging buffers).
#include "../../include/dflash.h"
#include "common.h"
#include "fuse.h"

#include <stdlib.h>
#include <string.h>

#include <mutex>

using namespace dfl;

namespace {

constexpr int LMH_GRID = 256;         // standalone LM-head kernel: one block per CU
constexpr int KEYS_MAX = 1024;        // argmax key slots (blocks of either LM-head launch)
constexpr long BARRIER_WAIT_US = 500000;   // grid-barrier wait bound (0.5 s of wall clock)
constexpr long BARRIER_WAIT_US_MAX = 10000000;

// The barrier wait bound in microseconds: BARRIER_WAIT_US, or
// DFLASH_BARRIER_TIMEOUT_US from the environment (read on every call, 0 ..
// 10^7) so that tests can drive the give-up path.
long barrier_wait_us() {
  const char* e = getenv("DFLASH_BARRIER_TIMEOUT_US");
  if (!e || !*e) return BARRIER_WAIT_US;
  char* end = nullptr;
  const long v = strtol(e, &end, 10);
  return end && *end == 0 && v >= 0 && v <= BARRIER_WAIT_US_MAX ? v : BARRIER_WAIT_US;
}

// Constant-clock ticks per microsecond per device (a hardware property).
double ticks_per_us() {
  static double cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0.0;
  if (cache[dev] == 0.0) {
    double t = 0.0;
    if (wall_clock_ticks_per_us(dev, &t) != hipSuccess) return 0.0;
    cache[dev] = t;
  }
  return cache[dev];
}

// Co-resident grid of the pass kernel per device (a hardware property).
int pass_grid() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int g = 0;
    if (draft_pass_max_grid(dev, &g) != hipSuccess) return 0;
    cache[dev] = g > KEYS_MAX ? KEYS_MAX : g;
  }
  return cache[dev];
}
constexpr int SMALL_ROWS = 64;        // fuse/project: skinny path up to here
// Projections of more rows write their cells from the GEMM's epilogue (the
// same bits as the GEMM's fp32 output through k_kv_post): 0.974 -> 0.863 ms
// at 32768 rows, 0.098 -> 0.089 ms at 2432; with fewer 256-row tiles than
// the CUs hold, one tile's epilogue is the critical path and the separate
// kernel is faster (0.078 vs 0.082 ms at 1536 rows).
constexpr int KV_FUSED_MIN_ROWS = 2048;
constexpr int FC_SPLITS = 10;         // k splits of the fc GEMV (K = 12800)
constexpr int KV_SPLITS = 2;          // k splits of the Wk / Wv GEMV (K = 2560)
constexpr size_t PART_FLOATS = static_cast<size_t>(FC_SPLITS) * GEMV_ROWS * H;
static_assert(static_cast<size_t>(KV_SPLITS) * GEMV_ROWS * KV_N <= PART_FLOATS,
              "the Wk / Wv partials share the fc partials' workspace");

struct Layout {
  size_t part, po, pm, pl, keys, lse, rope, ss, qkv, hv, h16, ov, uv, bar, tab, yc, fcp, cn, ckv, y;
  size_t fixed;  // bytes before y
};

size_t take(size_t& off, size_t bytes) {
  const size_t o = off;
  off = (off + bytes + 255) & ~static_cast<size_t>(255);
  return o;
}

Layout layout() {
  Layout L;
  size_t off = 0;
  L.part = take(off, sizeof(float) * PART_FLOATS);
  L.po = take(off, pass_po_bytes());
  L.pm = take(off, pass_pml_bytes());
  L.pl = take(off, pass_pml_bytes());
  L.keys = take(off, sizeof(uint64_t) * KEYS_MAX * MAXB);
  L.lse = take(off, sizeof(uint64_t) * KEYS_MAX * MAXB);
  L.rope = take(off, sizeof(float) * 2 * (2 * MAXB) * (D / 2));  // block rows, commit rows
  // per-layer / per-version copies used by the persistent pass
  constexpr size_t HV = 2 * dfl::L + 1, NL = dfl::L;
  L.ss = take(off, sizeof(float) * HV * (H / 16) * MAXB);
  L.qkv = take(off, sizeof(uint16_t) * NL * MAXB * QKV_N);
  L.hv = take(off, sizeof(float) * HV * MAXB * H);
  L.h16 = take(off, sizeof(uint16_t) * HV * MAXB * H);
  L.ov = take(off, 2 * NL * MAXB * NQ * D);
  L.uv = take(off, 2 * NL * MAXB * F);
  L.bar = take(off, pass_bar_bytes());
  L.tab = take(off, pass_tab_bytes());
  // commit rows of the fused draft-commit cycle: fc outputs, fused rows, raw K | V
  L.yc = take(off, sizeof(float) * MAXB * H);
  L.fcp = take(off, pass_fcp_bytes());
  L.cn = take(off, sizeof(uint16_t) * MAXB * H);
  L.ckv = take(off, sizeof(float) * dfl::L * MAXB * 2 * NKV * D);
  L.fixed = off;
  L.y = off;
  return L;
}

// Row-dependent tail of the workspace: fp32 GEMM output [rows][5120] and,
// for quantized weights, the bf16 copy of the widest matrix the GEMM path
// decodes (fc, 2560 x 12800).
constexpr size_t DQ_ELEMS = static_cast<size_t>(H) * T * H;

size_t y_bytes(int rows) { return sizeof(float) * static_cast<size_t>(rows) * KV_N; }

size_t rows_bytes(int rows, int fmt) {
  if (rows <= SMALL_ROWS) return 0;
  const size_t y = (y_bytes(rows) + 255) & ~static_cast<size_t>(255);
  return y + (fmt != W_BF16 ? 2 * DQ_ELEMS : 0);
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Device buffers are read and written with 16-byte vector accesses.
bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Row-major matrices (fc, the 35 layer matrices, the LM head) may be null
// once w->packed holds their streaming copies: every call then reads those.
// Packing itself (need_rowmajor) reads the row-major tensors.
int check_weights(const dflash_weights* w, bool need_rowmajor = false) {
  if (!w) return DFLASH_EINVAL;
  if (w->hidden != H || w->n_layers != L || w->n_q_heads != NQ || w->n_kv_heads != NKV ||
      w->head_dim != D || w->ffn != F || w->n_taps != T)
    return DFLASH_EGEOMETRY;
  if (w->vocab < 16 || w->vocab % 16 != 0 || w->vocab > (1 << 24)) return DFLASH_EGEOMETRY;
  if (w->rope_theta != 1.0e7f || w->attn_scale != 0.0625f || w->rms_eps != 1.0e-6f)
    return DFLASH_EGEOMETRY;
  if (w->backbone_type != DFLASH_W_BF16 && w->backbone_type != DFLASH_W_Q8_0 &&
      w->backbone_type != DFLASH_W_Q4_0 && w->backbone_type != DFLASH_W_Q5_0)
    return DFLASH_EINVAL;
  if (w->lm_head_type != DFLASH_W_BF16 && w->lm_head_type != DFLASH_W_Q8_0) return DFLASH_EINVAL;
  const bool rm = need_rowmajor || !w->packed;  // row-major matrices required
  if (!w->hidden_norm || !w->final_norm || !w->embed || (rm && (!w->fc || !w->lm_head)))
    return DFLASH_EINVAL;
  if (!a16(w->fc) || !a16(w->hidden_norm) || !a16(w->final_norm) || !a16(w->embed) ||
      !a16(w->lm_head) || !a16(w->packed))
    return DFLASH_EINVAL;
  for (int l = 0; l < L; ++l) {
    const dflash_layer_weights& y = w->layer[l];
    const void* gains[4] = {y.in_norm, y.q_norm, y.k_norm, y.post_norm};
    const void* mats[7] = {y.wq, y.wk, y.wv, y.wo, y.wg, y.wu, y.wd};
    for (const void* p : gains)
      if (!p || !a16(p)) return DFLASH_EINVAL;
    for (const void* p : mats)
      if ((rm && !p) || !a16(p)) return DFLASH_EINVAL;
  }
  return DFLASH_OK;
}

int check_kv(const dflash_kv* kv) {
  if (!kv || !kv->k || !kv->vt || !a16(kv->k) || !a16(kv->vt)) return DFLASH_EINVAL;
  if (kv->capacity <= 0 || kv->capacity % 256 != 0) return DFLASH_ERANGE;
  if (kv->window <= 0 || kv->window > kv->capacity) return DFLASH_ERANGE;
  return DFLASH_OK;
}

// The streaming copies inside w->packed: the LM head (bf16), then every
// layer's wq, wk, wv, wo, wg, wu, wd in the backbone's format: bf16, or the
// quants followed by their block scales (and Q5_0's high-bit words), all
// regrouped per 16-row tile and 64-byte row piece.
struct PackedMat {
  int N, K;
};
constexpr PackedMat LAYER_MATS[7] = {{NQ * D, H}, {NKV * D, H}, {NKV * D, H}, {H, NQ * D},
                                     {F, H},      {F, H},       {H, F}};

// Bytes of one [N][K] matrix in format fmt (quants, then scales, then
// Q5_0's high-bit words).
size_t mat_bytes(int fmt, size_t N, size_t K) {
  if (fmt == DFLASH_W_Q8_0) return N * K + N * (K / 32) * 2;
  if (fmt == DFLASH_W_Q4_0) return N * K / 2 + N * (K / 32) * 2;
  if (fmt == DFLASH_W_Q5_0) return N * K / 2 + N * (K / 32) * 6;
  return 2 * N * K;
}

size_t layer_bytes(int fmt) {
  size_t b = 0;
  for (const PackedMat& m : LAYER_MATS) b += mat_bytes(fmt, m.N, m.K);
  return b;
}

// The LM head's streaming copy comes first, in its own format.
size_t lm_bytes(const dflash_weights* w) {
  return mat_bytes(w->lm_head_type, static_cast<size_t>(w->vocab), H);
}

size_t packed_bytes(const dflash_weights* w) {
  return lm_bytes(w) + L * layer_bytes(w->backbone_type) +
         mat_bytes(w->backbone_type, H, static_cast<size_t>(T) * H);
}

// Packed copy of fc [2560][12800], after the layers.
uint8_t* packed_fc(const dflash_weights* w) {
  return static_cast<uint8_t*>(w->packed) + lm_bytes(w) + L * layer_bytes(w->backbone_type);
}

// Packed copies of layer l's seven matrices, in LAYER_MATS order.
void packed_layer(const dflash_weights* w, int l, uint8_t* (&out)[7]) {
  uint8_t* p = static_cast<uint8_t*>(w->packed) + lm_bytes(w) + l * layer_bytes(w->backbone_type);
  for (int i = 0; i < 7; ++i) {
    out[i] = p;
    p += mat_bytes(w->backbone_type, LAYER_MATS[i].N, LAYER_MATS[i].K);
  }
}

// One matrix into its streaming copy: the 64-byte row pieces of the quants
// (or bf16 values) move as the bf16 shuffle moves 32-element blocks; the
// scales of a quantized matrix follow as 4-byte (Q8_0: one 64-k piece) or
// 8-byte (Q4_0 / Q5_0: one 128-k piece) units per row, and Q5_0's high-bit
// words as 16-byte units with their bits reordered for the decoder.
hipError_t pack_matrix(int fmt, const void* src, int N, int K, void* dst, hipStream_t st) {
  if (fmt == DFLASH_W_BF16) return launch_pack_bf16(src, N, K, dst, st);
  const size_t qbytes = fmt == DFLASH_W_Q8_0 ? static_cast<size_t>(N) * K : static_cast<size_t>(N) * K / 2;
  const int kq = fmt == DFLASH_W_Q8_0 ? K / 2 : K / 4;  // row bytes / 2 (bf16 units)
  hipError_t e = launch_pack_bf16(src, N, kq, dst, st);
  if (e != hipSuccess) return e;
  const int per_row = fmt == DFLASH_W_Q8_0 ? K / 64 : K / 128;
  const uint8_t* s8 = static_cast<const uint8_t*>(src);
  uint8_t* d8 = static_cast<uint8_t*>(dst);
  e = launch_pack_units(s8 + qbytes, N, per_row, fmt == DFLASH_W_Q8_0 ? 4 : 8, d8 + qbytes, st);
  if (e != hipSuccess || fmt != DFLASH_W_Q5_0) return e;
  const size_t sbytes = static_cast<size_t>(N) * (K / 32) * 2;
  return launch_pack_q5_bits(s8 + qbytes + sbytes, N, per_row, d8 + qbytes + sbytes, st);
}

SegTable seg1(const void* p, int rows) {
  SegTable t;
  memset(&t, 0, sizeof(t));
  t.ptr[0] = p;
  t.row_end[0] = rows;
  t.nseg = 1;
  return t;
}

SegTable seg_qkv(const dflash_layer_weights& y) {
  SegTable t;
  memset(&t, 0, sizeof(t));
  t.ptr[0] = y.wq;
  t.row_end[0] = NQ * D;
  t.ptr[1] = y.wk;
  t.row_end[1] = NQ * D + NKV * D;
  t.ptr[2] = y.wv;
  t.row_end[2] = QKV_N;
  t.nseg = 3;
  return t;
}

SegTable seg_kv(const dflash_weights* w) {
  SegTable t;
  memset(&t, 0, sizeof(t));
  for (int l = 0; l < L; ++l) {
    t.ptr[2 * l] = w->layer[l].wk;
    t.row_end[2 * l] = (2 * l + 1) * NKV * D;
    t.ptr[2 * l + 1] = w->layer[l].wv;
    t.row_end[2 * l + 1] = (2 * l + 2) * NKV * D;
  }
  t.nseg = 2 * L;
  return t;
}

#define HIP_TRY(expr)                                   \
  do {                                                  \
    if ((expr) != hipSuccess) return DFLASH_EHIP;       \
  } while (0)

const uint16_t* u16p(const void* p) { return static_cast<const uint16_t*>(p); }

// Workspace of dflash_draft_block_static, for callers that cannot allocate:
// a file-scope device array (each device the library runs on holds its own
// copy until the process ends).  The pass needs layout().fixed bytes of it
// whatever the context length or block size.  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address is looked
// up once per device (scratch_on_device) and only that address is used.
constexpr size_t SCRATCH_BYTES = static_cast<size_t>(67) << 20;
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

// Device address of `scratch` on the current device (null on failure),
// looked up on the first call on that device.
void* scratch_on_device() {
  static std::mutex mu;
  static void* ptr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[dev] = a;
  }
  return ptr[dev];
}

}  // namespace

extern "C" size_t dflash_workspace_size(const dflash_weights* w, int32_t max_rows,
                                        int32_t max_block) {
  (void)w;
  if (max_rows < 0 || max_block < 0 || max_block > MAXB) return 0;
  const int fmt = w ? w->backbone_type : W_BF16;
  return layout().fixed + rows_bytes(max_rows, fmt);
}

extern "C" size_t dflash_packed_size(const dflash_weights* w) {
  if (check_weights(w) != DFLASH_OK) return 0;
  return packed_bytes(w);
}

extern "C" int32_t dflash_pack_weights(const dflash_weights* w, void* stream) {
  int rc = check_weights(w, true);
  if (rc) return rc;
  if (!w->packed) return DFLASH_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIP_TRY(pack_matrix(w->lm_head_type, w->lm_head, w->vocab, H, w->packed, st));
  for (int l = 0; l < L; ++l) {
    const dflash_layer_weights& y = w->layer[l];
    const void* src[7] = {y.wq, y.wk, y.wv, y.wo, y.wg, y.wu, y.wd};
    uint8_t* dst[7];
    packed_layer(w, l, dst);
    for (int i = 0; i < 7; ++i)
      HIP_TRY(pack_matrix(w->backbone_type, src[i], LAYER_MATS[i].N, LAYER_MATS[i].K, dst[i], st));
  }
  HIP_TRY(pack_matrix(w->backbone_type, w->fc, H, T * H, packed_fc(w), st));
  return DFLASH_OK;
}

extern "C" int32_t dflash_fuse_context(const dflash_weights* w, const void* taps, int32_t n,
                                       void* ctx, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_weights(w);
  if (rc) return rc;
  if (n < 0) return DFLASH_EINVAL;
  if (n == 0) return DFLASH_OK;
  if (!taps || !ctx || !ws || !a16(taps) || !a16(ctx) || !a16(ws)) return DFLASH_EINVAL;
  const Layout Lw = layout();
  const int fmt = w->backbone_type;
  if (ws_bytes < Lw.fixed + rows_bytes(n, fmt)) return DFLASH_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* x = u16p(taps);
  uint16_t* out = static_cast<uint16_t*>(ctx);
  if (n <= SMALL_ROWS) {
    float* part = at<float>(ws, Lw.part);
    for (int c0 = 0; c0 < n; c0 += GEMV_ROWS) {
      const int rows = n - c0 < GEMV_ROWS ? n - c0 : GEMV_ROWS;
      GemvArgs a;
      a.w = seg1(w->packed ? packed_fc(w) : w->fc, H);
      a.packed = w->packed != nullptr;
      a.fmt = fmt;
      a.N = H;
      a.K = T * H;
      a.x = x + static_cast<size_t>(c0) * T * H;
      a.x_stride = T * H;
      a.B = rows;
      a.out = part;
      a.S = FC_SPLITS;
      HIP_TRY(launch_gemv(a, st));
      HIP_TRY(launch_rownorm(nullptr, part, FC_SPLITS, static_cast<size_t>(rows) * H, H, rows,
                             u16p(w->hidden_norm), w->rms_eps, out + static_cast<size_t>(c0) * H,
                             H, nullptr, st));
    }
  } else {
    float* y = at<float>(ws, Lw.y);
    // W in the streaming layout (contiguous 1 KiB loads): bf16 -> fc's
    // streaming copy when there is one; quantized -> decoded once into it
    bool wp = fmt == W_BF16 && w->packed;
    SegTable wt = seg1(wp ? packed_fc(w) : w->fc, H);
    if (fmt != W_BF16) {
      uint16_t* dq = at<uint16_t>(ws, Lw.y + rows_bytes(n, fmt) - 2 * DQ_ELEMS);
      const bool pk = w->packed != nullptr;
      HIP_TRY(launch_dequant_bf16(pk ? packed_fc(w) : w->fc, fmt, H, T * H, dq, 0, pk, st));
      wt = seg1(dq, H);
      wp = true;
    }
    // Each of the 256 compute units runs one 256 x 256 output tile at a time.
    // The k range is split in two when there are fewer tiles than compute
    // units (n <= 6400 rows), or when the halves finish in fewer tile times
    // than whole tiles whose last wave leaves most units idle (8192 rows: 320
    // tiles take two tile times, 640 halves three half tile times).  The fp32
    // region then holds two partial outputs, which the row norm sums.
    constexpr int CUS = 256;
    const int tiles = (n + 255) / 256 * (H / 256);
    const int waves1 = (tiles + CUS - 1) / CUS, waves2 = (2 * tiles + CUS - 1) / CUS;
    if (tiles < CUS || waves2 < 2 * waves1) {
      const size_t cs = static_cast<size_t>(n) * H;
      HIP_TRY(launch_gemm_bf16(x, T * H, n, wt, wp, T * H, y, H, H, 2, cs, st));
      HIP_TRY(launch_rownorm(nullptr, y, 2, cs, H, n, u16p(w->hidden_norm), w->rms_eps, out, H,
                             nullptr, st));
    } else {
      // The GEMM writes the rows in bf16 with their fp32 tile sums of squares
      // (half the bytes of fp32 rows, written as whole rows), inside the fp32
      // region: y16 [n][H], then ss [n][H / 256].
      uint16_t* y16 = reinterpret_cast<uint16_t*>(y);
      float* ss = reinterpret_cast<float*>(y16 + static_cast<size_t>(n) * H);
      HIP_TRY(launch_gemm_fuse_bf16(x, T * H, n, wt, wp, T * H, FuseEpi{y16, ss}, st));
      HIP_TRY(launch_rownorm_tiles(y16, ss, n, u16p(w->hidden_norm), w->rms_eps, out, H, st));
    }
  }
  return DFLASH_OK;
}

extern "C" int32_t dflash_project_ctx_kv(const dflash_weights* w, const void* ctx, int32_t n,
                                         int64_t pos0, const dflash_kv* kv, void* ws,
                                         size_t ws_bytes, void* stream) {
  int rc = check_weights(w);
  if (rc) return rc;
  rc = check_kv(kv);
  if (rc) return rc;
  if (n < 0 || pos0 < 0) return DFLASH_EINVAL;
  if (n > kv->capacity) return DFLASH_ERANGE;
  if (n == 0) return DFLASH_OK;
  if (!ctx || !ws || !a16(ctx) || !a16(ws)) return DFLASH_EINVAL;
  const Layout Lw = layout();
  const int fmt = w->backbone_type;
  if (ws_bytes < Lw.fixed + rows_bytes(n, fmt)) return DFLASH_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const void* knorms[L];
  for (int l = 0; l < L; ++l) knorms[l] = w->layer[l].k_norm;
  const uint16_t* x = u16p(ctx);
  uint16_t* rk = static_cast<uint16_t*>(kv->k);
  uint16_t* rv = static_cast<uint16_t*>(kv->vt);
  const double theta = static_cast<double>(w->rope_theta);
  if (n <= SMALL_ROWS) {
    float* part = at<float>(ws, Lw.part);
    for (int c0 = 0; c0 < n; c0 += GEMV_ROWS) {
      const int rows = n - c0 < GEMV_ROWS ? n - c0 : GEMV_ROWS;
      GemvArgs a;
      a.w = seg_kv(w);
      a.packed = w->packed != nullptr;
      if (a.packed) {  // the layers' packed Wk / Wv
        for (int l = 0; l < L; ++l) {
          uint8_t* pm[7];
          packed_layer(w, l, pm);
          a.w.ptr[2 * l] = pm[1];
          a.w.ptr[2 * l + 1] = pm[2];
        }
      }
      a.fmt = fmt;
      a.N = KV_N;
      a.K = H;
      a.x = x + static_cast<size_t>(c0) * H;
      a.x_stride = H;
      a.B = rows;
      a.out = part;
      a.S = KV_SPLITS;
      HIP_TRY(launch_gemv(a, st));
      HIP_TRY(launch_kv_post(part, KV_N, KV_SPLITS, static_cast<size_t>(rows) * KV_N, rows, pos0 + c0,
                             knorms, w->rms_eps, theta, rk, rv, kv->capacity, st));
    }
  } else {
    SegTable wt = seg_kv(w);
    bool wp = w->packed != nullptr;
    if (wp) {  // the layers' packed Wk / Wv (bf16, or quantized blocks decoded below)
      for (int l = 0; l < L; ++l) {
        uint8_t* pm[7];
        packed_layer(w, l, pm);
        wt.ptr[2 * l] = pm[1];
        wt.ptr[2 * l + 1] = pm[2];
      }
    }
    if (fmt != W_BF16) {  // decode the ten K/V matrices into one bf16 [5120][2560], streaming layout
      uint16_t* dq = at<uint16_t>(ws, Lw.y + rows_bytes(n, fmt) - 2 * DQ_ELEMS);
      for (int s = 0; s < wt.nseg; ++s) {
        const int r0 = s ? wt.row_end[s - 1] : 0;
        HIP_TRY(launch_dequant_bf16(wt.ptr[s], fmt, wt.row_end[s] - r0, H, dq, r0, wp, st));
      }
      wt = seg1(dq, KV_N);
      wp = true;
    }
    if (n > KV_FUSED_MIN_ROWS) {
      // the cells come straight out of the GEMM's epilogue; the fp32 output
      // region holds the rows' RoPE table instead
      float2* rope = at<float2>(ws, Lw.y);
      HIP_TRY(launch_rope_rows(rope, pos0, n, theta, st));
      KvEpi ke;
      ke.ring_k = rk;
      ke.ring_vt = rv;
      ke.cap = kv->capacity;
      ke.pos0 = pos0;
      ke.rope = rope;
      for (int l = 0; l < L; ++l) ke.kg[l] = static_cast<const uint16_t*>(knorms[l]);
      ke.eps = w->rms_eps;
      HIP_TRY(launch_gemm_kv_bf16(x, H, n, wt, wp, ke, st));
    } else {  // fewer tiles than CUs: the separate epilogue kernel spreads wider
      float* y = at<float>(ws, Lw.y);
      HIP_TRY(launch_gemm_bf16(x, H, n, wt, wp, H, y, KV_N, KV_N, 1, 0, st));
      HIP_TRY(launch_kv_post(y, KV_N, 1, 0, n, pos0, knorms, w->rms_eps, theta, rk, rv, kv->capacity, st));
    }
  }
  return DFLASH_OK;
}

namespace {
// Shared body of dflash_draft_block and dflash_draft_block_gated (conf and
// nkeep null for the former).
// static_ws: the workspace is the library's device array (ws and ws_bytes
// ignored), resolved after the arguments are checked.
// taps / nc: commit rows of the fused draft-commit cycle (nc = 0: none),
// at positions p - nc .. p - 1.
// Positions of a pass held in device memory: {p, anchor, n_commit} (int64),
// with the commit taps as rows of a position-indexed buffer.
struct DevPos {
  const int64_t* state;
  const void* taps;
  int64_t taps_pos0, taps_rows;
};

int32_t draft_block_impl(const dflash_weights* w, const dflash_kv* kv, int64_t p,
                         int32_t anchor_id, int32_t mask_id, int32_t block, int32_t* cand,
                         float* conf, int32_t* nkeep, float min_p, void* logits_opt,
                         void* hidden_opt, void* ws, size_t ws_bytes, void* stream,
                         bool static_ws = false, const void* taps = nullptr, int32_t nc = 0,
                         const DevPos* dev = nullptr) {
  int rc = check_weights(w);
  if (rc) return rc;
  rc = check_kv(kv);
  if (rc) return rc;
  if (dev) {  // p, the anchor and n_commit are checked by the kernels when they read them
    if (!dev->state || (reinterpret_cast<uintptr_t>(dev->state) & 7u) || !dev->taps ||
        !a16(dev->taps) || dev->taps_pos0 < 0 || dev->taps_rows < 0)
      return DFLASH_EINVAL;
    p = 0;
    anchor_id = 0;
    nc = 0;
  }
  if (block < 1 || block > MAXB || p < 0) return DFLASH_EINVAL;
  if (nc < 0 || nc > MAXB || p < nc || (nc > 0 && (!taps || !a16(taps)))) return DFLASH_EINVAL;
  if (anchor_id < 0 || anchor_id >= w->vocab || mask_id < 0 || mask_id >= w->vocab)
    return DFLASH_EINVAL;
  if ((!ws && !static_ws) || (block > 1 && !cand)) return DFLASH_EINVAL;
  if (!a16(ws) || !a16(logits_opt) || !a16(hidden_opt) || (reinterpret_cast<uintptr_t>(cand) & 3u))
    return DFLASH_EINVAL;
  const Layout Lw = layout();
  if (static_ws) {
    ws = scratch_on_device();
    ws_bytes = SCRATCH_BYTES;
    if (!ws) return DFLASH_EHIP;
  }
  if (ws_bytes < Lw.fixed) return DFLASH_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!w->packed) return DFLASH_EINVAL;  // the streaming copy (dflash_pack_weights)
  const int grid = pass_grid();
  if (grid < QKV_N / 32) return DFLASH_EHIP;  // the pass needs >= 224 resident blocks
  PassLaunch q;
  q.fmt = w->backbone_type;
  for (int l = 0; l < L; ++l) {
    const dflash_layer_weights& y = w->layer[l];
    uint8_t* pm[7];  // the pass streams the packed copies
    packed_layer(w, l, pm);
    q.wq[l] = u16p(pm[0]);
    q.wk[l] = u16p(pm[1]);
    q.wv[l] = u16p(pm[2]);
    q.wo[l] = u16p(pm[3]);
    q.wg[l] = u16p(pm[4]);
    q.wu[l] = u16p(pm[5]);
    q.wd[l] = u16p(pm[6]);
    q.in_norm[l] = u16p(y.in_norm);
    q.q_norm[l] = u16p(y.q_norm);
    q.k_norm[l] = u16p(y.k_norm);
    q.post_norm[l] = u16p(y.post_norm);
  }
  q.final_norm = u16p(w->final_norm);
  q.embed = u16p(w->embed);
  q.lm = u16p(w->packed);  // streaming copy of the LM head (bf16 or Q8_0)
  q.lm_fmt = w->lm_head_type;
  q.vocab = w->vocab;
  q.eps = w->rms_eps;
  q.scale_log2 = w->attn_scale * 1.4426950408889634f;
  q.theta = static_cast<double>(w->rope_theta);
  q.ring_k = static_cast<const uint16_t*>(kv->k);
  q.ring_vt = static_cast<const uint16_t*>(kv->vt);
  q.cap = kv->capacity;
  // Attention split over the visible context [lo, p): one block per (KV head,
  // chunk of cb 32-cell blocks), at most min(grid / 2, 128) chunks per head;
  // the last chunk of each head also takes the block rows.
  // Commit rows (positions p-nc .. p-1) are attended to from the workspace:
  // the ring is read at [lo, p - nc).
  q.lo = p - kv->window > 0 ? p - kv->window : 0;
  q.hi = p - nc;
  if (q.hi > q.lo) {
    const int maxch = grid / 2 < 128 ? grid / 2 : 128;
    q.p0 = q.lo & ~static_cast<int64_t>(31);
    q.nb = static_cast<int>((q.hi - q.p0 + 31) / 32);
    q.cb = (q.nb + maxch - 1) / maxch;
    q.nch = (q.nb + q.cb - 1) / q.cb;
  } else {
    q.p0 = 0;
    q.nb = 0;
    q.cb = 1;
    q.nch = 1;  // block rows only
  }
  q.B = block;
  q.p = p;
  q.anchor = anchor_id;
  q.mask = mask_id;
  q.h = at<float>(ws, Lw.hv);
  q.h16 = at<uint16_t>(ws, Lw.h16);
  q.ss = at<float>(ws, Lw.ss);
  q.qkv = at<uint16_t>(ws, Lw.qkv);
  q.rope = at<float2>(ws, Lw.rope);
  q.po = at<uint16_t>(ws, Lw.po);
  q.pm = at<float>(ws, Lw.pm);
  q.pl = at<float>(ws, Lw.pl);
  q.o16 = at<uint16_t>(ws, Lw.ov);
  q.u16 = at<uint16_t>(ws, Lw.uv);
  q.keys = at<uint64_t>(ws, Lw.keys);
  q.bar = at<unsigned>(ws, Lw.bar);
  q.tab = at<void>(ws, Lw.tab);
  const double tpu = ticks_per_us();
  if (tpu <= 0.0) return DFLASH_EHIP;
  q.wait_ticks = static_cast<uint64_t>(static_cast<double>(barrier_wait_us()) * tpu);
  q.grid = grid;
  q.cand = cand;
  q.logits = static_cast<uint16_t*>(logits_opt);
  q.hidden = static_cast<uint16_t*>(hidden_opt);
  q.lse = at<uint64_t>(ws, Lw.lse);
  q.conf = conf;
  q.nkeep = nkeep;
  q.min_p = min_p;
  q.nc = nc;
  q.pos0 = p - nc;
  q.taps = static_cast<const uint16_t*>(taps);
  q.fc = packed_fc(w);
  q.hidden_norm = u16p(w->hidden_norm);
  q.yc = at<float>(ws, Lw.yc);
  q.fcp = at<float>(ws, Lw.fcp);
  q.cn = at<uint16_t>(ws, Lw.cn);
  q.ckv = at<float>(ws, Lw.ckv);
  if (dev) {
    q.dstate = dev->state;
    q.taps_base = static_cast<const uint16_t*>(dev->taps);
    q.taps_pos0 = dev->taps_pos0;
    q.taps_rows = dev->taps_rows;
    q.window = kv->window;
    q.maxch = grid / 2 < 128 ? grid / 2 : 128;
  }
  HIP_TRY(launch_draft_pass(q, st));
  return DFLASH_OK;
}
}  // namespace

extern "C" int32_t dflash_draft_block(const dflash_weights* w, const dflash_kv* kv, int64_t p,
                                      int32_t anchor_id, int32_t mask_id, int32_t block,
                                      int32_t* cand, void* logits_opt, void* hidden_opt,
                                      void* ws, size_t ws_bytes, void* stream) {
  return draft_block_impl(w, kv, p, anchor_id, mask_id, block, cand, nullptr, nullptr, 0.f,
                          logits_opt, hidden_opt, ws, ws_bytes, stream);
}

extern "C" int32_t dflash_draft_block_commit(const dflash_weights* w, const dflash_kv* kv,
                                             const void* taps, int32_t n_commit, int64_t p,
                                             int32_t anchor_id, int32_t mask_id, int32_t block,
                                             int32_t* cand, void* logits_opt, void* hidden_opt,
                                             void* ws, size_t ws_bytes, void* stream) {
  return draft_block_impl(w, kv, p, anchor_id, mask_id, block, cand, nullptr, nullptr, 0.f,
                          logits_opt, hidden_opt, ws, ws_bytes, stream, false, taps, n_commit);
}

extern "C" int32_t dflash_draft_block_commit_dev(const dflash_weights* w, const dflash_kv* kv,
                                                 const void* taps, int64_t taps_pos0,
                                                 int64_t taps_rows, const int64_t* state,
                                                 int32_t mask_id, int32_t block, int32_t* cand,
                                                 void* logits_opt, void* hidden_opt, void* ws,
                                                 size_t ws_bytes, void* stream) {
  const DevPos dev{state, taps, taps_pos0, taps_rows};
  return draft_block_impl(w, kv, 0, 0, mask_id, block, cand, nullptr, nullptr, 0.f, logits_opt,
                          hidden_opt, ws, ws_bytes, stream, false, nullptr, 0, &dev);
}

extern "C" int32_t dflash_draft_block_static(const dflash_weights* w, const dflash_kv* kv,
                                             int64_t p, int32_t anchor_id, int32_t mask_id,
                                             int32_t block, int32_t* cand, void* logits_opt,
                                             void* hidden_opt, void* stream) {
  static_assert(SCRATCH_BYTES % 256 == 0, "scratch holds whole 256-byte workspace regions");
  return draft_block_impl(w, kv, p, anchor_id, mask_id, block, cand, nullptr, nullptr, 0.f,
                          logits_opt, hidden_opt, nullptr, 0, stream, true);
}

extern "C" int32_t dflash_draft_block_gated(const dflash_weights* w, const dflash_kv* kv,
                                            int64_t p, int32_t anchor_id, int32_t mask_id,
                                            int32_t block, float min_p, int32_t* cand,
                                            float* conf, int32_t* n_keep, void* ws,
                                            size_t ws_bytes, void* stream) {
  if (block < 2 || !cand || !conf || !n_keep) return DFLASH_EINVAL;
  if ((reinterpret_cast<uintptr_t>(conf) & 3u) || (reinterpret_cast<uintptr_t>(n_keep) & 3u))
    return DFLASH_EINVAL;
  if (!(min_p >= 0.f && min_p <= 1.f)) return DFLASH_EINVAL;  // rejects NaN too
  return draft_block_impl(w, kv, p, anchor_id, mask_id, block, cand, conf, n_keep, min_p,
                          nullptr, nullptr, ws, ws_bytes, stream);
}

extern "C" int32_t dflash_lm_head_argmax(const dflash_weights* w, const void* hidden,
                                         int32_t rows, int32_t* cand, void* logits_opt, void* ws,
                                         size_t ws_bytes, void* stream) {
  int rc = check_weights(w);
  if (rc) return rc;
  if (rows < 1 || rows > MAXB || !hidden || !cand || !ws) return DFLASH_EINVAL;
  if (!a16(hidden) || !a16(ws) || !a16(logits_opt) || (reinterpret_cast<uintptr_t>(cand) & 3u))
    return DFLASH_EINVAL;
  const Layout Lw = layout();
  if (ws_bytes < Lw.fixed) return DFLASH_EWORKSPACE;
  HIP_TRY(launch_lmhead_argmax(w->packed ? w->packed : w->lm_head, w->lm_head_type,
                               w->packed != nullptr, w->vocab, u16p(hidden), rows,
                               at<uint64_t>(ws, Lw.keys), LMH_GRID,
                               static_cast<uint16_t*>(logits_opt), cand,
                               static_cast<hipStream_t>(stream)));
  return DFLASH_OK;
}

extern "C" int32_t dflash_verify_greedy(const int32_t* cand, const int32_t* target, int32_t k,
                                        int32_t* out, void* stream) {
  if (k < 0 || k > MAXB - 1) return DFLASH_EINVAL;
  if (!target || !out || (k > 0 && !cand)) return DFLASH_EINVAL;
  if (launch_verify(cand, target, k, nullptr, out, nullptr, static_cast<hipStream_t>(stream)) != hipSuccess)
    return DFLASH_EHIP;
  return DFLASH_OK;
}

extern "C" int32_t dflash_verify_greedy_gated(const int32_t* cand, const int32_t* target,
                                              int32_t k_max, const int32_t* n_keep, int32_t* out,
                                              void* stream) {
  if (k_max < 0 || k_max > MAXB - 1) return DFLASH_EINVAL;
  if (!target || !out || !n_keep || (k_max > 0 && !cand)) return DFLASH_EINVAL;
  if ((reinterpret_cast<uintptr_t>(n_keep) & 3u) || (reinterpret_cast<uintptr_t>(out) & 3u) ||
      (reinterpret_cast<uintptr_t>(target) & 3u) || (reinterpret_cast<uintptr_t>(cand) & 3u))
    return DFLASH_EINVAL;
  if (launch_verify(cand, target, k_max, n_keep, out, nullptr, static_cast<hipStream_t>(stream)) != hipSuccess)
    return DFLASH_EHIP;
  return DFLASH_OK;
}

extern "C" int32_t dflash_verify_greedy_advance(const int32_t* cand, const int32_t* target,
                                                int32_t k, int64_t* state, int32_t* out,
                                                void* stream) {
  if (k < 0 || k > MAXB - 1) return DFLASH_EINVAL;
  if (!target || !out || !state || (k > 0 && !cand)) return DFLASH_EINVAL;
  if ((reinterpret_cast<uintptr_t>(state) & 7u) || (reinterpret_cast<uintptr_t>(out) & 3u) ||
      (reinterpret_cast<uintptr_t>(target) & 3u) || (reinterpret_cast<uintptr_t>(cand) & 3u))
    return DFLASH_EINVAL;
  if (launch_verify(cand, target, k, nullptr, out, state, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return DFLASH_EHIP;
  return DFLASH_OK;
}

extern "C" int32_t dflash_draft_status(const void* ws, size_t ws_bytes, int32_t* status,
                                       void* stream) {
  if (!ws || !status || !a16(ws) || (reinterpret_cast<uintptr_t>(status) & 3u)) return DFLASH_EINVAL;
  const Layout Lw = layout();
  if (ws_bytes < Lw.fixed) return DFLASH_EWORKSPACE;
  HIP_TRY(launch_pass_status(at<const unsigned>(const_cast<void*>(ws), Lw.bar), status,
                             DFLASH_ETIMEOUT, DFLASH_EINVAL, static_cast<hipStream_t>(stream)));
  return DFLASH_OK;
}

extern "C" int32_t dflash_draft_stage(const void* ws, size_t ws_bytes, int32_t stage, int32_t index,
                                      int32_t rows, void* dst, size_t dst_bytes, void* stream) {
  if (!ws || !dst || !a16(ws) || !a16(dst) || rows < 1 || rows > MAXB) return DFLASH_EINVAL;
  const Layout Lw = layout();
  if (ws_bytes < Lw.fixed) return DFLASH_EWORKSPACE;
  // per-layer regions hold MAXB rows each; rows 0..rows-1 are contiguous
  size_t base, row_bytes, slot_bytes;
  int32_t count;
  switch (stage) {
    case DFLASH_STAGE_RESIDUAL:
      base = Lw.hv, row_bytes = sizeof(float) * H, count = 2 * dfl::L + 1;
      break;
    case DFLASH_STAGE_QKV:
      base = Lw.qkv, row_bytes = 2 * static_cast<size_t>(QKV_N), count = dfl::L;
      break;
    case DFLASH_STAGE_ATTN:
      base = Lw.ov, row_bytes = 2 * static_cast<size_t>(NQ) * D, count = dfl::L;
      break;
    case DFLASH_STAGE_MLP:
      base = Lw.uv, row_bytes = 2 * static_cast<size_t>(F), count = dfl::L;
      break;
    default: return DFLASH_EINVAL;
  }
  if (index < 0 || index >= count) return DFLASH_EINVAL;
  slot_bytes = row_bytes * MAXB;
  const size_t n = row_bytes * static_cast<size_t>(rows);
  if (dst_bytes < n) return DFLASH_EINVAL;
  HIP_TRY(hipMemcpyAsync(dst, static_cast<const char*>(ws) + base + slot_bytes * index, n,
                         hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream)));
  return DFLASH_OK;
}

extern "C" int32_t dflash_check_finite(const void* x, int64_t count, int32_t dtype, int32_t* status,
                                       void* stream) {
  if (!status || (reinterpret_cast<uintptr_t>(status) & 3) || count < 0 || dtype < 0 || dtype > 2)
    return DFLASH_EINVAL;
  if (count > 0 && (!x || !a16(x))) return DFLASH_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  HIP_TRY(launch_check_finite(x, count, dtype, status, DFLASH_ENONFINITE, st));
  return DFLASH_OK;
}

extern "C" const char* dflash_strerror(int32_t code) {
  switch (code) {
    case DFLASH_OK: return "ok";
    case DFLASH_EINVAL: return "invalid argument";
    case DFLASH_EGEOMETRY: return "descriptor does not match the DFlash geometry";
    case DFLASH_ERANGE: return "K/V ring capacity/window/range violation";
    case DFLASH_EWORKSPACE: return "workspace too small";
    case DFLASH_EHIP: return "HIP launch failed";
    case DFLASH_ENONFINITE: return "non-finite value found";
    case DFLASH_ETIMEOUT: return "proposal pass gave up waiting at a grid barrier";
    default: return "unknown error";
  }
}
