/*
 * dflash.h -- C ABI of the MI355X (gfx950) DFlash block-drafter library.
 *
 * The library computes the proposal pass of the standalone DeepSpec DFlash
 * block drafter described on the Strata PR #1426 page ("dflash: experimental
 * standalone DeepSpec DFlash block drafter for Qwen3.8-Flash-Next"):
 *   - context fusion rmsnorm(fc(concat(taps)))          (section "Drafter runtime")
 *   - per-layer context K/V projection, fp16 cells      ("Drafter runtime",
 *                                                         "Owned DFlash K/V state")
 *   - one parallel, non-causal five-layer forward over [anchor, mask x K]
 *     with a greedy argmax through the shared LM head   ("Target feature taps",
 *                                                         "Drafter runtime")
 *   - greedy verification of the K candidates           ("Speculative decode
 *                                                         integration"; Strata RFC
 *                                                         #366, "Verification and
 *                                                         state management")
 *
 * Conventions for every entry point
 *   - Pointers are device pointers (HBM of the current HIP device) unless a
 *     comment says "host".  The caller owns every buffer: weights, K/V ring,
 *     workspace and outputs.  The library allocates nothing, frees nothing and
 *     keeps no state between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     device work is enqueued on it and the call returns without waiting;
 *     results are valid once the stream has been synchronised.  Calls that
 *     share a workspace must be ordered on one stream.
 *   - Argument checks happen on the host before anything is enqueued; a
 *     non-zero return means nothing was enqueued (except DFLASH_EHIP, which
 *     reports a failed launch).
 *   - Device buffers (weights, streaming copies, K/V ring, workspace, inputs
 *     and outputs) must be 16-byte aligned; int32 buffers 4-byte aligned.
 *     Otherwise the call returns DFLASH_EINVAL.
 *   - bf16 is the upper half of an IEEE binary32; fp16 is IEEE binary16.
 *     Matrices are row-major [out][in].
 *   - Not thread-safe beyond stream order.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

/* Exported entry points; the library is built with hidden visibility, so
 * these are its only dynamic symbols. */
#define DFLASH_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define DFLASH_OK          0
#define DFLASH_EINVAL     -1 /* null or misaligned pointer, negative size, block
                                outside 1..8, token id outside [0, vocab),
                                position < 0 */
#define DFLASH_EGEOMETRY  -2 /* descriptor differs from the DFlash geometry */
#define DFLASH_ERANGE     -3 /* K/V ring: window > capacity, capacity not a
                                multiple of 256, or n > capacity in one call
                                (the only way one projection call can overwrite
                                a cell of the window that ends at its last
                                position: with window <= capacity, the cells it
                                evicts are older than that window) */
#define DFLASH_EWORKSPACE -4 /* workspace smaller than dflash_workspace_size() */
#define DFLASH_EHIP       -5 /* a kernel launch failed */
#define DFLASH_ENONFINITE -6 /* written by dflash_check_finite into its device
                                status word: a NaN or infinity was found */
#define DFLASH_ETIMEOUT   -7 /* written by dflash_draft_status into its device
                                status word: the last proposal pass gave up
                                waiting at a grid barrier (outputs undefined) */

/* Fixed drafter geometry ("Drafter runtime" on the PR #1426 page). */
#define DFLASH_HIDDEN     2560
#define DFLASH_LAYERS     5
#define DFLASH_Q_HEADS    24
#define DFLASH_KV_HEADS   2
#define DFLASH_HEAD_DIM   256
#define DFLASH_FFN        7680
#define DFLASH_TAPS       5
#define DFLASH_MAX_BLOCK  8   /* anchor + at most 7 candidates ("Current limitations") */

/* Storage format of the 36 backbone matrices (fc and the 35 layer matrices;
 * the PR #3322 pages list BF16, Q8_0, Q5_0 and Q4_0 backbones).  The
 * quantized formats use 32-element blocks along the input dimension of each
 * output row, one fp16 scale per block.  A quantized [N][K] matrix is one
 * buffer:
 *   Q8_0: N*K int8 values (row-major), then N*K/32 fp16 scales (row-major);
 *         weight = scale * q.
 *   Q4_0: N*K/2 bytes (row-major, 16 bytes per block: element j of a block in
 *         the low nibble of byte j, element j+16 in the high nibble), then
 *         N*K/32 fp16 scales; weight = scale * (nibble - 8).
 *   Q5_0: Q4_0's nibbles and scales, then N*K/32 little-endian uint32 words
 *         (row-major, one per block: bit j is the fifth bit of element j);
 *         weight = scale * ((nibble | bit << 4) - 16).
 * Gains and the embedding are always bf16; the LM head is bf16 or Q8_0
 * (lm_head_type). */
typedef enum {
  DFLASH_W_BF16 = 0,
  DFLASH_W_Q8_0 = 1,
  DFLASH_W_Q4_0 = 2,
  DFLASH_W_Q5_0 = 3
} dflash_wtype;

typedef struct {
  const void* in_norm;   /* bf16 [2560]       input RMSNorm gain            */
  const void* wq;        /* [6144][2560]       query projection              */
  const void* wk;        /* [512][2560]        key projection                */
  const void* wv;        /* [512][2560]        value projection              */
  const void* q_norm;    /* bf16 [256]         per-head query RMSNorm gain   */
  const void* k_norm;    /* bf16 [256]         per-head key RMSNorm gain     */
  const void* wo;        /* [2560][6144]       output projection             */
  const void* post_norm; /* bf16 [2560]        post-attention RMSNorm gain   */
  const void* wg;        /* [7680][2560]       MLP gate                      */
  const void* wu;        /* [7680][2560]       MLP up                        */
  const void* wd;        /* [2560][7680]       MLP down                      */
} dflash_layer_weights;

/* Caller-owned weight descriptor; must not change during a call. */
typedef struct {
  int32_t hidden, n_layers, n_q_heads, n_kv_heads, head_dim, ffn, vocab, n_taps;
  float rope_theta;      /* 1e7                                               */
  float attn_scale;      /* 1/16                                              */
  float rms_eps;         /* 1e-6                                              */
  int32_t backbone_type; /* dflash_wtype                                      */
  const void* fc;        /* [2560][12800]      fusion projection             */
  const void* hidden_norm; /* bf16 [2560]      fusion RMSNorm gain           */
  dflash_layer_weights layer[DFLASH_LAYERS];
  const void* final_norm;  /* bf16 [2560]                                     */
  const void* embed;       /* bf16 [vocab][2560] target embedding (shared)    */
  const void* lm_head;     /* bf16 [vocab][2560] target LM head (shared)      */
  /* Device buffer of dflash_packed_size() bytes holding the streaming
   * copies of the matrices the calls stream (the LM head, every layer's seven
   * matrices and fc, in the backbone's format), written by
   * dflash_pack_weights after the weights are loaded (and again whenever
   * those tensors change).  Required by dflash_draft_block (NULL ->
   * DFLASH_EINVAL).  When it is set, every call reads the matrices from it
   * (a quantized backbone's many-row fusion / projection decodes its blocks
   * from here) and the row-major matrix pointers above (fc, the 35 layer
   * matrices, lm_head) may be NULL: the weights can then be held once, in
   * the streaming layout.  Gains and the embedding are always read from
   * their own pointers.  Without it, the row-major matrices are required and
   * read directly.  Caller-owned, like everything else. */
  void* packed;
  /* Storage format of lm_head (PR #3322 later snapshot, "How to enable the
   * pushed optimization options": a shared LM head in Q8_0):
   * DFLASH_W_BF16 (0) or DFLASH_W_Q8_0 -- blocks of 32 consecutive input-dim
   * weights of one vocabulary row with an fp16 scale, stored like the Q8_0
   * backbone (vocab*2560 int8 row-major, then vocab*80 fp16 scales).  The
   * embedding stays bf16 (a Q8_0 LM head is never tied to it).  With Q8_0
   * the pass and dflash_lm_head_argmax decode the blocks in registers and
   * take the contraction in fp16 x fp16 -> fp32; logits, argmax and the
   * confidence gate are otherwise unchanged.  Appended after `packed` so the
   * fields above keep their offsets. */
  int32_t lm_head_type;
} dflash_weights;

/* Drafter-owned context K/V ("Owned DFlash K/V state": fp16, one state per
 * layer).  Position m lives in cell m % capacity ("Speculative decode
 * integration": position-addressed cells, overwritten on a later commit).
 *   k : fp16 [5 layers][2 kv heads][capacity cells][256]
 *   vt: fp16 [5 layers][2 kv heads][capacity/32][256][32]  (values transposed in
 *       blocks of 32 cells: cell c, dimension d is at [c/32][d][c%32], so each
 *       32-cell block of values is one contiguous 16 KiB run)
 * capacity must be a multiple of 256 and >= window.  A draft at anchor
 * position p reads positions max(0, p-window) .. p-1, which must have been
 * projected (and not overwritten since) by the caller. */
typedef struct {
  void* k;
  void* vt;
  int32_t capacity;
  int32_t window;        /* 32768 by default ("Current limitations")         */
} dflash_kv;

/* Bytes of device workspace needed for calls with up to `max_rows` context
 * rows (fuse/project) and blocks of up to `max_block` rows (draft).  Returns 0
 * for invalid arguments. */
DFLASH_API size_t dflash_workspace_size(const dflash_weights* w, int32_t max_rows,
                             int32_t max_block);

/* Bytes of the streaming copies: vocab * 2560 LM-head weights at 2 (bf16) or
 * 34/32 (Q8_0) bytes each, plus the 35 layer matrices (5 x (6144*2560 +
 * 2*512*2560 + 2560*6144 + 2*7680*2560 + 2560*7680) weights) and fc
 * (2560*12800 weights) at 2 (bf16), 34/32 (Q8_0), 18/32 (Q4_0) or 22/32
 * (Q5_0) bytes per weight.  0 for an invalid descriptor. */
DFLASH_API size_t dflash_packed_size(const dflash_weights* w);

/* Writes the streaming copies into w->packed, enqueued on `stream`.  A bf16
 * [N][K] matrix becomes, in order, its 16-row tiles; within a tile its
 * 32-wide k blocks; within a block the 64 lanes of an MFMA 16x16x32 A operand
 * (lane L holds row L%16, k 8*(L/16) .. +8), 16 bytes per lane -- so every
 * 64-lane load of the draft pass reads 1 KiB of contiguous memory instead of
 * 64 bytes from each of 16 rows.  Element (n, k) sits at
 * ((n/16 * K/32 + k/32) * 64 + n%16 + 16 * ((k%32)/8)) * 8 + k%8.
 * Order in the buffer: lm_head [vocab][2560] (in lm_head_type); then for each layer 0..4:
 * wq [6144][2560], wk [512][2560], wv [512][2560], wo [2560][6144],
 * wg [7680][2560], wu [7680][2560], wd [2560][7680]; then fc [2560][12800].
 * A quantized matrix
 * keeps its parts: its quants get the same shuffle with each row seen as
 * 64-byte pieces (64 k for Q8_0, 128 k for Q4_0 / Q5_0) in place of
 * 32-element bf16 blocks, i.e. byte j of piece kb of row n at
 * ((n/16 * P + kb) * 64 + n%16 + 16 * (j/16)) * 16 + j%16 with P pieces per
 * row; its fp16 scales follow, the S = 2 (Q8_0) or 4 (Q4_0, Q5_0) scales of
 * piece kb of row n at ((n/16 * P + kb) * 16 + n%16) * S + s.  Q5_0's
 * high-bit words come last, word s of piece kb of row n at
 * ((n/16 * P + kb) * 16 + n%16) * 4 + s, each with its bits reordered for
 * the decoder: the fifth bit of element e = 8 a + 4 b + c of the block
 * (a < 4, b < 2, c < 4) at bit 2 a + b + 8 c.
 * Returns DFLASH_EINVAL if w->packed is NULL. */
DFLASH_API int32_t dflash_pack_weights(const dflash_weights* w, void* stream);

/* Context fusion ("Drafter runtime": rmsnorm(fc(concat(target taps)))).
 *   taps: bf16 [n][5][2560], the five target taps of each position in tap order
 *   ctx : bf16 [n][2560] output, ctx[t] = rmsnorm(fc . concat(taps[t]), hidden_norm)
 * n may be 0 (no work).  ws/ws_bytes: workspace. */
DFLASH_API int32_t dflash_fuse_context(const dflash_weights* w, const void* taps, int32_t n,
                            void* ctx, void* ws, size_t ws_bytes, void* stream);

/* Per-layer context K/V projection ("Drafter runtime": the fused context is
 * projected into independent per-layer K/V state).  For t in [0, n) and each
 * layer l and KV head j, position m = pos0 + t:
 *   K_l[j][m % cap] = fp16(RoPE_m(rmsnorm(Wk_l ctx[t])_j, k_norm_l))
 *   V_l[j][m % cap] = fp16((Wv_l ctx[t])_j)
 *   ctx: bf16 [n][2560] (output of dflash_fuse_context); pos0 >= 0; n <= capacity. */
DFLASH_API int32_t dflash_project_ctx_kv(const dflash_weights* w, const void* ctx, int32_t n,
                              int64_t pos0, const dflash_kv* kv, void* ws,
                              size_t ws_bytes, void* stream);

/* One parallel proposal pass ("Target feature taps", "Drafter runtime").
 * Block row 0 is the anchor token at position p, rows 1..block-1 the mask
 * token at p+1..p+block-1; attention is non-causal over the context window
 * and all block rows, scale 1/16.  Mask row i proposes position p+i:
 *   cand      : int32 [block-1]            greedy ids (lowest id on ties)
 *   logits_opt: bf16 [block-1][vocab] or NULL   LM-head logits of the mask rows
 *   hidden_opt: bf16 [block][2560] or NULL      final-normed hidden states
 * block in [1, 8]; anchor_id, mask_id in [0, vocab); p >= 0.  Reads the
 * streaming copy w->packed (see dflash_pack_weights), which must be current.
 * The pass is one persistent kernel of one block per compute unit whose
 * blocks wait for each other: it needs the whole device.  Every wait at a
 * grid barrier is bounded in wall-clock time (the device's constant-rate
 * counter): if other work keeps some of its blocks from starting for longer
 * than 0.5 s, the pass gives up, sets every cand to -1 and records the
 * give-up in the workspace (dflash_draft_status reads it); its outputs are
 * then undefined.  After one give-up no later barrier of the pass waits, so
 * the pass still ends about one bound after it started waiting.  The
 * environment variable DFLASH_BARRIER_TIMEOUT_US (read by the host on each
 * call, 0 .. 10000000 microseconds; 0 = give up after about 32 polls that
 * do not see the release) replaces the 0.5 s bound -- meant for tests. */
DFLASH_API int32_t dflash_draft_block(const dflash_weights* w, const dflash_kv* kv, int64_t p,
                           int32_t anchor_id, int32_t mask_id, int32_t block,
                           int32_t* cand, void* logits_opt, void* hidden_opt,
                           void* ws, size_t ws_bytes, void* stream);

/* One decode cycle's drafter work as one pass ("Speculative decode
 * integration" on the PR #1426 page: propose [anchor, K candidates], verify,
 * commit the accepted cells plus the verifier's continuation token as the
 * next anchor; position-addressed cells).  Equivalent to
 *   dflash_fuse_context(taps, n_commit) ; dflash_project_ctx_kv(ctx, n_commit,
 *   pos0 = p - n_commit) ; dflash_draft_block(p, ...)
 * with one launch: the commit rows' fusion runs as a first phase of the pass
 * and their per-layer K/V projection rides the pass's own Wk / Wv weight
 * stream (extra MFMA columns), so a cycle streams the backbone once.  The
 * commit cells are written to the ring (as dflash_project_ctx_kv would) and
 * attended to by this pass from the workspace.
 *   taps    : bf16 [n_commit][5][2560], the target taps of positions
 *             p - n_commit .. p - 1 (the anchor and accepted candidates of
 *             the previous cycle); may be NULL when n_commit is 0
 *   n_commit: 0 .. 8 (0: a plain dflash_draft_block); p >= n_commit
 * Other arguments, outputs, checks and give-up behaviour as
 * dflash_draft_block.  The candidates and logits agree with the separate
 * calls within rounding (the fusion's sums run in another order). */
DFLASH_API int32_t dflash_draft_block_commit(const dflash_weights* w, const dflash_kv* kv,
                                  const void* taps, int32_t n_commit, int64_t p,
                                  int32_t anchor_id, int32_t mask_id, int32_t block,
                                  int32_t* cand, void* logits_opt, void* hidden_opt,
                                  void* ws, size_t ws_bytes, void* stream);

/* The decode cycle with its positions in device memory, so that a cycle
 * needs no device-to-host read ("Speculative decode integration" on the PR
 * #1426 page: each cycle commits what the last verify accepted and drafts at
 * the next position; the PR #3322 page's "Draft attention fix (2026-10-20)"
 * replays drafting windows from a graph).  Same pass as
 * dflash_draft_block_commit, with p, anchor_id and n_commit read by the
 * kernels, when they run, from
 *   state : int64 [3] device words {p, anchor_id, n_commit} (8-byte
 *           aligned), advanced by dflash_verify_greedy_advance
 *   taps  : bf16 [taps_rows][5][2560] device buffer, row r holding the target
 *           taps of position taps_pos0 + r; the commit rows are positions
 *           p - n_commit .. p - 1, which must lie in it
 * The state is checked on the device as the host entry points check their
 * arguments (p >= n_commit, n_commit in 0..8, anchor_id in [0, vocab), the
 * commit rows inside taps); when it fails the pass reads nothing from it,
 * writes cand = -1 (conf NaN, n_keep 0) and dflash_draft_status reports
 * DFLASH_EINVAL.  Host checks (returned): as dflash_draft_block, plus state
 * and taps non-NULL and aligned, taps_pos0 >= 0, taps_rows >= 0. */
DFLASH_API int32_t dflash_draft_block_commit_dev(const dflash_weights* w, const dflash_kv* kv,
                                                 const void* taps, int64_t taps_pos0,
                                                 int64_t taps_rows, const int64_t* state,
                                                 int32_t mask_id, int32_t block, int32_t* cand,
                                                 void* logits_opt, void* hidden_opt, void* ws,
                                                 size_t ws_bytes, void* stream);

/* dflash_draft_block for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument; the pass runs in a 67 MiB device array
 * inside the library (each device the library runs on holds its own copy
 * from the first call until the process ends; the pass needs 66.5 MiB of it
 * whatever the context length and block size, and a layout that would not
 * fit returns DFLASH_EWORKSPACE).  The call allocates nothing: on its first
 * call on a device it only looks up the array's device address.  Same
 * arguments (minus the workspace), checks, outputs and give-up behaviour as
 * dflash_draft_block.  Every call on one device shares that device's array:
 * calls on one device must be ordered on one stream (calls that overlap in
 * time on one device race and give undefined results). */
DFLASH_API int32_t dflash_draft_block_static(const dflash_weights* w, const dflash_kv* kv, int64_t p,
                                  int32_t anchor_id, int32_t mask_id, int32_t block,
                                  int32_t* cand, void* logits_opt, void* hidden_opt,
                                  void* stream);

/* One proposal pass with a confidence gate (PR #3322 "support the official
 * Flash-Next DFlash2 checkpoint", section "Long-prompt diagnosis and fix": the
 * spec-min-p probability floor, default 0.5, cut verify rows 133 -> 113; its
 * later snapshot's 256K run uses spec_min_p=0.7).  Reading: a candidate's
 * probability is its softmax probability under the drafter's logits.  Same
 * pass, inputs and cand as dflash_draft_block; in the same vocabulary sweep
 * the LM head also keeps each mask row's softmax normaliser, so that
 *   conf  : fp32 [block-1]  conf[i] = softmax(logits_i)[cand[i]]
 *                           = exp(l_max - logsumexp(logits_i)) = 1 / sum_v exp(l_v - l_max),
 *                           on the fp32 logits the argmax is decided on
 *   n_keep: int32 device word = number of leading candidates with
 *           conf >= min_p (the proposal is cut at the first one below it;
 *           min_p = 0 keeps all block-1)
 * block in [2, 8]; min_p in [0, 1] (else DFLASH_EINVAL); cand, conf, n_keep
 * non-null and 4-byte aligned.  No logits / hidden outputs.  No extra weight
 * traffic.  A pass whose barriers gave up waiting sets cand to -1, conf to
 * NaN and n_keep to 0. */
DFLASH_API int32_t dflash_draft_block_gated(const dflash_weights* w, const dflash_kv* kv, int64_t p,
                                 int32_t anchor_id, int32_t mask_id, int32_t block,
                                 float min_p, int32_t* cand, float* conf, int32_t* n_keep,
                                 void* ws, size_t ws_bytes, void* stream);

/* Greedy argmax through the shared LM head ("Drafter runtime": target LM head
 * reused directly; greedy proposal path) for final-normed hidden rows:
 *   hidden    : bf16 [rows][2560]  final-normed hidden states
 *   cand      : int32 [rows]       argmax_v (lm_head[v] . hidden[r]), lowest v on ties,
 *                                   decided on fp32 logits
 *   logits_opt: bf16 [rows][vocab] or NULL
 * rows in [1, 8].  Reads w->packed when set, else w->lm_head; both give the
 * same bits.  dflash_draft_block computes the same readout on its mask rows. */
DFLASH_API int32_t dflash_lm_head_argmax(const dflash_weights* w, const void* hidden, int32_t rows,
                              int32_t* cand, void* logits_opt, void* ws, size_t ws_bytes,
                              void* stream);

/* Greedy verification ("Speculative decode integration"; RFC #366
 * "Verification and state management").
 *   cand  : int32 [k]   proposals for positions p+1..p+k
 *   target: int32 [k+1] the target's greedy tokens for the same positions and
 *           the one after
 *   out   : int32 [2] = {accepted, next}: accepted = longest prefix with
 *           cand[i] == target[i]; next = target[accepted] (the verifier's
 *           continuation token).  k in [0, 7]. */
DFLASH_API int32_t dflash_verify_greedy(const int32_t* cand, const int32_t* target, int32_t k,
                             int32_t* out, void* stream);

/* dflash_verify_greedy that also advances a device-resident decode state
 * (the state words of dflash_draft_block_commit_dev): after computing
 * out = {accepted, next} it sets p += accepted + 1, anchor_id = next and
 * n_commit = accepted + 1, so the next cycle's pass commits the accepted
 * candidates' cells and the anchor's and drafts after them (RFC #366,
 * "Verification and state management": the accepted tokens plus the
 * verifier's continuation token are committed).  state: int64 [3], 8-byte
 * aligned; other arguments as dflash_verify_greedy (pointers 4-byte
 * aligned). */
DFLASH_API int32_t dflash_verify_greedy_advance(const int32_t* cand, const int32_t* target,
                                                int32_t k, int64_t* state, int32_t* out,
                                                void* stream);

/* Greedy verification of the candidates a confidence gate kept, with the
 * count read on the device (the n_keep word of dflash_draft_block_gated), so
 * that truncating the proposal needs no device-to-host read (PR #3322,
 * "Long-prompt diagnosis and fix": the floor cuts the rows the target
 * verifies).  Same as dflash_verify_greedy with k = min(max(*n_keep, 0),
 * k_max), read when the kernel runs:
 *   cand  : int32 [k_max]     target: int32 [k_max+1] (entries past k+1 unused)
 *   n_keep: int32 device word  out: int32 [2] = {accepted, next}
 * k_max in [0, 7]; all pointers 4-byte aligned. */
DFLASH_API int32_t dflash_verify_greedy_gated(const int32_t* cand, const int32_t* target, int32_t k_max,
                                   const int32_t* n_keep, int32_t* out, void* stream);

/* Outcome of the last proposal pass (any dflash_draft_block* entry point
 * with a workspace) enqueued with the workspace `ws`: writes, in stream order
 * after that pass, DFLASH_OK, DFLASH_ETIMEOUT (the pass gave up waiting at a
 * grid barrier) or DFLASH_EINVAL (dflash_draft_block_commit_dev found its
 * device state invalid and did nothing) into the int32 device word
 * `status`.  Lets callers that read only logits_opt / hidden_opt, or block 1
 * (no candidates), see a give-up.  Undefined before the workspace's first
 * pass. */
DFLASH_API int32_t dflash_draft_status(const void* ws, size_t ws_bytes, int32_t* status, void* stream);

/* Optional finite check of a device buffer, for callers that want the
 * pages' refusal of non-finite values (RFC #366 page, "3. First small
 * experiment: verifier and rollback correctness", pass criteria: no
 * non-finite values are introduced; the DFlash2 test list on the PR #3322
 * page: nonfinite refusal).  No other entry point calls it: it costs one read
 * of the buffer, so it is a debugging aid -- e.g. on the taps before
 * dflash_fuse_context, on the context or the K/V ring after
 * dflash_project_ctx_kv, on logits_opt / hidden_opt after dflash_draft_block.
 *   x     : device buffer of `count` elements (16-byte aligned)
 *   dtype : 0 = bf16, 1 = fp16, 2 = fp32
 *   status: int32 device word; enqueued on `stream`, it is set to DFLASH_OK
 *           and then, if any of the count elements is NaN or +-infinity (all
 *           exponent bits set), to DFLASH_ENONFINITE.  count 0 -> DFLASH_OK.
 * Returns DFLASH_EINVAL for a null or misaligned pointer (x may be NULL only
 * when count is 0), count < 0 or an unknown dtype. */
DFLASH_API int32_t dflash_check_finite(const void* x, int64_t count, int32_t dtype, int32_t* status,
                            void* stream);

/* Stage readout of the last proposal pass run in a workspace, for stage-wise
 * parity ("Parity validation" on the PR #1426 page compares every block row
 * at every stage of the layer, not only the logits).  The pass keeps each
 * layer's intermediates in the caller's workspace; this copies one of them,
 * rows 0..rows-1 (rows = the pass's block, 1..8), into dst on `stream`:
 *   DFLASH_STAGE_RESIDUAL, index v in [0, 2*5]: fp32 [rows][2560], the
 *     residual stream: v = 0 the block-token embeddings, v = 2l+1 after
 *     layer l's attention residual, v = 2l+2 after its MLP residual (v = 10
 *     is the input of the final norm)
 *   DFLASH_STAGE_QKV, index l in [0, 5): fp16 [rows][7168], layer l's raw
 *     projections q (24 heads x 256) | k (2 x 256) | v (2 x 256) before the
 *     q/k norms
 *   DFLASH_STAGE_ATTN, index l: [rows][24 x 256] attention output of layer
 *     l (head-major, before the output projection), in the activation format
 *     (bf16 beside bf16 weights, fp16 beside Q8_0 / Q4_0 weights)
 *   DFLASH_STAGE_MLP, index l: [rows][7680] SiLU(gate) * up of layer l, in
 *     the activation format
 * dst: device buffer of at least dst_bytes >= the stage's size.  Valid after
 * dflash_draft_block, _gated or _commit on this workspace has run (stream
 * order) and before the next call that uses it; a pass that gave up at a
 * barrier leaves them undefined.  Errors: DFLASH_EINVAL (null / misaligned
 * pointer, unknown stage, index or rows out of range, dst_bytes too small),
 * DFLASH_EWORKSPACE, DFLASH_EHIP. */
#define DFLASH_STAGE_RESIDUAL 0
#define DFLASH_STAGE_QKV      1
#define DFLASH_STAGE_ATTN     2
#define DFLASH_STAGE_MLP      3
DFLASH_API int32_t dflash_draft_stage(const void* ws, size_t ws_bytes, int32_t stage, int32_t index,
                                      int32_t rows, void* dst, size_t dst_bytes, void* stream);

/* Static description of a return code (host string, never NULL). */
DFLASH_API const char* dflash_strerror(int32_t code);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H */
