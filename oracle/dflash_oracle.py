"""CPU oracle for the DFlash block-drafter proposal pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The library never
calls it, and it shares no code, table or helper with the HIP path.

Plain numpy in float64, written step by step from the pages:

* Strata PR #1426 page ("dflash: experimental standalone DeepSpec DFlash
  block drafter"), sections "Target feature taps" (anchor and mask rows,
  non-causal block attention, scale 1/16), "Drafter runtime" (geometry,
  NeoX RoPE theta 1e7, shared embedding / LM head, feature fusion
  rmsnorm(fc(concat(taps))), per-layer context K/V), "Owned DFlash K/V state"
  (FP16 K/V), "Speculative decode integration" ([anchor, K candidates],
  position-addressed cells, no drafter rollback), "Parity validation" (stage
  order xn, q raw, q normed, q, k, v, attention, attn+o+res, MLP, final
  norm) and "Current limitations" (greedy only, 32768-cell window, at most 7
  candidates).
* Strata RFC #366 page ("Investigate DFlash2 support"), section
  "Verification and state management" (commit the accepted tokens plus the
  verifier's continuation token).

Precision: everything is float64 except where a value is *stored* in a
format the pages or the library boundary fix: fused context rows are bf16
(the runtime executes in BF16 and the fusion output is handed to the
projection as bf16) and drafter K/V cells are fp16 ("Owned DFlash K/V
state").  The greedy argmax is taken on logits rounded to fp32, the
precision the GPU decides in; ties go to the lowest index.

Parity status: every stage has pins in tests/test_oracle_pins.py.  The
composite five-layer pass has no printed values on the pages to compare
against, so its end-to-end output is "parity unpinned" beyond those stage
pins and special cases.
"""
from __future__ import annotations

import numpy as np

GEOMETRY = dict(hidden=2560, n_layers=5, n_q_heads=24, n_kv_heads=2,
                head_dim=256, ffn=7680, vocab=151936, n_taps=5,
                rope_theta=1.0e7, attn_scale=1.0 / 16.0, rms_eps=1.0e-6,
                window=32768)


def geometry(**over) -> dict:
    g = dict(GEOMETRY)
    g.update(over)
    return g


# --------------------------------------------------------------------------
# Number formats (IEEE-754 binary16 and the bfloat16 truncation of binary32)
# --------------------------------------------------------------------------

def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns -> float64: the 16 bits are the upper half of an
    IEEE binary32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """float64 -> bf16 bit patterns, rounding to nearest with ties to even.
    The value is first rounded to binary32 (exact for every bf16 result of a
    binary32 input; double rounding only matters within 2^-24 relative of a
    tie, far below any tolerance used here)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def f16_decode(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def f16_round(x) -> np.ndarray:
    """float64 -> fp16 value (as float64), IEEE round-to-nearest-even."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


# --------------------------------------------------------------------------
# Weight access, including the Q8_0 / Q4_0 / Q5_0 block formats
# --------------------------------------------------------------------------

def dequant_q8_0(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Q8_0: blocks of 32 consecutive input-dim weights of one output row,
    one fp16 scale d per block, value = d * q with q int8.  Byte layout:
    rows*cols int8 quants, then rows*cols/32 fp16 scales."""
    nq = rows * cols
    q = raw[:nq].view(np.int8).astype(np.float64).reshape(rows, cols // 32, 32)
    d = f16_decode(raw[nq:nq + 2 * nq // 32].view(np.uint16))
    d = d.reshape(rows, cols // 32, 1)
    return (q * d).reshape(rows, cols)


def dequant_q4_0(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Q4_0: blocks of 32 weights, fp16 scale d, 16 bytes of nibbles; element
    j of the block is the low nibble of byte j and element j+16 the high
    nibble; value = d * (nibble - 8).  Byte layout: rows*cols/2 packed
    bytes, then rows*cols/32 fp16 scales."""
    nb = rows * cols // 2
    by = raw[:nb].reshape(rows, cols // 32, 16)
    lo = (by & 0x0F).astype(np.float64)
    hi = (by >> 4).astype(np.float64)
    nib = np.concatenate([lo, hi], axis=2)
    d = f16_decode(raw[nb:nb + 2 * rows * cols // 32].view(np.uint16))
    d = d.reshape(rows, cols // 32, 1)
    return ((nib - 8.0) * d).reshape(rows, cols)


def dequant_q5_0(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Q5_0: blocks of 32 weights, fp16 scale d, a 5-bit code per weight:
    the low four bits as in Q4_0 (element j of the block in the low nibble of
    byte j, element j+16 in the high nibble) and the fifth in bit j of the
    block's 32-bit word; value = d * (code - 16).  (PR #3322 names Q5_0
    among the backbone formats without defining it; this is the plain
    reading of a 5-bit sibling of Q4_0: offset half the code range.)  Byte
    layout: rows*cols/2 packed bytes, rows*cols/32 fp16 scales, then
    rows*cols/32 little-endian uint32 high-bit words."""
    nb = rows * cols // 2
    ns = rows * cols // 32
    by = raw[:nb].reshape(rows, cols // 32, 16)
    nib = np.concatenate([by & 0x0F, by >> 4], axis=2).astype(np.int64)
    d = f16_decode(raw[nb:nb + 2 * ns].view(np.uint16)).reshape(rows, cols // 32, 1)
    hw = raw[nb + 2 * ns:nb + 6 * ns].view("<u4").astype(np.int64).reshape(rows, cols // 32, 1)
    hbit = (hw >> np.arange(32)) & 1
    code = nib | (hbit << 4)
    return ((code - 16).astype(np.float64) * d).reshape(rows, cols)


def storage_format(w: dict, name: str) -> str:
    """Format of a stored matrix: the LM head has its own (bf16, or Q8_0 for
    the shared quantized head of PR #3322's later snapshot, "How to enable
    the pushed optimization options"); every other matrix has the
    backbone's."""
    if name == "lm_head":
        return w.get("__lm_format__", "bf16")
    return w.get("__format__", "bf16")


def matrix(w: dict, name: str, shape) -> np.ndarray:
    """A weight matrix [out][in] as float64, whatever its stored format."""
    fmt = storage_format(w, name)
    a = w[name]
    if a.dtype == np.uint16:
        return bf16_decode(a).reshape(shape)
    if fmt == "q8_0":
        return dequant_q8_0(a, *shape)
    if fmt == "q4_0":
        return dequant_q4_0(a, *shape)
    if fmt == "q5_0":
        return dequant_q5_0(a, *shape)
    raise ValueError(f"unknown weight format for {name}")


def gain(w: dict, name: str) -> np.ndarray:
    return bf16_decode(w[name])


def enable_cache(w: dict) -> dict:
    """Keep decoded float64 matrices with the weights so that repeated passes
    skip the decoding (about 8 bytes per weight of host memory)."""
    w["__cache__"] = {}
    return w


def matvec_rows(w: dict, name: str, shape, x: np.ndarray,
                chunk: int = 8192) -> np.ndarray:
    """y[b][o] = sum_i W[o][i] x[b][i], W converted to float64 a block of
    output rows at a time to bound memory."""
    rows, cols = shape
    cache = w.get("__cache__")
    if cache is not None:
        if name not in cache:
            cache[name] = matrix(w, name, shape)
        return x @ cache[name].T
    out = np.empty((x.shape[0], rows), dtype=np.float64)
    a = w[name]
    if a.dtype == np.uint16:
        a2 = a.reshape(rows, cols)
        for s in range(0, rows, chunk):
            e = min(rows, s + chunk)
            out[:, s:e] = x @ bf16_decode(a2[s:e]).T
        return out
    return x @ matrix(w, name, shape).T


# --------------------------------------------------------------------------
# Elementary steps
# --------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis (plain gain)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """theta^(-2i/head_dim), i = 0 .. head_dim/2 - 1 (full-head rotation)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


def rope_neox(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """NeoX-style rotary embedding over the full head: element i pairs with
    element i + D/2 and the pair turns by angle pos * theta^(-2i/D).  x has
    shape [..., n_rows, D] with one position per row (pos has n_rows
    entries).  Angles, sines and cosines are float64."""
    D = x.shape[-1]
    half = D // 2
    ang = np.asarray(pos, dtype=np.float64)[:, None] * rope_inv_freq(D, theta)[None, :]
    c = np.cos(ang)
    s = np.sin(ang)
    shape = [1] * (x.ndim - 2) + [len(pos), half]
    c = c.reshape(shape)
    s = s.reshape(shape)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
              scale: float) -> np.ndarray:
    """Softmax attention with no mask: q [R][D], k [S][D], v [S][D]
    -> [R][D]; weights = softmax_s(scale * q.k_s), max-subtracted."""
    s = (q @ k.T) * scale
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=1, keepdims=True)) @ v


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def argmax_lowest(x: np.ndarray) -> int:
    """Index of the largest entry; the lowest index among equal maxima."""
    return int(np.argmax(x))  # numpy returns the first occurrence


# --------------------------------------------------------------------------
# The four operations of the pass
# --------------------------------------------------------------------------

def fuse_context(w: dict, taps_bits: np.ndarray, g: dict | None = None,
                 chunk: int = 1024) -> np.ndarray:
    """Context fusion rmsnorm(fc(concat(taps))) ("Drafter runtime").
    taps_bits: bf16 bits [n][n_taps][H] in tap order.  Returns the fused
    context as bf16 bits [n][H]."""
    g = g or GEOMETRY
    H, T = g["hidden"], g["n_taps"]
    n = taps_bits.shape[0]
    out = np.empty((n, H), dtype=np.uint16)
    cache = w.get("__cache__")
    if cache is not None:
        if "fc" not in cache:
            cache["fc"] = matrix(w, "fc", (H, T * H))
        fc = cache["fc"]
    else:
        fc = matrix(w, "fc", (H, T * H))
    gh = gain(w, "hidden_norm")
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = bf16_decode(taps_bits[s:e].reshape(e - s, T * H))  # concat of taps
        y = x @ fc.T
        out[s:e] = bf16_round(rmsnorm(y, gh, g["rms_eps"]))
    return out


def project_ctx_kv(w: dict, ctx_bits: np.ndarray, pos0: int,
                   g: dict | None = None):
    """Per-layer context K/V ("Drafter runtime": the fused context is
    projected into independent per-layer K/V state).  The fused context row
    goes straight into each layer's Wk / Wv (it is already normalised); K
    then gets the per-head k-norm and RoPE at the row's absolute position,
    like block keys.  Values are stored as fp16 ("Owned DFlash K/V state").

    Returns (K, V) as float64 arrays [L][n_kv][n][D] holding fp16 values for
    positions pos0 .. pos0+n-1."""
    g = g or GEOMETRY
    H, D, L, nkv = g["hidden"], g["head_dim"], g["n_layers"], g["n_kv_heads"]
    n = ctx_bits.shape[0]
    c = bf16_decode(ctx_bits)
    pos = pos0 + np.arange(n)
    K = np.empty((L, nkv, n, D))
    V = np.empty((L, nkv, n, D))
    for l in range(L):
        kk = matvec_rows(w, f"layers.{l}.wk", (nkv * D, H), c).reshape(n, nkv, D)
        vv = matvec_rows(w, f"layers.{l}.wv", (nkv * D, H), c).reshape(n, nkv, D)
        kk = rmsnorm(kk, gain(w, f"layers.{l}.k_norm"), g["rms_eps"])
        kk = rope_neox(kk.transpose(1, 0, 2), pos, g["rope_theta"])  # [nkv][n][D]
        K[l] = f16_round(kk)
        V[l] = f16_round(vv.transpose(1, 0, 2))
    return K, V


def draft_block(w: dict, ctx_k: np.ndarray, ctx_v: np.ndarray, p: int,
                anchor_id: int, mask_id: int, block: int,
                g: dict | None = None, row_tokens=None,
                row_positions=None, stages: dict | None = None) -> dict:
    """One parallel proposal pass over the block [anchor, mask x (block-1)].

    ctx_k / ctx_v: [L][n_kv][n][D] for the context positions visible from p,
    i.e. max(0, p - window) .. p - 1 in increasing order (n may be 0).

    Row i carries position p + i; row 0 is the anchor (the bonus token at p)
    and rows 1.. are the mask token ("Target feature taps").  Each layer
    follows the stage order of the "Parity validation" table: input norm,
    q/k/v projection, per-head q/k norm, NeoX RoPE, non-causal GQA attention
    over the context cells and every block row with scale 1/16, output
    projection plus residual, post-attention norm, SiLU-gated MLP plus
    residual.  The final norm and the shared LM head give one greedy
    candidate per mask row (row i proposes position p + i).

    Returns dict(cand [block-1] int, logits [block-1][V] float64, hidden
    [block][H] final-normed float64, margin [block-1] top1-top2 of the fp32
    logits, x_last [block][H] residual stream before the final norm).

    row_tokens / row_positions override the per-row token ids and positions;
    they exist only so tests can probe the structure of the pass (mask-row
    order, non-causality).  Block keys are always taken in position order.

    stages, if a dict, receives the intermediates of this same computation
    for stage-wise comparison ("Parity validation" table): "resid" the
    residual stream after the embedding and after every attention and MLP
    residual (2L + 1 arrays [B][H]); per layer, "qkv" the raw q | k | v
    projections before the q/k norms [B][(nq + 2 nkv) D], "attn" the
    attention output before the output projection [B][nq D] and "mlp"
    SiLU(gate) * up [B][F]."""
    g = g or GEOMETRY
    H, D, L = g["hidden"], g["head_dim"], g["n_layers"]
    nq, nkv, F, V = g["n_q_heads"], g["n_kv_heads"], g["ffn"], g["vocab"]
    eps, theta, scale = g["rms_eps"], g["rope_theta"], g["attn_scale"]
    grp = nq // nkv
    B = int(block)
    n = ctx_k.shape[2]
    assert n == min(p, g["window"]), "context must be the window before p"
    tokens = np.array([anchor_id] + [mask_id] * (B - 1))
    pos = p + np.arange(B)
    if row_tokens is not None:
        tokens = np.asarray(row_tokens)
    if row_positions is not None:
        pos = np.asarray(row_positions)
    order = np.argsort(pos, kind="stable")  # block keys in position order
    E = w["embed"].reshape(V, H)
    h = bf16_decode(E[tokens])
    rec = stages if stages is not None else {}
    rec.update(resid=[h], qkv=[], attn=[], mlp=[])
    for l in range(L):
        pre = f"layers.{l}."
        x = rmsnorm(h, gain(w, pre + "in_norm"), eps)
        q = matvec_rows(w, pre + "wq", (nq * D, H), x).reshape(B, nq, D)
        k = matvec_rows(w, pre + "wk", (nkv * D, H), x).reshape(B, nkv, D)
        v = matvec_rows(w, pre + "wv", (nkv * D, H), x).reshape(B, nkv, D)
        rec["qkv"].append(np.concatenate([q.reshape(B, -1), k.reshape(B, -1),
                                          v.reshape(B, -1)], axis=1))
        q = rmsnorm(q, gain(w, pre + "q_norm"), eps)
        k = rmsnorm(k, gain(w, pre + "k_norm"), eps)
        q = rope_neox(q.transpose(1, 0, 2), pos, theta)       # [nq][B][D]
        k = f16_round(rope_neox(k.transpose(1, 0, 2), pos, theta))  # [nkv][B][D]
        v = f16_round(v.transpose(1, 0, 2))
        o = np.empty((B, nq, D))
        for j in range(nkv):
            keys = np.concatenate([ctx_k[l, j], k[j][order]], axis=0)
            vals = np.concatenate([ctx_v[l, j], v[j][order]], axis=0)
            for hh in range(j * grp, (j + 1) * grp):
                o[:, hh, :] = attention(q[hh], keys, vals, scale)
        rec["attn"].append(o.reshape(B, nq * D))
        h = h + matvec_rows(w, pre + "wo", (H, nq * D), o.reshape(B, nq * D))
        rec["resid"].append(h)
        y = rmsnorm(h, gain(w, pre + "post_norm"), eps)
        gt = matvec_rows(w, pre + "wg", (F, H), y)
        up = matvec_rows(w, pre + "wu", (F, H), y)
        rec["mlp"].append(silu(gt) * up)
        h = h + matvec_rows(w, pre + "wd", (H, F), rec["mlp"][-1])
        rec["resid"].append(h)
    z = rmsnorm(h, gain(w, "final_norm"), eps)
    logits = matvec_rows(w, "lm_head", (V, H), z[1:], chunk=16384) if B > 1 \
        else np.zeros((0, V))
    cand, margin = [], []
    for r in range(B - 1):
        l32 = logits[r].astype(np.float32)
        c = argmax_lowest(l32)
        cand.append(c)
        top2 = np.partition(l32, -2)[-2:]
        margin.append(float(top2[1]) - float(top2[0]))
    conf = [candidate_confidence(logits[r]) for r in range(B - 1)]
    return dict(cand=np.array(cand, dtype=np.int64), logits=logits,
                hidden=z, margin=np.array(margin), x_last=h, conf=np.array(conf))


def candidate_confidence(logits_row) -> float:
    """Probability the drafter's own distribution gives its greedy candidate:
    the softmax of the row's logits over the whole vocabulary, evaluated at
    the argmax, p = exp(l_c) / sum_v exp(l_v).  (PR #3322 "support the
    official Flash-Next DFlash2 checkpoint", section "Long-prompt diagnosis
    and fix": proposals are gated by a probability floor, spec-min-p.  The
    pages do not print the formula; this is the plain reading: softmax of
    the drafter's logits, no temperature.)  exp is taken after subtracting
    the maximum, which changes nothing mathematically."""
    l = np.asarray(logits_row, dtype=np.float64)
    c = argmax_lowest(l.astype(np.float32))
    e = np.exp(l - l.max())
    return float(e[c] / e.sum())


def gate_candidates(conf, min_p: float) -> int:
    """Confidence gate (same section): the proposal keeps its candidates in
    order up to, not including, the first whose probability is below the
    floor; returns how many are kept.  A floor of 0 keeps all."""
    n = 0
    while n < len(conf) and conf[n] >= min_p:
        n += 1
    return n


def verify_greedy(cand, target):
    """Greedy verification ("Speculative decode integration"; RFC #366
    "Verification and state management"): accepted = length of the longest
    prefix of candidates equal to the target's greedy tokens at the same
    positions; the continuation token is the target's token right after that
    prefix (target has one more entry than cand)."""
    cand = list(int(c) for c in cand)
    target = list(int(t) for t in target)
    assert len(target) == len(cand) + 1
    a = 0
    while a < len(cand) and cand[a] == target[a]:
        a += 1
    return a, target[a]


# --------------------------------------------------------------------------
# Decode loop (propose -> verify -> commit), position-addressed context
# --------------------------------------------------------------------------

class ContextStore:
    """Drafter context K/V by absolute position (fp16 values as float64).
    Committing a position again overwrites its cell, so rejected proposals
    need no rollback ("Speculative decode integration").  Positions live in
    one contiguous range [base, base + size)."""

    def __init__(self, g: dict | None = None):
        self.g = g or GEOMETRY
        self.base = None
        self.k = None
        self.v = None
        self.written = None

    def _ensure(self, lo, hi):
        L, nkv, D = self.g["n_layers"], self.g["n_kv_heads"], self.g["head_dim"]
        if self.base is None:
            self.base = lo
            self.k = np.zeros((L, nkv, 0, D))
            self.v = np.zeros((L, nkv, 0, D))
            self.written = np.zeros(0, dtype=bool)
        assert lo >= self.base, "positions below the first committed one"
        need = hi - self.base
        if need > self.k.shape[2]:
            grow = max(need, 2 * self.k.shape[2])
            k = np.zeros((L, nkv, grow, D))
            v = np.zeros((L, nkv, grow, D))
            wr = np.zeros(grow, dtype=bool)
            n0 = self.k.shape[2]
            k[:, :, :n0] = self.k
            v[:, :, :n0] = self.v
            wr[:n0] = self.written
            self.k, self.v, self.written = k, v, wr

    def put(self, K, V, pos0):
        n = K.shape[2]
        self._ensure(pos0, pos0 + n)
        s = pos0 - self.base
        self.k[:, :, s:s + n] = K
        self.v[:, :, s:s + n] = V
        self.written[s:s + n] = True

    def window(self, p):
        """K, V [L][n_kv][n][D] of positions max(0, p - window) .. p - 1."""
        lo = max(0, p - self.g["window"])
        L, nkv, D = self.g["n_layers"], self.g["n_kv_heads"], self.g["head_dim"]
        if p - lo == 0:
            z = np.zeros((L, nkv, 0, D))
            return z, z.copy()
        s, e = lo - self.base, p - self.base
        assert s >= 0 and e <= self.k.shape[2] and self.written[s:e].all(), \
            "context window holds positions that were never committed"
        return self.k[:, :, s:e], self.v[:, :, s:e]


def commit(w: dict, store: ContextStore, taps_bits, pos0: int, g=None):
    """Fuse and project the target taps of newly committed positions."""
    ctx = fuse_context(w, taps_bits, g)
    K, V = project_ctx_kv(w, ctx, pos0, g)
    store.put(K, V, pos0)
    return ctx
