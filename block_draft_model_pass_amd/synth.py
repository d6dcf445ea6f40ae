"""Seeded synthetic inputs for the DFlash block-drafter proposal pass.

This module only *draws* data: weights, target feature taps, token ids and the
stand-in target model's greedy stream.  It holds none of the drafter's
arithmetic (no norms, projections, attention, argmax or verification) so that
the HIP library and the CPU oracle can both consume the very same bytes
without sharing any code of the method.

Shapes follow the DFlash drafter geometry described on the Strata PR #1426
page ("Drafter runtime": 5 dense layers, hidden 2560, GQA 24 Q / 2 KV heads of
256, MLP 7680; "Target feature taps": five 2560-wide taps).  Value
distributions: matrices, the embedding and the LM head ~ N(0, 0.02); norm
gains 1 + N(0, 0.02); taps ~ N(0, 1).  Every draw is fp32 from numpy's PCG64
and is rounded to bf16 with round-to-nearest-even.

Quantized backbones use a structure-of-arrays byte layout per matrix
``[N][K]``: ``N*K`` (Q8_0: int8) or ``N*K/2`` (Q4_0: packed nibbles) quant
bytes, followed by ``N*K/32`` little-endian fp16 block scales in row order.
Q4_0: within each 32-element block element ``j`` is the low nibble of byte
``j`` and element ``j+16`` the high nibble; the stored nibble is the value
plus 8.  Q5_0: the same nibbles and scales, then ``N*K/32`` little-endian
uint32 words, bit ``j`` of a block's word the fifth bit of element ``j``;
the stored 5-bit code is the value plus 16.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Fixed drafter geometry (Strata PR #1426, "Drafter runtime" and
# "Target feature taps").
HIDDEN = 2560
N_LAYERS = 5
N_Q_HEADS = 24
N_KV_HEADS = 2
HEAD_DIM = 256
FFN = 7680
VOCAB = 151936
N_TAPS = 5
ROPE_THETA = 1.0e7
ATTN_SCALE = 1.0 / 16.0
RMS_EPS = 1.0e-6
WINDOW = 32768
MAX_BLOCK = 8
MASK_ID = VOCAB - 1  # the pages name "the mask token" without an id

# Seeds of the four independent streams.
SEED_WEIGHTS = 0
SEED_TAPS = 1
SEED_TOKENS = 2
SEED_VERIFY = 3

LAYER_TENSORS = ("in_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo",
                 "post_norm", "wg", "wu", "wd")
MATRIX_KINDS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")

_CHUNK = 1 << 24  # elements per independently seeded chunk


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def weight_specs(geom: dict | None = None):
    """(name, shape, kind) for the 58 drafter tensors plus the target's
    embedding and LM head.  kind is 'matrix', 'gain' or 'table'."""
    g = dict(hidden=HIDDEN, n_layers=N_LAYERS, n_q_heads=N_Q_HEADS,
             n_kv_heads=N_KV_HEADS, head_dim=HEAD_DIM, ffn=FFN, vocab=VOCAB,
             n_taps=N_TAPS)
    if geom:
        g.update(geom)
    H, D, F = g["hidden"], g["head_dim"], g["ffn"]
    qd, kd = g["n_q_heads"] * D, g["n_kv_heads"] * D
    specs = [("fc", (H, g["n_taps"] * H), "matrix"),
             ("hidden_norm", (H,), "gain")]
    shapes = {"in_norm": (H,), "wq": (qd, H), "wk": (kd, H), "wv": (kd, H),
              "q_norm": (D,), "k_norm": (D,), "wo": (H, qd),
              "post_norm": (H,), "wg": (F, H), "wu": (F, H), "wd": (H, F)}
    for layer in range(g["n_layers"]):
        for t in LAYER_TENSORS:
            kind = "matrix" if t in MATRIX_KINDS else "gain"
            specs.append((f"layers.{layer}.{t}", shapes[t], kind))
    specs.append(("final_norm", (H,), "gain"))
    specs.append(("embed", (g["vocab"], H), "table"))
    specs.append(("lm_head", (g["vocab"], H), "table"))
    return specs


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 samples to bf16 (nearest, ties to even); returns the
    16-bit patterns as uint16."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
            >> np.uint32(16)).astype(np.uint16)


def _normal_f32(seed_words, n: int, std: float, mean: float,
                bf16: bool = False) -> np.ndarray:
    """n fp32 samples of N(mean, std^2) (or their bf16 bit patterns), drawn in
    fixed-size chunks that each have their own seed so the result does not
    depend on threading."""
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    starts = list(range(0, n, _CHUNK))

    def work(ci):
        s = starts[ci]
        e = min(n, s + _CHUNK)
        rng = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence(list(seed_words) + [ci])))
        v = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        if mean != 0.0:
            v += np.float32(mean)
        out[s:e] = bf16_bits_from_f32(v) if bf16 else v

    if len(starts) == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(len(starts))))
    return out


def _bf16_normal(seed_words, shape, std, mean=0.0) -> np.ndarray:
    n = int(np.prod(shape))
    return _normal_f32(seed_words, n, std, mean, bf16=True).reshape(shape)


def quantize_q8_0(w: np.ndarray) -> np.ndarray:
    """Q8_0 bytes for an fp32 matrix [N][K]: per 32-element block the scale is
    amax/127 stored as fp16, values round(w/scale) clipped to [-127, 127]."""
    N, K = w.shape
    assert K % 32 == 0
    blk = w.reshape(N, K // 32, 32).astype(np.float32)
    amax = np.abs(blk).max(axis=2)
    d16 = (amax / np.float32(127.0)).astype(np.float16)
    d32 = d16.astype(np.float32)
    inv = np.where(d32 > 0, np.float32(1.0) / np.where(d32 > 0, d32, 1), 0)
    q = np.clip(np.rint(blk * inv[:, :, None]), -127, 127).astype(np.int8)
    return np.concatenate([q.reshape(-1).view(np.uint8),
                           d16.reshape(-1).view(np.uint8)])


def quantize_q4_0(w: np.ndarray) -> np.ndarray:
    """Q4_0 bytes for an fp32 matrix [N][K]: per block the element of largest
    magnitude maps to -8; scale = that element / -8 stored as fp16; nibble =
    clip(round(w/scale) + 8, 0, 15)."""
    N, K = w.shape
    assert K % 32 == 0
    blk = w.reshape(N, K // 32, 32).astype(np.float32)
    idx = np.abs(blk).argmax(axis=2)
    vmax = np.take_along_axis(blk, idx[:, :, None], axis=2)[:, :, 0]
    d16 = (vmax / np.float32(-8.0)).astype(np.float16)
    d32 = d16.astype(np.float32)
    inv = np.where(d32 != 0, np.float32(1.0) / np.where(d32 != 0, d32, 1), 0)
    nib = np.clip(np.rint(blk * inv[:, :, None]) + 8, 0, 15).astype(np.uint8)
    packed = (nib[:, :, :16] | (nib[:, :, 16:] << 4)).astype(np.uint8)
    return np.concatenate([packed.reshape(-1), d16.reshape(-1).view(np.uint8)])


def quantize_q5_0(w: np.ndarray) -> np.ndarray:
    """Q5_0 bytes for an fp32 matrix [N][K]: per block the element of largest
    magnitude maps to -16; scale = that element / -16 stored as fp16; code =
    clip(round(w/scale) + 16, 0, 31), its low nibble packed as in Q4_0 and
    its fifth bit in the block's high-bit word."""
    N, K = w.shape
    assert K % 32 == 0
    blk = w.reshape(N, K // 32, 32).astype(np.float32)
    idx = np.abs(blk).argmax(axis=2)
    vmax = np.take_along_axis(blk, idx[:, :, None], axis=2)[:, :, 0]
    d16 = (vmax / np.float32(-16.0)).astype(np.float16)
    d32 = d16.astype(np.float32)
    inv = np.where(d32 != 0, np.float32(1.0) / np.where(d32 != 0, d32, 1), 0)
    code = np.clip(np.rint(blk * inv[:, :, None]) + 16, 0, 31).astype(np.uint32)
    nib = (code & 15).astype(np.uint8)
    packed = (nib[:, :, :16] | (nib[:, :, 16:] << 4)).astype(np.uint8)
    hw = ((code >> 4) << np.arange(32, dtype=np.uint32)).sum(axis=2, dtype=np.uint32)
    return np.concatenate([packed.reshape(-1), d16.reshape(-1).view(np.uint8),
                           hw.astype("<u4").reshape(-1).view(np.uint8)])


def make_weights(seed: int = SEED_WEIGHTS, fmt: str = "bf16",
                 geom: dict | None = None, lm_fmt: str = "bf16") -> dict:
    """All drafter tensors, the embedding and the LM head, keyed by name.

    bf16 tensors are uint16 bit patterns of their shape.  With fmt 'q8_0',
    'q4_0' or 'q5_0' the 36 backbone matrices (fc and the 35 layer matrices) are flat
    uint8 buffers in the layout described in the module docstring; gains and
    the embedding stay bf16.  lm_fmt 'q8_0' stores the LM head as Q8_0 blocks
    (same draws, quantized) in the same layout."""
    assert fmt in ("bf16", "q8_0", "q4_0", "q5_0") and lm_fmt in ("bf16", "q8_0")
    out = {}
    for ti, (name, shape, kind) in enumerate(weight_specs(geom)):
        words = (seed, ti)
        qfmt = lm_fmt if name == "lm_head" else (fmt if kind == "matrix" else "bf16")
        if kind == "gain":
            out[name] = _bf16_normal(words, shape, 0.02, 1.0)
        elif qfmt == "bf16":
            out[name] = _bf16_normal(words, shape, 0.02)
        else:
            v = _normal_f32(words, int(np.prod(shape)), 0.02, 0.0)
            v = v.reshape(shape)
            out[name] = {"q8_0": quantize_q8_0, "q4_0": quantize_q4_0,
                         "q5_0": quantize_q5_0}[qfmt](v)
    out["__format__"] = fmt
    out["__lm_format__"] = lm_fmt
    return out


def make_taps(positions, seed: int = SEED_TAPS,
              n_taps: int = N_TAPS, hidden: int = HIDDEN) -> np.ndarray:
    """Target feature taps for the given absolute positions: uint16 bf16 bits
    [n][n_taps][hidden], N(0,1), one independent stream per position so that
    a position's taps are the same whenever they are drawn."""
    positions = [int(m) for m in positions]
    out = np.empty((len(positions), n_taps, hidden), dtype=np.uint16)

    def work(rng_slice):
        for i in rng_slice:
            g = np.random.Generator(np.random.PCG64(
                np.random.SeedSequence([seed, positions[i]])))
            v = g.standard_normal(n_taps * hidden, dtype=np.float32)
            out[i] = bf16_bits_from_f32(v).reshape(n_taps, hidden)

    n = len(positions)
    nt = _threads() if n >= 256 else 1
    parts = [range(s, n, nt) for s in range(nt)]
    if nt == 1:
        work(range(n))
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(work, parts))
    return out


def anchor_token(index: int = 0, seed: int = SEED_TOKENS,
                 vocab: int = VOCAB) -> int:
    """A seeded token id for the anchor row of a standalone draft pass."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, index])))
    return int(g.integers(0, vocab - 1))  # never the mask id


def random_targets(k: int, index: int = 0, seed: int = SEED_TOKENS,
                   vocab: int = VOCAB) -> np.ndarray:
    """k+1 seeded target ids (independent of any proposal)."""
    g = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed, 1 << 20, index])))
    return g.integers(0, vocab, size=k + 1).astype(np.int32)


def target_draws(pass_index: int, k: int, seed: int = SEED_VERIFY,
                 p_match: float = 0.75, vocab: int = VOCAB):
    """Per-pass draws of the stand-in target model: (match[k] bool,
    offset[k] in [0, vocab-2], tail id)."""
    g = np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed, pass_index])))
    match = g.random(k) < p_match
    offset = g.integers(0, vocab - 1, size=k)
    tail = int(g.integers(0, vocab))
    return match, offset, tail


def synthetic_target(cand: np.ndarray, pass_index: int,
                     seed: int = SEED_VERIFY, p_match: float = 0.75,
                     vocab: int = VOCAB) -> np.ndarray:
    """Stand-in for the target model's greedy tokens over a verify window:
    entry i agrees with candidate i with probability p_match, otherwise it is
    a different id; the last entry (after the final candidate) is uniform."""
    cand = np.asarray(cand, dtype=np.int64)
    k = cand.shape[0]
    match, offset, tail = target_draws(pass_index, k, seed, p_match, vocab)
    tgt = np.where(match, cand, (cand + 1 + offset) % vocab)
    return np.concatenate([tgt, [tail]]).astype(np.int32)


def make_rows(n: int, width: int, seed: int, dtype: str = "bf16",
              std: float = 1.0) -> np.ndarray:
    """n seeded rows of N(0, std^2): bf16 bits (uint16) or fp16 bits (uint16)."""
    v = _normal_f32((seed, 1 << 24, width), n * width, std, 0.0)
    if dtype == "bf16":
        return bf16_bits_from_f32(v).reshape(n, width)
    return v.astype(np.float16).view(np.uint16).reshape(n, width)
