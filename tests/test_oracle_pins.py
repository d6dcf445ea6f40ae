"""Pins for the CPU oracle: each check compares the oracle with something
other than itself -- values the pages print, closed forms, special cases that
reduce to a textbook formula or library routine, or brute force on tiny
inputs.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

from oracle import dflash_oracle as O
from block_draft_model_pass_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def page():
    with open(GOLDEN) as f:
        return json.load(f)


def b16(x):
    """Encode exactly representable test values as bf16 bits."""
    bits = synth.bf16_bits_from_f32(np.asarray(x, dtype=np.float32))
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, np.asarray(x, dtype=np.float32)), "not exact in bf16"
    return bits


# ---------------------------------------------------------------- constants

def test_geometry_matches_page_values():
    pg = page()["geometry"]
    g = O.GEOMETRY
    for key in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim",
                "ffn", "rope_theta", "attn_scale"):
        assert g[key] == pg[key], key
    assert g["window"] == page()["limits"]["window_cells"]
    assert synth.MAX_BLOCK - 1 == page()["limits"]["max_candidates"]


def test_attention_scale_is_inverse_sqrt_head_dim():
    s = O.GEOMETRY["attn_scale"]
    assert s == 1.0 / math.sqrt(O.GEOMETRY["head_dim"])
    assert s * s * 256 == 1.0


def test_weight_inventory_matches_artifact_counts():
    """58 drafter tensors and ~498M parameters (embedding and LM head come
    from the target and are not part of the artifact)."""
    specs = [s for s in synth.weight_specs() if s[2] != "table"]
    art = page()["artifact"]
    assert len(specs) == art["n_tensors"]
    params = sum(int(np.prod(s[1])) for s in specs)
    assert params == 498_106_880
    assert round(params / 1e6) == art["params_millions"]
    assert sum(1 for s in specs if s[2] == "matrix") == 36


# ---------------------------------------------------------------- formats

def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x3E80, 0x4049, 0x7F80, 0x0001],
                    dtype=np.uint16)
    want = [1.0, -2.0, 0.0, 0.25, 3.140625, np.inf, 2.0 ** -133]
    assert list(O.bf16_decode(bits)) == want


def test_bf16_round_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                  -3.140625, 65280.0])
    assert [int(v) for v in O.bf16_round(x)] == [0x3F80, 0x3F80, 0x3F82, 0x3F81,
                                                 0xC049, 0x477F]


def test_f16_round_known_values():
    assert O.f16_round(np.array([1.0 / 3.0]))[0] == 0.333251953125  # 0x3555
    assert O.f16_round(np.array([65519.0]))[0] == 65504.0
    assert O.f16_round(np.array([1.0 + 2 ** -11]))[0] == 1.0  # tie to even


def test_q8_0_dequant_hand_block():
    q = np.array(list(range(-127, -127 + 32)), dtype=np.int8)
    q[5] = 0
    q[6] = 127
    d = np.array([0.5], dtype=np.float16)   # exact fp16 0x3800
    raw = np.concatenate([q.view(np.uint8), d.view(np.uint8)])
    got = O.dequant_q8_0(raw, 1, 32)[0]
    want = [0.5 * int(v) for v in q]
    assert list(got) == want


def test_q4_0_dequant_hand_block():
    lo = np.arange(16, dtype=np.uint8)          # elements 0..15
    hi = (15 - np.arange(16)).astype(np.uint8)  # elements 16..31
    raw_q = (lo | (hi << 4)).astype(np.uint8)
    d = np.array([-0.25], dtype=np.float16)
    raw = np.concatenate([raw_q, d.view(np.uint8)])
    got = O.dequant_q4_0(raw, 1, 32)[0]
    want = [-0.25 * (j - 8) for j in range(16)] + [-0.25 * (7 - j) for j in range(16)]
    assert list(got) == want


def test_q5_0_dequant_hand_block():
    """Codes c_j = (7 j + 3) mod 32 (all 32 values once): low nibble of
    element j in byte j % 16 (high half for j >= 16), fifth bit in bit j of
    the word; value d * (c_j - 16)."""
    code = [(7 * j + 3) % 32 for j in range(32)]
    assert sorted(code) == list(range(32))
    raw_q = bytes((code[j] & 15) | ((code[j + 16] & 15) << 4) for j in range(16))
    word = sum((c >> 4) << j for j, c in enumerate(code))
    d = np.array([0.375], dtype=np.float16)
    raw = np.frombuffer(raw_q + d.tobytes() + int(word).to_bytes(4, "little"), dtype=np.uint8)
    got = O.dequant_q5_0(raw.copy(), 1, 32)[0]
    assert list(got) == [0.375 * (c - 16) for c in code]


def test_q5_0_is_q4_0_shifted_by_its_fifth_bit():
    """Same nibbles and scales: with every fifth bit clear a Q5_0 value is the
    Q4_0 value minus 8 d, with every bit set plus 8 d (two rows, two blocks
    each, mixed bits checked element by element)."""
    rng = np.random.default_rng(3)
    rows, cols = 2, 64
    q = rng.integers(0, 256, rows * cols // 2, dtype=np.uint8)
    d = rng.standard_normal(rows * cols // 32).astype(np.float16)
    q4 = O.dequant_q4_0(np.concatenate([q, d.view(np.uint8)]), rows, cols)
    dd = np.repeat(d.astype(np.float64).reshape(rows, cols // 32), 32, axis=1)
    for words, shift in ((np.zeros(4, np.uint32), -8), (np.full(4, 0xFFFFFFFF, np.uint32), 8)):
        raw = np.concatenate([q, d.view(np.uint8), words.astype("<u4").view(np.uint8)])
        assert np.array_equal(O.dequant_q5_0(raw, rows, cols), q4 + shift * dd)
    words = rng.integers(0, 2 ** 32, 4, dtype=np.uint64).astype(np.uint32)
    raw = np.concatenate([q, d.view(np.uint8), words.astype("<u4").view(np.uint8)])
    got = O.dequant_q5_0(raw, rows, cols)
    for r in range(rows):
        for k in range(cols):
            bit = (int(words[r * 2 + k // 32]) >> (k % 32)) & 1
            assert got[r, k] == q4[r, k] + (8 if bit else -8) * dd[r, k]


def test_quant_round_trip_within_half_step():
    """The harness quantizers and the oracle's decoders agree: every decoded
    weight is within half a quantisation step of the fp32 source."""
    rng = np.random.default_rng(5)
    w = rng.standard_normal((4, 64)).astype(np.float32) * 0.02
    d8 = O.dequant_q8_0(synth.quantize_q8_0(w), 4, 64)
    step8 = np.abs(w.reshape(4, 2, 32)).max(axis=2) / 127
    assert np.all(np.abs(d8 - w).reshape(4, 2, 32) <= step8[..., None] * 0.5 + 1e-4)
    # Q4_0 codes span -8..7 steps, so a value opposite in sign to the block's
    # largest-magnitude element may clip by up to one step.
    d4 = O.dequant_q4_0(synth.quantize_q4_0(w), 4, 64)
    step4 = np.abs(w.reshape(4, 2, 32)).max(axis=2) / 8
    err4 = np.abs(d4 - w).reshape(4, 2, 32)
    assert np.all(err4 <= step4[..., None] * 1.0 + 1e-4)
    assert np.mean(err4 <= step4[..., None] * 0.5 + 1e-4) > 0.9
    # Q5_0 codes span -16..15 steps of amax/16: the same one-step clip bound.
    d5 = O.dequant_q5_0(synth.quantize_q5_0(w), 4, 64)
    step5 = np.abs(w.reshape(4, 2, 32)).max(axis=2) / 16
    err5 = np.abs(d5 - w).reshape(4, 2, 32)
    assert np.all(err5 <= step5[..., None] * 1.0 + 1e-4)
    assert np.mean(err5 <= step5[..., None] * 0.5 + 1e-4) > 0.9


# ---------------------------------------------------------------- rmsnorm

def test_rmsnorm_closed_forms():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 64))
    eps = 1e-6
    y = O.rmsnorm(x, np.ones(64), eps)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-12)
    c = 0.75
    yc = O.rmsnorm(np.full((1, 64), c), np.ones(64), eps)
    assert np.allclose(yc, c / math.sqrt(c * c + eps), rtol=1e-14)
    g = rng.standard_normal(64)
    assert np.allclose(O.rmsnorm(x, g, eps), y * g, rtol=1e-14)


# ---------------------------------------------------------------- RoPE

def test_rope_inv_freq_closed_form():
    f = O.rope_inv_freq(256, 1e7)
    assert f[0] == 1.0
    assert math.isclose(f[64], 1.0 / math.sqrt(1e7), rel_tol=1e-14)
    assert math.isclose(f[127], 1e7 ** (-254 / 256), rel_tol=1e-14)


def test_rope_identity_at_zero_and_norm_preserving():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 256))
    assert np.array_equal(O.rope_neox(x, np.zeros(4), 1e7), x)
    for m in (1, 8191, 229376, 262151):
        y = O.rope_neox(x, np.full(4, m), 1e7)
        assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1),
                           rtol=1e-12)


def test_rope_half_split_pairing_and_sign():
    """A unit vector on element 0 turns into element 128 at frequency 1:
    (cos m, sin m) -- pins the (i, i+128) pairing and the rotation sign."""
    x = np.zeros((1, 256))
    x[0, 0] = 1.0
    m = 3
    y = O.rope_neox(x, np.array([m]), 1e7)[0]
    assert math.isclose(y[0], math.cos(m), abs_tol=1e-15)
    assert math.isclose(y[128], math.sin(m), abs_tol=1e-15)
    assert np.count_nonzero(np.abs(y) > 1e-15) == 2


def test_rope_equals_complex_rotation():
    """NeoX RoPE is z_i * exp(1j * m * f_i) with z_i = x_i + 1j * x_{i+128}."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 256))
    pos = np.array([0, 17, 262151])
    z = x[:, :128] + 1j * x[:, 128:]
    f = 1e7 ** (-np.arange(128) * 2.0 / 256)
    zr = z * np.exp(1j * pos[:, None] * f[None, :])
    want = np.concatenate([zr.real, zr.imag], axis=1)
    assert np.allclose(O.rope_neox(x, pos, 1e7), want, rtol=1e-9, atol=1e-9)


def test_rope_relative_position_property():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 256))
    k = rng.standard_normal((1, 256))
    for m, n, d in ((5, 3, 1000), (8191, 0, 254000), (100, 262000, -99)):
        a = O.rope_neox(q, np.array([m]), 1e7) @ O.rope_neox(k, np.array([n]), 1e7).T
        b = O.rope_neox(q, np.array([m + d]), 1e7) @ O.rope_neox(k, np.array([n + d]), 1e7).T
        assert math.isclose(a[0, 0], b[0, 0], rel_tol=1e-5, abs_tol=1e-9)


# ---------------------------------------------------------------- attention

def test_attention_single_key_returns_its_value():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((5, 8))
    k = rng.standard_normal((1, 8))
    v = rng.standard_normal((1, 8))
    assert np.array_equal(O.attention(q, k, v, 1 / 16), np.repeat(v, 5, axis=0))


def test_attention_uniform_keys_give_mean_value():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 8))
    k = np.repeat(rng.standard_normal((1, 8)), 7, axis=0)
    v = rng.standard_normal((7, 8))
    assert np.allclose(O.attention(q, k, v, 1 / 16), v.mean(axis=0), rtol=1e-13)


def test_attention_two_keys_logistic_weight():
    """Two keys: the weight of key 1 is the logistic of scale*(q.k1 - q.k2)."""
    q = np.array([[2.0, -1.0, 0.5, 0.0]])
    k = np.array([[1.0, 3.0, -2.0, 0.5], [0.5, 0.0, 1.0, -1.0]])
    v = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0]])
    o = O.attention(q, k, v, 1 / 16)[0]
    w1 = float(expit((q[0] @ k[0] - q[0] @ k[1]) / 16))
    assert math.isclose(o[0], w1, rel_tol=1e-14)
    assert math.isclose(o[1], 1 - w1, rel_tol=1e-14)


def test_argmax_lowest_index_on_ties():
    x = np.array([0.0, 3.0, -1.0, 3.0, 3.0], dtype=np.float32)
    assert O.argmax_lowest(x) == 1
    assert O.argmax_lowest(np.array([-np.inf, -5.0, -5.0])) == 1
    assert O.argmax_lowest(np.array([7.0])) == 0


# ---------------------------------------------------------------- verify

def test_verify_page_three_cases():
    for case in page()["verifier_cases"]["cases"]:
        a, nxt = O.verify_greedy(case["cand"], case["target"])
        assert (a, nxt) == (case["accepted"], case["next"]), case["name"]


def test_verify_matches_brute_force_exhaustive():
    V = 3
    for k in range(0, 5):
        for cand in itertools.product(range(V), repeat=k):
            for tgt in itertools.product(range(V), repeat=k + 1):
                best = max(j for j in range(k + 1) if cand[:j] == tgt[:j])
                assert O.verify_greedy(cand, tgt) == (best, tgt[best])


def test_synthetic_target_accepts_leading_matches():
    """With the stand-in target, the accepted length is the run of leading
    'match' draws, whatever the candidates are."""
    rng = np.random.default_rng(6)
    for t in range(200):
        cand = rng.integers(0, synth.VOCAB, size=7)
        tgt = synth.synthetic_target(cand, t)
        match, _, _ = synth.target_draws(t, 7)
        run = 0
        while run < 7 and match[run]:
            run += 1
        assert O.verify_greedy(cand, tgt)[0] == run
        assert np.all((tgt[:7] == cand) == match)


def test_synthetic_acceptance_rate_closed_form():
    """E[accepted]/K = sum_{i=1..K} 0.75^i / K for K = 7."""
    total = 0
    n = 20000
    for t in range(n):
        match, _, _ = synth.target_draws(t, 7)
        run = 0
        while run < 7 and match[run]:
            run += 1
        total += run
    expect = sum(0.75 ** i for i in range(1, 8)) / 7
    assert abs(total / (7 * n) - expect) < 0.01


# ---------------------------------------------------------------- tiny model
# Structural pins run the oracle at a tiny geometry with hand-built weights.

TINY = O.geometry(hidden=8, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=4,
                  ffn=6, vocab=11, n_taps=5, window=4)


def tiny_weights(fill=None, seed=0):
    """bf16 weights for TINY: random small values unless given in fill."""
    rng = np.random.default_rng(seed)
    w = {"__format__": "bf16"}
    for name, shape, kind in synth.weight_specs(TINY):
        if fill and name in fill:
            w[name] = b16(np.asarray(fill[name], dtype=np.float32).reshape(shape))
        elif kind == "gain":
            w[name] = b16(np.ones(shape, dtype=np.float32))
        else:
            v = rng.integers(-8, 9, size=shape).astype(np.float32) / 16
            w[name] = b16(v)
    return w


def test_fusion_concat_order_and_norm():
    """fc with W[i][H + i] = 1 and W[i][3H + i] = 0.5 makes the fused context
    rmsnorm(tap_1 + tap_3 / 2): pins concat order, fc orientation, norm."""
    H, T = 8, 5
    fc = np.zeros((H, T * H), dtype=np.float32)
    for i in range(H):
        fc[i, 1 * H + i] = 1.0
        fc[i, 3 * H + i] = 0.5
    w = tiny_weights({"fc": fc})
    rng = np.random.default_rng(7)
    taps = rng.integers(-16, 17, size=(3, T, H)).astype(np.float32) / 8
    ctx = O.fuse_context(w, b16(taps), TINY)
    t2 = taps[:, 1, :].astype(np.float64) + 0.5 * taps[:, 3, :]
    want = t2 / np.sqrt((t2 ** 2).mean(axis=1, keepdims=True) + 1e-6)
    assert np.allclose(O.bf16_decode(ctx), want, rtol=2 ** -8)


def test_project_kv_closed_form():
    """ctx = (a, 0, ..., 0) and Wk picking element 0 into each head's first
    slot: the normed key is (2, 0, 0, 0) (D = 4, mean of squares a^2/4) and
    RoPE at position m turns it into (2 cos m, 0, 2 sin m, 0).  Wv = I."""
    D, H = 4, 8
    wk = np.zeros((2 * D, H), dtype=np.float32)
    wk[0, 0] = 1.0
    wk[D, 0] = -1.0
    wv = np.eye(2 * D, H, dtype=np.float32)
    w = tiny_weights({"layers.0.wk": wk, "layers.1.wk": wk,
                      "layers.0.wv": wv, "layers.1.wv": wv})
    ctx = np.zeros((2, H), dtype=np.float32)
    ctx[:, 0] = [3.0, 0.5]
    ctx[1, 5] = 0.25
    K, V = O.project_ctx_kv(w, b16(ctx), pos0=40, g=TINY)
    for t, m in enumerate((40, 41)):
        a = ctx[t, 0]
        r = a / math.sqrt(a * a / 4 + 1e-6)
        want0 = [r * math.cos(m), 0.0, r * math.sin(m), 0.0]
        assert np.allclose(K[0, 0, t], want0, rtol=2 ** -10, atol=1e-3)
        assert np.allclose(K[1, 1, t], [-x for x in want0], rtol=2 ** -10, atol=1e-3)
        assert np.allclose(V[0, 0, t], ctx[t, :4])
        assert np.allclose(V[1, 1, t], ctx[t, 4:])


def _const_embed(vals, H=8, V=11):
    e = np.zeros((V, H), dtype=np.float32)
    for tok, c in vals.items():
        e[tok] = c
    return e


def test_pass_with_zero_branches_reduces_to_lm_head():
    """Wo = Wd = 0 leaves the residual stream at the embedding, so hidden =
    final-norm of E[token] and the candidate of mask row i is the LM-head row
    best aligned with the mask embedding.  Pins: anchor row 0 vs mask rows,
    candidates from mask rows only, final norm, LM-head orientation."""
    H, V = 8, 11
    E = _const_embed({3: 0.5, 10: -0.25})
    lm = np.zeros((V, H), dtype=np.float32)
    lm[6] = -1.0          # best for a negative (mask) hidden state
    lm[2] = 1.0           # best for a positive (anchor) hidden state
    lm[7, 0] = -0.5
    fill = {"embed": E, "lm_head": lm}
    for l in range(2):
        fill[f"layers.{l}.wo"] = np.zeros((H, 16))
        fill[f"layers.{l}.wd"] = np.zeros((H, 6))
    w = tiny_weights(fill)
    z = np.zeros((2, 2, 0, 4))
    r = O.draft_block(w, z, z, p=0, anchor_id=3, mask_id=10, block=3, g=TINY)
    sa = 0.5 / math.sqrt(0.25 + 1e-6)
    sm = 0.25 / math.sqrt(0.0625 + 1e-6)
    assert np.allclose(r["hidden"][0], sa, rtol=1e-12)
    assert np.allclose(r["hidden"][1:], -sm, rtol=1e-12)
    assert list(r["cand"]) == [6, 6]
    assert np.allclose(r["logits"][:, 6], 8 * sm, rtol=1e-12)
    assert np.allclose(r["logits"][:, 7], 0.5 * sm, rtol=1e-12)
    assert np.allclose(r["logits"][:, 2], -8 * sm, rtol=1e-12)


def test_pass_uniform_attention_over_window_and_block():
    """Wq = Wk = 0 makes every score 0, so each head's output is the plain
    mean of the values of its KV group over the context window and all block
    rows.  Wo copies head 0 (group 0) into h[0:4] and head 3 (group 1) into
    h[4:8]; Wd = 0.  Pins the key set, the GQA head->group map, the window
    and the residual add."""
    H, D = 8, 4
    E = _const_embed({1: 1.0, 10: 2.0})
    wv = np.zeros((2 * D, H), dtype=np.float32)
    wv[:, 0] = [1, 2, 3, 4, -1, -2, -3, -4]      # x is all-ones after the norm
    wo = np.zeros((H, 16), dtype=np.float32)
    for i in range(4):
        wo[i, 0 * D + i] = 1.0        # head 0 -> h[0:4]
        wo[4 + i, 3 * D + i] = 1.0    # head 3 -> h[4:8]
    fill = {"embed": E, "layers.0.wv": wv, "layers.0.wo": wo,
            "layers.0.wq": np.zeros((16, H)), "layers.0.wk": np.zeros((8, H)),
            "layers.0.wd": np.zeros((H, 6)), "layers.1.wo": np.zeros((H, 16)),
            "layers.1.wd": np.zeros((H, 6))}
    w = tiny_weights(fill)
    rng = np.random.default_rng(8)
    p = 6                                    # window 4 -> context positions 2..5
    store = O.ContextStore(TINY)
    Kc = rng.standard_normal((2, 2, p, D))
    Vc = O.f16_round(rng.standard_normal((2, 2, p, D)))
    store.put(Kc, Vc, 0)
    ck, cv = store.window(p)
    assert ck.shape[2] == 4 and np.array_equal(cv, Vc[:, :, 2:6])
    r = O.draft_block(w, ck, cv, p=p, anchor_id=1, mask_id=10, block=3, g=TINY)
    v_blk = np.array([1, 2, 3, 4, -1, -2, -3, -4], dtype=np.float64)
    vg0 = np.concatenate([Vc[0, 0, 2:6], np.repeat(v_blk[None, :4], 3, 0)]).mean(0)
    vg1 = np.concatenate([Vc[0, 1, 2:6], np.repeat(v_blk[None, 4:], 3, 0)]).mean(0)
    for row, e in ((0, 1.0), (1, 2.0), (2, 2.0)):
        want = np.concatenate([e + vg0, e + vg1])
        assert np.allclose(r["x_last"][row], want, rtol=1e-3, atol=1e-3), row


def test_pass_stage_record_in_the_uniform_attention_case():
    """The stages the pass records (for stage-wise comparison) in the
    uniform-attention case above: the raw v projection is the Wv column, the
    attention output of head 0 / head 3 is the mean of its group's values,
    the residual after layer 0's attention is the embedding plus those means,
    Wd = 0 leaves the MLP residual unchanged, and the last record is the
    stream the final norm reads."""
    H, D = 8, 4
    E = _const_embed({1: 1.0, 10: 2.0})
    wv = np.zeros((2 * D, H), dtype=np.float32)
    wv[:, 0] = [1, 2, 3, 4, -1, -2, -3, -4]
    wo = np.zeros((H, 16), dtype=np.float32)
    for i in range(4):
        wo[i, 0 * D + i] = 1.0
        wo[4 + i, 3 * D + i] = 1.0
    fill = {"embed": E, "layers.0.wv": wv, "layers.0.wo": wo,
            "layers.0.wq": np.zeros((16, H)), "layers.0.wk": np.zeros((8, H)),
            "layers.0.wd": np.zeros((H, 6)), "layers.1.wo": np.zeros((H, 16)),
            "layers.1.wd": np.zeros((H, 6))}
    w = tiny_weights(fill)
    rng = np.random.default_rng(8)
    p = 6
    store = O.ContextStore(TINY)
    store.put(rng.standard_normal((2, 2, p, D)), O.f16_round(rng.standard_normal((2, 2, p, D))), 0)
    ck, cv = store.window(p)
    rec = {}
    r = O.draft_block(w, ck, cv, p=p, anchor_id=1, mask_id=10, block=3, g=TINY, stages=rec)
    assert len(rec["resid"]) == 5 and len(rec["qkv"]) == len(rec["attn"]) == len(rec["mlp"]) == 2
    assert [a.shape for a in rec["qkv"]] == [(3, 16 + 8 + 8)] * 2
    v_blk = np.array([1, 2, 3, 4, -1, -2, -3, -4], dtype=np.float64)
    assert np.allclose(rec["qkv"][0][:, 24:], v_blk, rtol=1e-3)
    assert np.allclose(rec["qkv"][0][:, :24], 0.0)
    vg0 = np.concatenate([cv[0, 0], np.repeat(v_blk[None, :4], 3, 0)]).mean(0)
    vg1 = np.concatenate([cv[0, 1], np.repeat(v_blk[None, 4:], 3, 0)]).mean(0)
    for row, e in ((0, 1.0), (1, 2.0), (2, 2.0)):
        assert np.allclose(rec["attn"][0][row, 0:4], vg0, rtol=1e-3, atol=1e-3)
        assert np.allclose(rec["attn"][0][row, 12:16], vg1, rtol=1e-3, atol=1e-3)
        assert np.allclose(rec["resid"][0][row], e)
        assert np.allclose(rec["resid"][1][row], np.concatenate([e + vg0, e + vg1]),
                           rtol=1e-3, atol=1e-3)
    assert np.array_equal(rec["resid"][2], rec["resid"][1])      # Wd = 0
    assert np.array_equal(rec["resid"][4], r["x_last"])


def test_pass_mlp_special_case():
    """Attention contributes nothing (Wv = Wo = 0); Wg picks y_0 * a, Wu
    picks y_0 * b, Wd sends unit j to h_j: h_j += silu(a y_0) * b y_0 for
    j < ffn, with silu(z) = z * logistic(z)."""
    H, F = 8, 6
    E = _const_embed({4: 0.5, 10: 0.5})
    a, b = 1.5, -0.75
    wg = np.zeros((F, H), dtype=np.float32)
    wu = np.zeros((F, H), dtype=np.float32)
    wg[:, 0] = a
    wu[:, 0] = b
    wd = np.zeros((H, F), dtype=np.float32)
    for j in range(F):
        wd[j, j] = 1.0
    fill = {"embed": E, "layers.0.wv": np.zeros((8, H)),
            "layers.0.wo": np.zeros((H, 16)), "layers.0.wg": wg,
            "layers.0.wu": wu, "layers.0.wd": wd,
            "layers.1.wo": np.zeros((H, 16)), "layers.1.wd": np.zeros((H, F))}
    w = tiny_weights(fill)
    z = np.zeros((2, 2, 0, 4))
    r = O.draft_block(w, z, z, p=0, anchor_id=4, mask_id=10, block=2, g=TINY)
    y0 = 0.5 / math.sqrt(0.25 + 1e-6)
    add = a * y0 * expit(a * y0) * b * y0
    want = np.array([0.5 + add] * F + [0.5, 0.5])
    assert np.allclose(r["x_last"][0], want, rtol=1e-12)


def test_pass_anchor_only_attends_to_itself():
    """No context and block 1: the anchor's single key is its own, so every
    head's attention output is its group's v (single-cell special case)."""
    H, D = 8, 4
    E = _const_embed({5: 1.0})
    wv = np.zeros((2 * D, H), dtype=np.float32)
    wv[:, 0] = [0.5, -1, 2, 0.25, 3, -0.5, 1, -2]
    wo = np.zeros((H, 16), dtype=np.float32)
    for i in range(4):
        wo[i, 1 * D + i] = 1.0        # head 1 (group 0)
        wo[4 + i, 2 * D + i] = 1.0    # head 2 (group 1)
    fill = {"embed": E, "layers.0.wv": wv, "layers.0.wo": wo,
            "layers.0.wd": np.zeros((H, 6)), "layers.1.wo": np.zeros((H, 16)),
            "layers.1.wd": np.zeros((H, 6))}
    w = tiny_weights(fill, seed=3)
    z = np.zeros((2, 2, 0, 4))
    r = O.draft_block(w, z, z, p=0, anchor_id=5, mask_id=10, block=1, g=TINY)
    x = 1.0 / math.sqrt(1.0 + 1e-6)
    v = np.array([0.5, -1, 2, 0.25, 3, -0.5, 1, -2]) * x
    want = 1.0 + v.astype(np.float16).astype(np.float64)  # V cells are fp16
    assert np.allclose(r["x_last"][0], want, rtol=1e-12)
    assert r["cand"].shape == (0,)


def _tiny_random_pass(**kw):
    w = tiny_weights(seed=11)
    rng = np.random.default_rng(12)
    Kc = O.f16_round(rng.standard_normal((2, 2, 3, 4)))
    Vc = O.f16_round(rng.standard_normal((2, 2, 3, 4)))
    return O.draft_block(w, Kc, Vc, p=3, anchor_id=2, mask_id=10, block=5,
                         g=TINY, **kw)


def test_mask_row_order_only_matters_through_positions():
    """Permuting the positions of the mask rows permutes their outputs
    exactly; the anchor row does not change."""
    base = _tiny_random_pass()
    sigma = [3, 1, 4, 2]                       # mask row i gets position p + sigma
    r = _tiny_random_pass(row_positions=[3] + [3 + s for s in sigma])
    assert np.array_equal(r["hidden"][0], base["hidden"][0])
    for i, s in enumerate(sigma, start=1):
        assert np.array_equal(r["hidden"][i], base["hidden"][s])
        assert np.array_equal(r["logits"][i - 1], base["logits"][s - 1])


def test_block_attention_is_non_causal():
    """Changing the token of the last block row changes row 1 (a causal mask
    would hide the later row from it)."""
    base = _tiny_random_pass()
    r = _tiny_random_pass(row_tokens=[2, 10, 10, 10, 7])
    assert not np.allclose(r["hidden"][1], base["hidden"][1])


def test_q8_0_lm_head_logits_closed_form():
    """A Q8_0 LM head (hidden 32, one quant block per vocabulary row): with
    the attention and MLP branches zeroed the hidden state is the final norm
    of the embedding row, here the constant 1/sqrt(1 + eps), so logit v is
    d_v * sum_j q_vj / sqrt(1 + eps).  Pins that the LM head's own format
    is used (not the backbone's), the int8 sign and the fp16 scale."""
    G = O.geometry(hidden=32, n_layers=1, n_q_heads=2, n_kv_heads=1, head_dim=4,
                   ffn=8, vocab=5, window=4)
    rng = np.random.default_rng(31)
    w = {"__format__": "bf16", "__lm_format__": "q8_0"}
    for name, shape, kind in synth.weight_specs(G):
        if kind == "gain":
            w[name] = b16(np.ones(shape, dtype=np.float32))
        elif name in ("layers.0.wo", "layers.0.wd"):
            w[name] = b16(np.zeros(shape, dtype=np.float32))
        else:
            w[name] = b16(rng.integers(-8, 9, size=shape).astype(np.float32) / 16)
    w["embed"] = b16(np.ones((5, 32), dtype=np.float32))
    q = rng.integers(-127, 128, size=(5, 32)).astype(np.int8)
    q[3] = 127                       # the largest row sum
    q[1] = -127
    d = np.array([0.5, 0.25, 2.0 ** -6, 0.125, 1.5], dtype=np.float16)
    w["lm_head"] = np.concatenate([q.reshape(-1).view(np.uint8), d.view(np.uint8)])
    z = np.zeros((1, 1, 0, 4))
    r = O.draft_block(w, z, z, p=0, anchor_id=2, mask_id=4, block=3, g=G)
    want = d.astype(np.float64) * q.astype(np.float64).sum(axis=1) / math.sqrt(1 + 1e-6)
    assert np.allclose(r["logits"], np.tile(want, (2, 1)), rtol=1e-12)
    assert list(r["cand"]) == [int(np.argmax(want))] * 2


# ------------------------------------------------------------ q/k path
# Pins in which a score depends on the query's norm, gain and position and on
# the block keys' rotation (PR #1426 "Drafter runtime": per-head q/k RMSNorm
# before full-head NeoX RoPE at each row's own position p + i; "Correctness
# debugging and fixes": rows must not share the anchor's position; "Parity
# validation": the "q normed" stage).  TINY has head_dim 4, so the pair
# (0, 2) turns at frequency theta^0 = 1: a vector (c, 0, 0, 0) at position m
# becomes (c cos m, 0, c sin m, 0).

def _rms1(v, gain0, dim=4):
    """RMSNorm of a head vector (v, 0, ..., 0) over `dim` entries, entry 0
    only: v / sqrt(v^2 / dim + eps) * gain0 (closed form of the norm)."""
    return v / math.sqrt(v * v / dim + 1e-6) * gain0


def _x0(e, H=8):
    """Input RMSNorm (unit gains) of a constant row of value e: every entry
    is e / sqrt(e^2 + eps)."""
    return e / math.sqrt(e * e + 1e-6)


def test_query_norm_gain_and_row_position_against_one_context_key():
    """One visible context cell with key kappa (cos phi, 0, sin phi, 0) and
    value Vc; block keys and values are zero (Wk = Wv = 0).  Query head h is
    (a_h x_0, 0, 0, 0) before its norm, so after the norm (gain g0 = 1.5) and
    RoPE at p + i its score against the context key is
    scale * q0_h * kappa * cos(p + i - phi) with q0_h the closed-form norm.
    The block's three zero keys add e^0 each to the softmax denominator, so
    the head output is w Vc with w = e^s / (e^s + 3).  Wo copies head 1
    (group 0) into h[0:4] and head 2 (group 1) into h[4:8]."""
    H, D, B, p, phi = 8, 4, 3, 1, 0.7
    a = [0.5, -0.75, 1.25, 2.0]
    wq = np.zeros((16, H), dtype=np.float32)
    for h in range(4):
        wq[h * D, 0] = a[h]
    wo = np.zeros((H, 16), dtype=np.float32)
    for i in range(4):
        wo[i, 1 * D + i] = 1.0
        wo[4 + i, 2 * D + i] = 1.0
    qn = np.ones(4, dtype=np.float32)
    qn[0] = 1.5
    fill = {"embed": _const_embed({1: 1.0, 10: 2.0}), "layers.0.wq": wq,
            "layers.0.wk": np.zeros((8, H)), "layers.0.wv": np.zeros((8, H)),
            "layers.0.q_norm": qn, "layers.0.wo": wo, "layers.0.wd": np.zeros((H, 6)),
            "layers.1.wo": np.zeros((H, 16)), "layers.1.wd": np.zeros((H, 6))}
    w = tiny_weights(fill, seed=21)
    kappa = [8.0, -6.0]
    Vc = np.array([[1.0, -2.0, 3.0, 0.5], [-1.0, 0.25, 2.0, 4.0]])
    ck = np.zeros((2, 2, 1, D))
    cv = np.zeros((2, 2, 1, D))
    for j in range(2):
        ck[0, j, 0] = [kappa[j] * math.cos(phi), 0.0, kappa[j] * math.sin(phi), 0.0]
        cv[0, j, 0] = Vc[j]
    r = O.draft_block(w, ck, cv, p=p, anchor_id=1, mask_id=10, block=B, g=TINY)
    for i, e in enumerate((1.0, 2.0, 2.0)):
        m = p + i
        want = [e] * H
        for head, j, off in ((1, 0, 0), (2, 1, 4)):
            q0 = _rms1(a[head] * _x0(e), 1.5)
            s = (1.0 / 16.0) * q0 * kappa[j] * math.cos(m - phi)
            wgt = math.exp(s) / (math.exp(s) + B)
            for d in range(D):
                want[off + d] += wgt * Vc[j, d]
        assert np.allclose(r["x_last"][i], want, rtol=1e-9, atol=1e-12), (i, r["x_last"][i], want)


def test_block_keys_rotate_at_their_own_positions():
    """No visible context keys carry weight (four zero cells: score 0, value
    0); queries and keys of all three block rows are (c, 0, 0, 0) before
    their norms (gains 4 and 3), so q = 8 (cos m_i, 0, sin m_i, 0) and the
    stored fp16 key of row r is (k cos m_r, 0, k sin m_r, 0) rounded to fp16,
    k = 6.  Values are +c_j (anchor) and -c_j (mask rows: their embedding
    alternates sign and Wv reads entry 1).  The output of row i is
    sum_r w_ir v_r with w_ir = e^(s_ir) / (sum_r' e^(s_ir') + 4) and
    s_ir = (1/16) q_i . k_r: the block keys enter at their own positions
    p + r, so the scores depend on m_i - m_r only up to the fp16 rounding."""
    H, D, B, p = 8, 4, 3, 5
    E = np.zeros((11, H), dtype=np.float32)
    E[1] = 1.0
    E[10] = [1.0, -1.0] * 4
    wq = np.zeros((16, H), dtype=np.float32)
    for h in range(4):
        wq[h * D, 0] = 1.0
    wk = np.zeros((8, H), dtype=np.float32)
    wk[0, 0] = wk[D, 0] = 1.0
    cvals = np.array([[1.0, 2.0, -1.0, 0.5], [0.25, -3.0, 1.5, 2.0]])
    wv = np.zeros((8, H), dtype=np.float32)
    for j in range(2):
        wv[j * D:(j + 1) * D, 1] = cvals[j]
    wo = np.zeros((H, 16), dtype=np.float32)
    for i in range(4):
        wo[i, 0 * D + i] = 1.0        # head 0 (group 0) -> h[0:4]
        wo[4 + i, 3 * D + i] = 1.0    # head 3 (group 1) -> h[4:8]
    qn = np.array([4.0, 1, 1, 1], dtype=np.float32)
    kn = np.array([3.0, 1, 1, 1], dtype=np.float32)
    fill = {"embed": E, "layers.0.wq": wq, "layers.0.wk": wk, "layers.0.wv": wv,
            "layers.0.q_norm": qn, "layers.0.k_norm": kn, "layers.0.wo": wo,
            "layers.0.wd": np.zeros((H, 6)), "layers.1.wo": np.zeros((H, 16)),
            "layers.1.wd": np.zeros((H, 6))}
    w = tiny_weights(fill, seed=22)
    z = np.zeros((2, 2, 4, D))
    r = O.draft_block(w, z, z, p=p, anchor_id=1, mask_id=10, block=B, g=TINY)
    x0 = _x0(1.0)                       # |entries| of both rows after the norm
    q0, k0 = _rms1(x0, 4.0), _rms1(x0, 3.0)
    f16 = lambda v: float(np.float16(v))
    keys = [(f16(k0 * math.cos(p + rr)), f16(k0 * math.sin(p + rr))) for rr in range(B)]
    sign = [1.0, -1.0, -1.0]            # entry 1 of the anchor / mask rows
    for i, e_row in enumerate((E[1], E[10], E[10])):
        m = p + i
        s = [(1.0 / 16.0) * q0 * (math.cos(m) * kc + math.sin(m) * ks) for kc, ks in keys]
        den = sum(math.exp(v) for v in s) + 4.0
        want = e_row.astype(np.float64).copy()
        for j, off in ((0, 0), (1, 4)):
            for d in range(D):
                want[off + d] += sum(math.exp(s[rr]) / den * f16(sign[rr] * x0 * cvals[j, d])
                                     for rr in range(B))
        assert np.allclose(r["x_last"][i], want, rtol=1e-9, atol=1e-12), (i, r["x_last"][i], want)


def test_query_and_key_norms_remove_projection_scale():
    """The per-head q/k RMSNorm makes the pass independent of the scale of
    Wq and Wk (up to eps): multiplying every layer's Wq by 4 and Wk by 1/4
    (exact in bf16) leaves the outputs unchanged to within the eps term and
    one fp16 rounding of a block key; dropping either norm would scale the
    scores by 4."""
    base = _tiny_random_pass()
    w = tiny_weights(seed=11)
    for l in range(2):
        for name, f in (("wq", 4.0), ("wk", 0.25)):
            v = O.bf16_decode(w[f"layers.{l}.{name}"]) * f
            w[f"layers.{l}.{name}"] = b16(v.astype(np.float32))
    rng = np.random.default_rng(12)
    Kc = O.f16_round(rng.standard_normal((2, 2, 3, 4)))
    Vc = O.f16_round(rng.standard_normal((2, 2, 3, 4)))
    r = O.draft_block(w, Kc, Vc, p=3, anchor_id=2, mask_id=10, block=5, g=TINY)
    scale = np.abs(base["x_last"]).max()
    assert np.abs(r["x_last"] - base["x_last"]).max() <= 2e-3 * scale
    assert np.abs(r["logits"] - base["logits"]).max() <= 2e-3 * np.abs(base["logits"]).max()


def test_mask_rows_with_distinct_tokens_permute_with_their_positions():
    """Mask rows carrying distinct tokens (so distinct queries, keys and
    values): permuting the (token, position) pairs among the mask rows
    permutes the outputs exactly, and swapping only the positions of two
    distinct rows changes both of them (the queries are roped at the row's
    own position, not the anchor's)."""
    toks = [2, 3, 5, 7, 9]
    pos = [3, 4, 5, 6, 7]
    base = _tiny_random_pass(row_tokens=toks, row_positions=pos)
    sigma = [3, 1, 4, 2]
    r = _tiny_random_pass(row_tokens=[toks[0]] + [toks[s] for s in sigma],
                          row_positions=[pos[0]] + [pos[s] for s in sigma])
    assert np.array_equal(r["hidden"][0], base["hidden"][0])
    for i, s in enumerate(sigma, start=1):
        assert np.array_equal(r["hidden"][i], base["hidden"][s])
    sw = _tiny_random_pass(row_tokens=toks, row_positions=[3, 5, 4, 6, 7])
    assert not np.allclose(sw["hidden"][1], base["hidden"][1])
    assert not np.allclose(sw["hidden"][2], base["hidden"][2])


# ------------------------------------------------------------ confidence gate

def test_confidence_uniform_logits_is_one_over_vocab():
    """Equal logits: every id has probability 1/V (closed form)."""
    for v in (1, 7, 151936):
        assert O.candidate_confidence(np.full(v, 0.37)) == pytest.approx(1.0 / v, rel=1e-12)


def test_confidence_one_raised_logit_closed_form():
    """One logit a above n-1 zeros: p = e^a / (e^a + n - 1); the candidate is
    the raised id wherever it sits (a wrong index or a min instead of a max
    gives 1 / (e^a + n - 1))."""
    for n, a, at in ((10, 2.0, 0), (1000, 5.5, 617), (151936, 12.25, 151935)):
        row = np.zeros(n)
        row[at] = a
        want = math.exp(a) / (math.exp(a) + n - 1)
        assert O.candidate_confidence(row) == pytest.approx(want, rel=1e-12)


def test_confidence_two_level_logits_and_ties():
    """k ids at a and n-k at b: p = e^a / (k e^a + (n-k) e^b) for the lowest
    of the tied top ids."""
    n, k, a, b = 50, 3, 1.5, -0.25
    row = np.full(n, b)
    row[[4, 9, 30]] = a
    want = math.exp(a) / (k * math.exp(a) + (n - k) * math.exp(b))
    assert O.candidate_confidence(row) == pytest.approx(want, rel=1e-12)


def test_confidence_is_shift_invariant_and_does_not_overflow():
    """Softmax ignores a common shift; logits near 1e3 stay finite."""
    rng = np.random.default_rng(5)
    row = rng.normal(size=4096) * 3
    base = O.candidate_confidence(row)
    assert 0.0 < base < 1.0
    assert O.candidate_confidence(row + 1000.0) == pytest.approx(base, rel=1e-9)
    assert O.candidate_confidence(row - 1000.0) == pytest.approx(base, rel=1e-9)


def test_confidence_matches_brute_force_on_tiny_rows():
    """Probability of the argmax by summing exp over a 4-entry row written
    out by hand."""
    row = [0.5, -1.0, 2.0, 0.0]
    want = math.exp(2.0) / (math.exp(0.5) + math.exp(-1.0) + math.exp(2.0) + math.exp(0.0))
    assert O.candidate_confidence(row) == pytest.approx(want, rel=1e-12)


def test_gate_stops_at_first_candidate_below_floor():
    conf = [0.9, 0.5, 0.05, 0.8]
    assert O.gate_candidates(conf, 0.0) == 4
    assert O.gate_candidates(conf, 0.1) == 2   # the later 0.8 is cut too
    assert O.gate_candidates(conf, 0.5) == 2   # at the floor is kept
    assert O.gate_candidates(conf, 0.51) == 1
    assert O.gate_candidates(conf, 0.95) == 0
    assert O.gate_candidates([], 0.5) == 0
