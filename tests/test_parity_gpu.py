"""GPU parity: every entry point of the C ABI against the CPU oracle on the
same seeded inputs.

Bars (identical for all cases):
  * candidate ids and accepted lengths: exactly equal wherever the oracle's
    top-2 logit margin exceeds 0.05 (a smaller margin lets both ids stand);
  * bf16 logits, hidden states, fused context and fp16 K/V: per row,
    max|gpu - oracle| / max|oracle| <= 2e-2.
"""
import math
import sys

import numpy as np
import pytest
import torch

from block_draft_model_pass_amd import synth
from block_draft_model_pass_amd.device import DeviceWeights, Drafter, KVRing, to_device
from oracle import dflash_oracle as O

pytestmark = pytest.mark.gpu

TOL = 2e-2
MARGIN = 0.05


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dec_bf16(t: torch.Tensor) -> np.ndarray:
    u = t.cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def dec_f16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.float16).astype(np.float64)


def row_rel_err(g: np.ndarray, o: np.ndarray) -> float:
    g = g.reshape(-1, g.shape[-1])
    o = o.reshape(-1, o.shape[-1])
    return float(np.max(np.abs(g - o).max(axis=1) / np.abs(o).max(axis=1)))


@pytest.fixture(scope="module")
def host_w():
    return synth.make_weights()


@pytest.fixture(scope="module")
def dev_w(host_w):
    return DeviceWeights(host_w)


@pytest.fixture(scope="module")
def ow(host_w):
    return O.enable_cache(dict(host_w))


def check_cands(c, ref_cand, ref_logits, margin):
    """Candidate ids: equal to the oracle's where its top-2 margin exceeds
    MARGIN; elsewhere more than one id is correct, and the id taken must
    still be one of them (its oracle logit within MARGIN of the row's
    maximum)."""
    c = np.asarray(c)
    sure = margin > MARGIN
    assert np.array_equal(c[sure], ref_cand[sure]), (c, ref_cand, margin)
    ref_logits = np.asarray(ref_logits, dtype=np.float64)
    got = ref_logits[np.arange(len(c)), c]
    assert np.all(got >= ref_logits.max(axis=1) - MARGIN), (c, ref_cand, got, margin)


def check_draft(res_gpu, ref, block, tag):
    cand, logits, hidden = res_gpu
    he = row_rel_err(dec_bf16(hidden), ref["hidden"])
    say(f"[{tag}] hidden rel err {he:.3e}")
    assert he <= TOL
    if block > 1:
        le = row_rel_err(dec_bf16(logits), ref["logits"])
        c = cand.cpu().numpy()
        say(f"[{tag}] logits rel err {le:.3e} cand {c.tolist()} ref {ref['cand'].tolist()} "
            f"margins {np.round(ref['margin'], 3).tolist()}")
        assert le <= TOL
        check_cands(c, ref["cand"], ref["logits"], ref["margin"])


def gpu_draft(dr: Drafter, p, anchor, block, vocab):
    cand = torch.empty(max(block - 1, 1), dtype=torch.int32, device="cuda")
    logits = torch.empty((max(block - 1, 1), vocab), dtype=torch.int16, device="cuda")
    hidden = torch.empty((block, synth.HIDDEN), dtype=torch.int16, device="cuda")
    dr.draft(p, anchor, block, cand=cand, logits=logits, hidden=hidden)
    torch.cuda.synchronize()
    return cand[:block - 1], logits[:block - 1], hidden


# ------------------------------------------------------------------ verify

def test_verify_greedy_matches_oracle():
    rng = np.random.default_rng(0)
    cases = [([11, 12], [11, 12, 13]), ([11, 99], [11, 12, 13]), ([98, 12], [11, 12, 13]),
             ([], [5])]
    for _ in range(150):
        k = int(rng.integers(0, 8))
        cases.append((rng.integers(0, 3, size=k).tolist(), rng.integers(0, 3, size=k + 1).tolist()))
    out = torch.empty(2, dtype=torch.int32, device="cuda")
    from block_draft_model_pass_amd import _lib
    for cand, tgt in cases:
        c = torch.tensor(cand + [0], dtype=torch.int32, device="cuda")
        t = torch.tensor(tgt, dtype=torch.int32, device="cuda")
        _lib.dflash_verify_greedy(c.data_ptr(), t.data_ptr(), len(cand), out.data_ptr())
        torch.cuda.synchronize()
        assert tuple(out.cpu().tolist()) == O.verify_greedy(cand, tgt), (cand, tgt)


# ------------------------------------------------------------------ fusion

@pytest.mark.parametrize("n", [1, 13, 40, 300])
def test_fuse_context(dev_w, ow, n):
    """n <= 64 runs the skinny GEMV path (ragged 16-row chunks), larger n the
    MFMA GEMM with a ragged last tile."""
    say(f"fuse n={n}")
    taps = synth.make_taps(range(1000, 1000 + n))
    dr = Drafter(dev_w, KVRing(256), max_rows=n)
    ctx = dr.fuse(to_device(taps))
    torch.cuda.synchronize()
    ref = O.bf16_decode(O.fuse_context(ow, taps))
    err = row_rel_err(dec_bf16(ctx), ref)
    say(f"fuse n={n} rel err {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("n", [13, 40, 300])
def test_few_row_paths_without_streaming_copies(dev_w, ow, n):
    """Fusion and projection read the row-major tensors when the descriptor
    carries no streaming copies -- the few-row GEMV (13, 40) and the many-row
    GEMM (300, k split in two): same bars."""
    saved = dev_w.desc.packed
    dev_w.desc.packed = None
    try:
        taps = synth.make_taps(range(700, 700 + n))
        dr = Drafter(dev_w, KVRing(2048, window=2048), max_rows=n)
        ctx = dr.fuse(to_device(taps))
        dr.project(ctx, 900)
        torch.cuda.synchronize()
    finally:
        dev_w.desc.packed = saved
    octx = O.fuse_context(ow, taps)
    err = row_rel_err(dec_bf16(ctx), O.bf16_decode(octx))
    K, V = O.project_ctx_kv(ow, ctx.cpu().numpy().view(np.uint16), 900)
    gK, gV = ring_cells(dr.kv, range(900, 900 + n))
    ek, ev = row_rel_err(gK, K), row_rel_err(gV, V)
    say(f"row-major few-row paths n={n}: fuse {err:.3e} K {ek:.3e} V {ev:.3e}")
    assert err <= TOL and ek <= TOL and ev <= TOL


@pytest.mark.parametrize("n", [2432, 2700, 6400, 6401, 12801])
def test_fuse_context_split_sampled(dev_w, ow, n):
    """Many-row fusion around the k-split rule: fewer output tiles than
    compute units split the k range in two (2432 rows: 100 tiles; 2700 rows:
    110 tiles; 6400 rows: 250 tiles), and so does a last wave of tiles that
    leaves most units idle (6401 rows: 260 tiles, ragged); 510 tiles do not
    (12801 rows, ragged last tile: the GEMM writes bf16 rows and tile sums of
    squares, which the tile norm reads); the oracle recomputes sampled rows
    including the ends of the first panel and of the buffer."""
    say(f"fuse split n={n}")
    taps = synth.make_taps(range(5000, 5000 + n))
    dr = Drafter(dev_w, KVRing(256), max_rows=n)
    ctx = dr.fuse(to_device(taps))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 255, 256, n - 2, n - 1],
                                     np.random.default_rng(n).integers(0, n, 19)]))
    ref = O.bf16_decode(O.fuse_context(ow, taps[rows]))
    err = row_rel_err(dec_bf16(ctx)[rows], ref)
    say(f"fuse split n={n} rel err {err:.3e}")
    assert err <= TOL


def test_fuse_context_full_size_sampled(dev_w, ow):
    """32768 x 12800 @ 12800 x 2560 (the long-context fusion GEMM); the
    oracle recomputes 40 sampled rows including both ends."""
    n = 32768
    say("fuse full n=32768")
    positions = np.arange(229376, 229376 + n)
    taps = synth.make_taps(positions)
    dr = Drafter(dev_w, KVRing(256), max_rows=n)
    ctx = dr.fuse(to_device(taps))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 127, 128, n - 1],
                                     np.random.default_rng(1).integers(0, n, 35)]))
    ref = O.bf16_decode(O.fuse_context(ow, taps[rows]))
    err = row_rel_err(dec_bf16(ctx)[rows], ref)
    say(f"fuse full rel err {err:.3e}")
    assert err <= TOL


# ------------------------------------------------------------------ projection

def ring_cells(kv: KVRing, positions):
    cells = np.asarray(positions) % kv.capacity
    K = dec_f16(kv.k)[:, :, cells, :]
    V = dec_f16(kv.values())[:, :, cells, :]
    return K, V


@pytest.mark.parametrize("n,pos0,cap", [(1, 0, 256), (40, 1000, 1024), (300, 229376, 32768),
                                         (200, 1000, 1024), (150, 1001, 1024),
                                         (2500, 1001, 2560), (2200, 229379, 32768)])
def test_project_ctx_kv(dev_w, ow, n, pos0, cap):
    """Skinny path with ring wrap-around (pos0 = 1000, capacity 1024), the
    GEMM path at 256K-range positions, and the GEMM path starting inside a
    32-cell value block and wrapping around the ring, with pos0 a multiple
    of 4 (values stored 4 cells at a time) and not.  Above 2048 rows the
    cells come from the GEMM's own epilogue: there with ring wrap-around,
    value blocks cut by the tile and half-tile boundaries (pos0 = 1001 and
    229379, not multiples of 32) and a partial last tile (2200 rows).  Cells
    outside the projected range must stay untouched (the ring starts
    zeroed)."""
    say(f"project n={n} pos0={pos0} cap={cap}")
    ctx = synth.make_rows(n, synth.HIDDEN, seed=77)
    kv = KVRing(cap, window=cap)
    dr = Drafter(dev_w, kv, max_rows=n)
    dr.project(to_device(ctx), pos0)
    torch.cuda.synchronize()
    K, V = O.project_ctx_kv(ow, ctx, pos0)
    gK, gV = ring_cells(kv, range(pos0, pos0 + n))
    ek = row_rel_err(gK, K)
    ev = row_rel_err(gV, V)
    say(f"project n={n} K err {ek:.3e} V err {ev:.3e}")
    assert ek <= TOL and ev <= TOL
    other = np.setdiff1d(np.arange(cap), np.arange(pos0, pos0 + n) % cap)
    assert not kv.k.cpu().numpy()[:, :, other, :].any()
    assert not kv.values().cpu().numpy()[:, :, other, :].any()


def test_project_full_size_sampled(dev_w, ow):
    n, pos0 = 32768, 229376
    say("project full n=32768")
    ctx = synth.make_rows(n, synth.HIDDEN, seed=78)
    kv = KVRing(32768)
    dr = Drafter(dev_w, kv, max_rows=n)
    dr.project(to_device(ctx), pos0)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 127, 128, n - 1],
                                     np.random.default_rng(2).integers(0, n, 27)]))
    K, V = O.project_ctx_kv(ow, ctx[rows], 0)  # positions fixed below
    # recompute keys at their true positions (RoPE depends on them)
    Kt = np.empty_like(K)
    for i, r in enumerate(rows):
        Kt[:, :, i:i + 1] = O.project_ctx_kv(ow, ctx[r:r + 1], pos0 + int(r))[0]
    gK, gV = ring_cells(kv, pos0 + rows)
    ek, ev = row_rel_err(gK, Kt), row_rel_err(gV, V)
    say(f"project full K err {ek:.3e} V err {ev:.3e}")
    assert ek <= TOL and ev <= TOL


# ------------------------------------------------------------------ draft pass

def end_to_end(dev_w, ow, n, block, p=None, cap=32768, window=32768, tag=""):
    """Fuse + project n context positions (0..n-1) on both sides, then draft
    one block at p = n."""
    p = n if p is None else p
    say(f"[{tag}] end-to-end n={n} block={block} p={p}")
    g = O.geometry(window=window)
    kv = KVRing(cap, window=window)
    dr = Drafter(dev_w, kv, max_rows=min(n, cap) if n else 16)
    store = O.ContextStore(g)
    step = min(n, cap) if n else 1
    for s in range(0, n, step):
        e = min(n, s + step)
        taps = synth.make_taps(range(s, e))
        dr.commit(to_device(taps), s)
        ctx = O.fuse_context(ow, taps)
        store.put(*O.project_ctx_kv(ow, ctx, s), s)
    anchor = synth.anchor_token(p)
    res = gpu_draft(dr, p, anchor, block, dev_w.vocab)
    ck, cv = store.window(p)
    ref = O.draft_block(ow, ck, cv, p, anchor, synth.MASK_ID, block, g)
    check_draft(res, ref, block, tag)
    return res, ref


def test_draft_config_smallest(dev_w, ow):
    """32 context positions, block of anchor + 3 masks at position 32."""
    end_to_end(dev_w, ow, 32, 4, tag="ctx32 b4")


@pytest.mark.parametrize("block", [1, 2, 5, 8])
def test_draft_no_context(dev_w, ow, block):
    """p = 0: attention over the block rows only (block 1: the anchor alone)."""
    end_to_end(dev_w, ow, 0, block, tag=f"ctx0 b{block}")


def test_draft_window_and_ring_wrap(dev_w, ow):
    """Capacity 1024, window 512, anchor at 1500: the visible positions
    988..1499 wrap around the ring and older cells are overwritten."""
    end_to_end(dev_w, ow, 1500, 8, cap=1024, window=512, tag="wrap")


def test_draft_config_short_prompt(dev_w, ow):
    """2432 context positions through the GEMM paths, block 8 at 2432."""
    end_to_end(dev_w, ow, 2432, 8, tag="ctx2432 b8")


def test_draft_long_resident_context(dev_w, ow):
    """32768 resident fp16 cells at positions 229376..262143, block 8 at
    262144 (cells written straight into the ring in the documented layout)."""
    n, lo, p = 32768, 229376, 262144
    say("long context 32768")
    kv = KVRing(32768)
    Kh = synth.make_rows(5 * 2 * n, 256, seed=91, dtype="f16").reshape(5, 2, n, 256)
    Vh = synth.make_rows(5 * 2 * n, 256, seed=92, dtype="f16").reshape(5, 2, n, 256)
    cells = np.arange(lo, p) % 32768
    assert np.array_equal(cells, np.arange(n))  # 229376 = 7 * 32768: cells in order
    kv.k.copy_(to_device(Kh).view(torch.float16))
    kv.set_values(to_device(Vh).view(torch.float16))
    dr = Drafter(dev_w, kv, max_rows=16)
    anchor = synth.anchor_token(p)
    res = gpu_draft(dr, p, anchor, 8, dev_w.vocab)
    ck = Kh.view(np.float16).astype(np.float64)
    cv = Vh.view(np.float16).astype(np.float64)
    ref = O.draft_block(ow, ck, cv, p, anchor, synth.MASK_ID, 8)
    check_draft(res, ref, 8, "ctx32768 b8")


def test_draft_is_deterministic(dev_w):
    """Two identical passes give bit-identical logits and ids."""
    kv = KVRing(1024)
    dr = Drafter(dev_w, kv, max_rows=64)
    dr.commit(to_device(synth.make_taps(range(64))), 0)
    a = gpu_draft(dr, 64, 7, 8, dev_w.vocab)
    b = gpu_draft(dr, 64, 7, 8, dev_w.vocab)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ------------------------------------------------------------------ decode loop

def test_decode_loop_short(dev_w, ow):
    """propose -> verify -> commit with the stand-in target: accepted lengths
    equal the oracle's on every pass; candidates agree (margin rule) until a
    near-tie candidate changes the next anchor."""
    ctx0, want = 256, 24
    say("decode loop ctx=256")
    kv = KVRing(1024)
    dr = Drafter(dev_w, kv, max_rows=ctx0)
    dr.commit(to_device(synth.make_taps(range(ctx0))), 0)
    store = O.ContextStore()
    store.put(*O.project_ctx_kv(ow, O.fuse_context(ow, synth.make_taps(range(ctx0))), 0), 0)
    p, anchor = ctx0, synth.anchor_token(0)
    o_p, o_anchor = p, anchor
    committed, t, same_path = 0, 0, True
    K = synth.MAX_BLOCK - 1
    cand = torch.empty(K, dtype=torch.int32, device="cuda")
    out = torch.empty(2, dtype=torch.int32, device="cuda")
    compared = 0
    while committed < want:
        dr.draft(p, anchor, K + 1, cand=cand)
        c = cand.cpu().numpy()
        tgt = synth.synthetic_target(c, t)
        dr.verify(cand, to_device(tgt), K, out=out)
        a, nxt = out.cpu().tolist()
        ck, cv = store.window(o_p)
        ref = O.draft_block(ow, ck, cv, o_p, o_anchor, synth.MASK_ID, K + 1)
        o_tgt = synth.synthetic_target(ref["cand"], t)
        oa, onxt = O.verify_greedy(ref["cand"], o_tgt)
        assert a == oa, (t, a, oa)
        if same_path:
            check_cands(c, ref["cand"], ref["logits"], ref["margin"])
            compared += 1
            if nxt != onxt:
                same_path = False
        dr.commit(to_device(synth.make_taps(range(p, p + a + 1))), p)
        store.put(*O.project_ctx_kv(ow, O.fuse_context(ow, synth.make_taps(range(o_p, o_p + oa + 1))), o_p), o_p)
        p, anchor = p + a + 1, nxt
        o_p, o_anchor = o_p + oa + 1, onxt
        committed += a + 1
        t += 1
    say(f"decode loop: {t} passes, {compared} compared on the same path")
    assert compared >= 1


def test_barrier_timeout_reports_minus_one(dev_w, monkeypatch):
    """A grid barrier that stops waiting (forced from the host with a
    wall-clock bound of 0) makes the pass report cand = -1; the next pass,
    with the default bound, is correct again (every pass starts from fresh
    barrier words).  No kernel waits unboundedly on this path."""
    kv = KVRing(256)
    dr = Drafter(dev_w, kv)
    good = dr.draft(100, 11, 8).cpu().numpy().copy()
    torch.cuda.synchronize()
    monkeypatch.setenv("DFLASH_BARRIER_TIMEOUT_US", "0")
    bad = dr.draft(100, 11, 8).cpu().numpy().copy()
    torch.cuda.synchronize()
    monkeypatch.delenv("DFLASH_BARRIER_TIMEOUT_US")
    again = dr.draft(100, 11, 8).cpu().numpy().copy()
    torch.cuda.synchronize()
    say(f"timeout path: good {good.tolist()} forced {bad.tolist()} again {again.tolist()}")
    assert (bad == -1).all()
    assert np.array_equal(good, again)
