"""GPU parity of the fused draft-commit cycle (dflash_draft_block_commit: the
commit of the cells the last verify accepted -- their fusion and per-layer
K/V projection -- and the next proposal pass in one launch) against the
oracle's commit (fuse_context + project_ctx_kv) followed by its draft_block,
on the same seeded inputs.

Bars as everywhere: ids exact where the oracle's top-2 margin exceeds 0.05,
logits and hidden states within 2e-2 per-row relative error, and the
committed fp16 K/V cells within 2e-2 of the oracle's.  With no commit rows
the call is the plain pass, bit for bit.
"""
import numpy as np
import pytest
import torch

from block_draft_model_pass_amd import _lib, synth
from block_draft_model_pass_amd.device import DeviceWeights, Drafter, KVRing, to_device
from oracle import dflash_oracle as O
from test_parity_gpu import (TOL, check_cands, check_draft, ring_cells, row_rel_err, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def host_w():
    return synth.make_weights()


@pytest.fixture(scope="module")
def dev_w(host_w):
    return DeviceWeights(host_w)


@pytest.fixture(scope="module")
def ow(host_w):
    return O.enable_cache(dict(host_w))


def outputs(block, vocab):
    return (torch.empty(max(block - 1, 1), dtype=torch.int32, device="cuda"),
            torch.empty((max(block - 1, 1), vocab), dtype=torch.int16, device="cuda"),
            torch.empty((block, synth.HIDDEN), dtype=torch.int16, device="cuda"))


def fused_case(dev_w, ow, n_ctx, nc, block, cap=32768, window=32768, tag=""):
    """Context positions 0 .. n_ctx-1 committed on both sides, then one fused
    call committing positions n_ctx .. n_ctx+nc-1 and drafting at
    p = n_ctx + nc; compared with the oracle's commit then draft."""
    p = n_ctx + nc
    say(f"[fused {tag}] ctx {n_ctx} commit {nc} block {block} cap {cap} window {window}")
    g = O.geometry(window=window)
    kv = KVRing(cap, window=window)
    dr = Drafter(dev_w, kv, max_rows=max(min(n_ctx, cap), 16))
    store = O.ContextStore(g)
    step = min(n_ctx, cap) if n_ctx else 1
    for s in range(0, n_ctx, step):
        e = min(n_ctx, s + step)
        taps = synth.make_taps(range(s, e))
        dr.commit(to_device(taps), s)
        store.put(*O.project_ctx_kv(ow, O.fuse_context(ow, taps), s), s)
    ctaps = synth.make_taps(range(n_ctx, p))
    store.put(*O.project_ctx_kv(ow, O.fuse_context(ow, ctaps), n_ctx), n_ctx)
    anchor = synth.anchor_token(p)
    cand, logits, hidden = outputs(block, dev_w.vocab)
    tg = to_device(ctaps)
    dr.draft_commit(tg.data_ptr() if nc else None, nc, p, anchor, block, cand=cand,
                    logits=logits, hidden=hidden)
    torch.cuda.synchronize()
    ck, cv = store.window(p)
    ref = O.draft_block(ow, ck, cv, p, anchor, synth.MASK_ID, block, g)
    check_draft((cand[:block - 1], logits[:block - 1], hidden), ref, block, f"fused {tag}")
    if nc:
        gK, gV = ring_cells(kv, range(n_ctx, p))
        oK = store.k[:, :, n_ctx - store.base:p - store.base]
        oV = store.v[:, :, n_ctx - store.base:p - store.base]
        ek, ev = row_rel_err(gK, oK), row_rel_err(gV, oV)
        say(f"[fused {tag}] committed cells K err {ek:.3e} V err {ev:.3e}")
        assert ek <= TOL and ev <= TOL
    return dr, (cand, logits, hidden), ref


def test_no_commit_rows_is_the_plain_pass(dev_w):
    """n_commit = 0: bit-identical to dflash_draft_block."""
    kv = KVRing(1024)
    dr = Drafter(dev_w, kv, max_rows=64)
    dr.commit(to_device(synth.make_taps(range(64))), 0)
    c1, l1, h1 = outputs(8, dev_w.vocab)
    c2, l2, h2 = outputs(8, dev_w.vocab)
    dr.draft(64, 7, 8, cand=c1, logits=l1, hidden=h1)
    dr.draft_commit(None, 0, 64, 7, 8, cand=c2, logits=l2, hidden=h2)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(l1, l2) and torch.equal(h1, h2)


@pytest.mark.parametrize("n_ctx,nc,block,cap,window", [
    (40, 1, 8, 1024, 1024),      # one commit row (a cycle that accepted nothing)
    (300, 5, 4, 32768, 32768),   # GEMM-built context, block 4
    (0, 8, 8, 256, 256),         # the commit rows are the whole context
    (1494, 6, 8, 1024, 512),     # ring wrap: positions 1494..1499 in cells 470..475
    (250, 6, 5, 256, 4),         # window 4 < 6 commit rows: only the last four visible
    (8185, 7, 8, 32768, 32768),  # the timed shape: 8192 cells visible at p = 8192
])
def test_fused_cycle_matches_oracle(dev_w, ow, n_ctx, nc, block, cap, window):
    fused_case(dev_w, ow, n_ctx, nc, block, cap, window, tag=f"{n_ctx}+{nc}")


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "q5_0"])
def test_fused_cycle_quantized(fmt):
    """Quantized fc and Wk / Wv: the commit rows' fusion decodes the fc blocks
    in the FC phase, the projection the Wk / Wv blocks in the QKV phase."""
    host = synth.make_weights(fmt=fmt)
    dev = DeviceWeights(host)
    ow = O.enable_cache(dict(host))
    fused_case(dev, ow, 300, 5, 8, tag=fmt)
    del dev
    torch.cuda.empty_cache()


def test_fused_decode_loop_ctx8192(dev_w, ow):
    """The timed decode loop with the fused cycle: 8192 cells committed
    through the GEMM path, then each pass commits the previous cycle's
    accepted cells and the anchor, and drafts block 8.  The target of each
    pass is built from the oracle's candidates and fed to both verifiers;
    both sides follow the oracle's accepted lengths, so every pass is
    compared (as in the unfused decode-loop test)."""
    ctx0, passes, B = 8192, 10, 8
    K = B - 1
    kv = KVRing(32768)
    dr = Drafter(dev_w, kv, max_rows=ctx0)
    taps0 = synth.make_taps(range(ctx0))
    dr.commit(to_device(taps0), 0)
    store = O.ContextStore()
    store.put(*O.project_ctx_kv(ow, O.fuse_context(ow, taps0), 0), 0)
    del taps0
    p, anchor = ctx0, synth.anchor_token(0)
    pending = None  # taps of the cells the last cycle accepted (positions p-n .. p-1)
    cand, logits, hidden = outputs(B, dev_w.vocab)
    out = torch.empty(2, dtype=torch.int32, device="cuda")
    same = 0
    for t in range(passes):
        if pending is None:
            dr.draft_commit(None, 0, p, anchor, B, cand=cand, logits=logits, hidden=hidden)
        else:
            tg = to_device(pending)
            dr.draft_commit(tg.data_ptr(), pending.shape[0], p, anchor, B, cand=cand,
                            logits=logits, hidden=hidden)
        torch.cuda.synchronize()
        ck, cv = store.window(p)
        ref = O.draft_block(ow, ck, cv, p, anchor, synth.MASK_ID, B)
        check_draft((cand, logits, hidden), ref, B, f"fused loop t={t} p={p}")
        c = cand.cpu().numpy()
        tgt = synth.synthetic_target(ref["cand"], t)
        dr.verify(cand, to_device(tgt), K, out=out)
        a, nxt = out.cpu().tolist()
        oa, onxt = O.verify_greedy(ref["cand"], tgt)
        assert (a, nxt) == O.verify_greedy(c, tgt)
        d = min(oa + 1, K)
        if np.array_equal(c[:d], ref["cand"][:d]):
            assert (a, nxt) == (oa, onxt)
            same += 1
        pending = synth.make_taps(range(p, p + oa + 1))
        store.put(*O.project_ctx_kv(ow, O.fuse_context(ow, pending), p), p)
        p, anchor = p + oa + 1, onxt
    say(f"[fused loop] {passes} passes compared, {same} with the oracle's deciding candidates")
    assert same >= 6
    # the last cycle's commit through a plain pass: the ring holds every cell
    gK, gV = ring_cells(kv, range(ctx0, p - pending.shape[0]))
    oK = store.k[:, :, ctx0 - store.base:p - pending.shape[0] - store.base]
    oV = store.v[:, :, ctx0 - store.base:p - pending.shape[0] - store.base]
    assert row_rel_err(gK, oK) <= TOL and row_rel_err(gV, oV) <= TOL
