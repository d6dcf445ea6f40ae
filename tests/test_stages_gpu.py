"""Stage-wise GPU parity of the proposal pass ("Parity validation" on the
PR #1426 page: every block row is compared at every stage of every layer,
not only at the logits).  After a pass, dflash_draft_stage copies the
intermediates the pass kept in its workspace; the oracle records the same
ones (draft_block's `stages`) on the same seeded inputs:

  resid v   the residual stream after the embedding (v = 0) and after each
            attention (2l+1) and MLP (2l+2) residual -- fp32
  qkv l     raw q | k | v projections before the q/k norms -- fp16
  attn l    attention output before the output projection -- activation
            format (bf16 beside bf16 weights, fp16 beside quantized ones)
  mlp l     SiLU(gate) * up -- activation format

Each stage is held to the bar of the final outputs, 2e-2 per-row relative
error, and the per-stage errors are printed so the growth of the error
through the layers can be read off a run.
"""
import numpy as np
import pytest
import torch

from block_draft_model_pass_amd import _lib, synth
from block_draft_model_pass_amd.device import DeviceWeights, Drafter, KVRing, to_device
from oracle import dflash_oracle as O
from test_parity_gpu import TOL, check_draft, dec_bf16, dec_f16, row_rel_err, say

pytestmark = pytest.mark.gpu

L = synth.N_LAYERS


@pytest.fixture(scope="module")
def host_w():
    return synth.make_weights()


@pytest.fixture(scope="module")
def dev_w(host_w):
    return DeviceWeights(host_w)


@pytest.fixture(scope="module")
def ow(host_w):
    return O.enable_cache(dict(host_w))


def committed(dev_w, ow, n, cap, window):
    """Context positions 0..n-1 committed on both sides."""
    g = O.geometry(window=window)
    kv = KVRing(cap, window=window)
    dr = Drafter(dev_w, kv, max_rows=max(min(n, cap), 16))
    store = O.ContextStore(g)
    step = min(n, cap) if n else 1
    for s in range(0, n, step):
        e = min(n, s + step)
        taps = synth.make_taps(range(s, e))
        dr.commit(to_device(taps), s)
        store.put(*O.project_ctx_kv(ow, O.fuse_context(ow, taps), s), s)
    return g, kv, dr, store


def compare_stages(dr, rec, block, act_dec, tag):
    """Every stage of the last pass in dr's workspace against the oracle's
    record; returns {stage: [errors]}."""
    S = _lib
    errs = {"resid": [], "qkv": [], "attn": [], "mlp": []}
    for v in range(2 * L + 1):
        gv = dr.stage(S.DFLASH_STAGE_RESIDUAL, v, block).cpu().numpy().astype(np.float64)
        errs["resid"].append(row_rel_err(gv, rec["resid"][v]))
    for l in range(L):
        errs["qkv"].append(row_rel_err(dec_f16(dr.stage(S.DFLASH_STAGE_QKV, l, block)),
                                       rec["qkv"][l]))
        errs["attn"].append(row_rel_err(act_dec(dr.stage(S.DFLASH_STAGE_ATTN, l, block)),
                                        rec["attn"][l]))
        errs["mlp"].append(row_rel_err(act_dec(dr.stage(S.DFLASH_STAGE_MLP, l, block)),
                                       rec["mlp"][l]))
    for k, e in errs.items():
        say(f"[stages {tag}] {k:5s} " + " ".join(f"{x:.2e}" for x in e))
    for k, e in errs.items():
        assert max(e) <= TOL, (k, e)
    return errs


def staged_case(dev_w, ow, n, block, cap=32768, window=32768, act_dec=dec_bf16, tag=""):
    p = n
    say(f"[stages {tag}] ctx {n} block {block}")
    g, kv, dr, store = committed(dev_w, ow, n, cap, window)
    anchor = synth.anchor_token(p)
    cand = torch.empty(max(block - 1, 1), dtype=torch.int32, device="cuda")
    logits = torch.empty((max(block - 1, 1), dev_w.vocab), dtype=torch.int16, device="cuda")
    hidden = torch.empty((block, synth.HIDDEN), dtype=torch.int16, device="cuda")
    dr.draft(p, anchor, block, cand=cand, logits=logits, hidden=hidden)
    torch.cuda.synchronize()
    ck, cv = store.window(p)
    rec = {}
    ref = O.draft_block(ow, ck, cv, p, anchor, synth.MASK_ID, block, g, stages=rec)
    check_draft((cand[:max(block - 1, 1)], logits, hidden), ref, block, f"stages {tag}")
    return compare_stages(dr, rec, block, act_dec, tag)


@pytest.mark.parametrize("n,block", [(0, 1), (0, 8), (40, 8), (300, 5)])
def test_stages_bf16(dev_w, ow, n, block):
    staged_case(dev_w, ow, n, block, cap=1024, window=1024, tag=f"bf16 ctx{n} b{block}")


def test_stages_bf16_ctx8192_block8(dev_w, ow):
    """The timed shape: 8192 context cells, block 8."""
    staged_case(dev_w, ow, 8192, 8, tag="bf16 ctx8192 b8")


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "q5_0"])
def test_stages_quantized(fmt):
    host = synth.make_weights(fmt=fmt)
    dev = DeviceWeights(host)
    ow = O.enable_cache(dict(host))
    staged_case(dev, ow, 300, 4, cap=1024, window=1024, act_dec=dec_f16, tag=f"{fmt} ctx300 b4")
    del dev
    torch.cuda.empty_cache()


def test_stages_after_fused_commit(dev_w, ow):
    """The fused draft-commit call keeps the same stages: 5 commit rows at
    positions 300..304, then block 8 at p = 305."""
    n, nc, block = 300, 5, 8
    p = n + nc
    g, kv, dr, store = committed(dev_w, ow, n, 1024, 1024)
    ctaps = synth.make_taps(range(n, p))
    store.put(*O.project_ctx_kv(ow, O.fuse_context(ow, ctaps), n), n)
    anchor = synth.anchor_token(p)
    cand = torch.empty(block - 1, dtype=torch.int32, device="cuda")
    tg = to_device(ctaps)
    dr.draft_commit(tg.data_ptr(), nc, p, anchor, block, cand=cand)
    torch.cuda.synchronize()
    ck, cv = store.window(p)
    rec = {}
    O.draft_block(ow, ck, cv, p, anchor, synth.MASK_ID, block, g, stages=rec)
    compare_stages(dr, rec, block, dec_bf16, "fused 300+5 b8")


def test_stage_readout_errors(dev_w):
    """Argument checks of dflash_draft_stage on a live workspace."""
    dr = Drafter(dev_w, KVRing(256))
    dst = torch.empty(8 * 7680, dtype=torch.float32, device="cuda")
    S = _lib
    ok = S.dflash_draft_stage(dr.ws_ptr, dr.ws_bytes, S.DFLASH_STAGE_RESIDUAL, 10, 8,
                              dst.data_ptr(), dst.numel() * 4, None, check=False)
    assert ok == S.DFLASH_OK
    bad = [(S.DFLASH_STAGE_RESIDUAL, 11, 8), (S.DFLASH_STAGE_QKV, 5, 8), (4, 0, 8),
           (S.DFLASH_STAGE_MLP, 0, 9), (S.DFLASH_STAGE_MLP, 0, 0), (-1, 0, 1)]
    for st, idx, rows in bad:
        assert S.dflash_draft_stage(dr.ws_ptr, dr.ws_bytes, st, idx, rows, dst.data_ptr(),
                                    dst.numel() * 4, None, check=False) == S.DFLASH_EINVAL
    assert S.dflash_draft_stage(dr.ws_ptr, dr.ws_bytes, S.DFLASH_STAGE_RESIDUAL, 0, 8,
                                dst.data_ptr(), 8 * 2560 * 4 - 1, None,
                                check=False) == S.DFLASH_EINVAL
    assert S.dflash_draft_stage(dr.ws_ptr, 1024, S.DFLASH_STAGE_RESIDUAL, 0, 8,
                                dst.data_ptr(), dst.numel() * 4, None,
                                check=False) == S.DFLASH_EWORKSPACE
    torch.cuda.synchronize()
