"""GPU tests of the decode cycle with device-resident positions
(dflash_draft_block_commit_dev + dflash_verify_greedy_advance): the pass
reads p, the anchor and the commit count from device words that the verify
advances, so a cycle needs no device-to-host read.

The same cycles driven from the host (dflash_draft_block_commit with the
positions as arguments, dflash_verify_greedy) must give bit-identical
candidates, logits, hidden states and ring cells -- the kernels are the
same, only where the positions come from differs -- and the candidates are
compared with the oracle's decode loop as in the fused-cycle tests.
Invalid device states must leave the ring untouched and report
DFLASH_EINVAL through the pass status word.
"""
import numpy as np
import pytest
import torch

from block_draft_model_pass_amd import _lib, synth
from block_draft_model_pass_amd.device import DeviceWeights, Drafter, KVRing, to_device
from oracle import dflash_oracle as O
from test_parity_gpu import check_draft, ring_cells, say

pytestmark = pytest.mark.gpu

B = 8
K = B - 1


@pytest.fixture(scope="module")
def host_w():
    return synth.make_weights()


@pytest.fixture(scope="module")
def dev_w(host_w):
    return DeviceWeights(host_w)


@pytest.fixture(scope="module")
def ow(host_w):
    return O.enable_cache(dict(host_w))


def outputs(vocab):
    return (torch.empty(K, dtype=torch.int32, device="cuda"),
            torch.empty((K, vocab), dtype=torch.int16, device="cuda"),
            torch.empty((B, synth.HIDDEN), dtype=torch.int16, device="cuda"))


def setup(dev_w, ctx0, cap, span):
    kv = KVRing(cap, window=cap)
    dr = Drafter(dev_w, kv, max_rows=min(ctx0, 2048) if ctx0 else 16)
    for s0 in range(0, ctx0, 2048):
        dr.commit(to_device(synth.make_taps(range(s0, min(ctx0, s0 + 2048)))), s0)
    taps = to_device(synth.make_taps(range(ctx0, ctx0 + span)))
    return kv, dr, taps


def targets(cycles):
    draws = [synth.target_draws(t, K) for t in range(cycles)]
    match = torch.tensor(np.stack([d[0] for d in draws]), device="cuda")
    offset = torch.tensor(np.stack([d[1] for d in draws]) + 1, dtype=torch.int32, device="cuda")
    tail = torch.tensor([d[2] for d in draws], dtype=torch.int32, device="cuda")
    return match, offset, tail


def stand_in_target(cand, t, match, offset, tail, vocab):
    """The bench's stand-in target, built on the device from the candidates."""
    tgt = torch.empty(K + 1, dtype=torch.int32, device="cuda")
    torch.where(match[t], cand, torch.remainder(cand + offset[t], vocab), out=tgt[:K])
    tgt[K] = tail[t]
    return tgt


@pytest.mark.parametrize("ctx0,cycles", [(1024, 12), (8192, 10)])
def test_device_cycle_equals_host_cycle(dev_w, ow, ctx0, cycles):
    """`cycles` decode cycles from ctx0, once with the positions on the host
    and once in device words; every cycle's outputs and the final ring cells
    are bit-identical, and the host cycle is compared with the oracle."""
    say(f"[device cycle] ctx0 {ctx0} cycles {cycles}")
    span = cycles * B + B
    cap = 32768 if ctx0 > 1024 else 2048
    match, offset, tail = targets(cycles)
    anchor0 = synth.anchor_token(0)
    # host-driven
    kv_h, dr_h, taps_h = setup(dev_w, ctx0, cap, span)
    row = taps_h.stride(0) * taps_h.element_size()
    p, anchor, n = ctx0, anchor0, 0
    host_out, host_pos = [], []
    out = torch.empty(2, dtype=torch.int32, device="cuda")
    for t in range(cycles):
        c, lg, hd = outputs(dev_w.vocab)
        ptr = taps_h.data_ptr() + (p - n - ctx0) * row if n else None
        dr_h.draft_commit(ptr, n, p, anchor, B, cand=c, logits=lg, hidden=hd)
        tgt = stand_in_target(c, t, match, offset, tail, dev_w.vocab)
        dr_h.verify(c, tgt, K, out=out)
        a, nxt = out.cpu().tolist()
        host_out.append((c.clone(), lg.clone(), hd.clone()))
        host_pos.append((p, anchor, n))
        p, anchor, n = p + a + 1, nxt, a + 1
    torch.cuda.synchronize()
    # device-driven: no host read inside the loop
    kv_d, dr_d, taps_d = setup(dev_w, ctx0, cap, span)
    state = torch.tensor([ctx0, anchor0, 0], dtype=torch.int64, device="cuda")
    outs = torch.empty((cycles, 2), dtype=torch.int32, device="cuda")
    dev_out = []
    for t in range(cycles):
        c, lg, hd = outputs(dev_w.vocab)
        dr_d.draft_commit_dev(taps_d, ctx0, state, B, cand=c, logits=lg, hidden=hd)
        tgt = stand_in_target(c, t, match, offset, tail, dev_w.vocab)
        dr_d.verify_advance(c, tgt, K, state, out=outs[t])
        dev_out.append((c, lg, hd))
    st = torch.empty(1, dtype=torch.int32, device="cuda")
    _lib.dflash_draft_status(dr_d.ws_ptr, dr_d.ws_bytes, st.data_ptr(), None)
    torch.cuda.synchronize()
    assert int(st.item()) == _lib.DFLASH_OK
    for t in range(cycles):
        for g, h in zip(dev_out[t], host_out[t]):
            assert torch.equal(g, h), f"cycle {t}"
    assert state.cpu().tolist() == [p, anchor, n]
    assert torch.equal(kv_d.k, kv_h.k) and torch.equal(kv_d.vt, kv_h.vt)
    # the host-driven cycles against the oracle (first, middle and last)
    store = O.ContextStore()
    for s0 in range(0, ctx0, 2048):
        taps = synth.make_taps(range(s0, min(ctx0, s0 + 2048)))
        store.put(*O.project_ctx_kv(ow, O.fuse_context(ow, taps), s0), s0)
    for t in range(cycles):
        pt, at, nt = host_pos[t]
        if nt:
            ctaps = synth.make_taps(range(pt - nt, pt))
            store.put(*O.project_ctx_kv(ow, O.fuse_context(ow, ctaps), pt - nt), pt - nt)
        if t in (0, cycles // 2, cycles - 1):
            ck, cv = store.window(pt)
            ref = O.draft_block(ow, ck, cv, pt, at, synth.MASK_ID, B)
            check_draft(dev_out[t], ref, B, f"device cycle t={t} p={pt}")
    say(f"[device cycle] final state {state.cpu().tolist()}")


def test_device_state_checks(dev_w):
    """States the host entry points would refuse: the pass reads nothing from
    them, leaves the ring untouched, writes cand = -1 and reports
    DFLASH_EINVAL; a valid state afterwards runs normally."""
    ctx0 = 256
    kv, dr, taps = setup(dev_w, ctx0, 1024, 32)
    V = dev_w.vocab
    bad = [
        (ctx0, 5, 9),             # n_commit > 8
        (3, 5, 4),                # p < n_commit
        (ctx0 + 4, V, 4),         # anchor outside the vocabulary
        (ctx0 + 4, -1, 4),        # negative anchor
        (ctx0 + 40, 5, 4),        # commit rows past the taps buffer
        (ctx0 - 1, 5, 2),         # commit rows before the taps buffer
        (-8, 5, 0),               # negative position
    ]
    k0, v0 = kv.k.clone(), kv.vt.clone()
    st = torch.empty(1, dtype=torch.int32, device="cuda")
    for p, anchor, n in bad:
        state = torch.tensor([p, anchor, n], dtype=torch.int64, device="cuda")
        cand = torch.zeros(K, dtype=torch.int32, device="cuda")
        dr.draft_commit_dev(taps, ctx0, state, B, cand=cand)
        _lib.dflash_draft_status(dr.ws_ptr, dr.ws_bytes, st.data_ptr(), None)
        torch.cuda.synchronize()
        say(f"[device state] {p, anchor, n}: status {int(st.item())} cand {cand.tolist()}")
        assert int(st.item()) == _lib.DFLASH_EINVAL
        assert cand.tolist() == [-1] * K
        assert torch.equal(kv.k, k0) and torch.equal(kv.vt, v0)
    # the edges that are valid: all 32 rows of taps, n_commit 8, p == n_commit
    for p, n in ((ctx0 + 32, 8), (ctx0 + 8, 8)):
        state = torch.tensor([p, 5, n], dtype=torch.int64, device="cuda")
        cand = torch.zeros(K, dtype=torch.int32, device="cuda")
        dr.draft_commit_dev(taps, ctx0, state, B, cand=cand)
        _lib.dflash_draft_status(dr.ws_ptr, dr.ws_bytes, st.data_ptr(), None)
        torch.cuda.synchronize()
        assert int(st.item()) == _lib.DFLASH_OK
        assert min(cand.tolist()) >= 0
    kv2, dr2, taps2 = setup(dev_w, 0, 1024, 8)
    state = torch.tensor([8, 5, 8], dtype=torch.int64, device="cuda")
    cand = torch.zeros(K, dtype=torch.int32, device="cuda")
    dr2.draft_commit_dev(taps2, 0, state, B, cand=cand)
    _lib.dflash_draft_status(dr2.ws_ptr, dr2.ws_bytes, st.data_ptr(), None)
    torch.cuda.synchronize()
    assert int(st.item()) == _lib.DFLASH_OK and min(cand.tolist()) >= 0


def test_verify_advance_updates_state(dev_w):
    """accepted a, next token t: p += a + 1, anchor = t, n_commit = a + 1;
    out = {a, t} as dflash_verify_greedy writes it."""
    dr = Drafter(dev_w, KVRing(256))
    cases = [([3, 4, 5, 6, 7, 8, 9], [3, 4, 5, 0, 7, 8, 9, 11], 3, 0),
             ([3, 4, 5, 6, 7, 8, 9], [3, 4, 5, 6, 7, 8, 9, 12], 7, 12),
             ([3, 4, 5, 6, 7, 8, 9], [1, 4, 5, 6, 7, 8, 9, 12], 0, 1)]
    for cand, tgt, a, nxt in cases:
        state = torch.tensor([1000, 77, 3], dtype=torch.int64, device="cuda")
        c = torch.tensor(cand, dtype=torch.int32, device="cuda")
        t = torch.tensor(tgt, dtype=torch.int32, device="cuda")
        out = dr.verify_advance(c, t, K, state)
        torch.cuda.synchronize()
        assert out.tolist() == [a, nxt]
        assert state.tolist() == [1000 + a + 1, nxt, a + 1]
        assert (a, nxt) == O.verify_greedy(np.array(cand), np.array(tgt))
