"""GPU test of the device-resident decode cycle captured in a HIP graph.

With {p, anchor, n_commit} in device words (dflash_draft_block_commit_dev +
dflash_verify_greedy_advance) a whole cycle -- the fused draft-commit pass,
the stand-in target built from the candidates and the verify that advances
the state -- has no host round trip, so it can be captured once and replayed
(the pages' graph-replayed drafting windows, PR #3322 "Draft attention fix
(2026-10-20)"; the persistent-cycle row of the speculative-decode
integration, PR #1426 "Speculative decode integration").

The graph is replayed once per cycle, with the host refreshing the stand-in
target's draws (eager copies) and synchronising between replays; every
replay's candidates, logits and hidden states, the final ring cells and the
final state must equal, bit for bit, the same cycles run eagerly.  The graph
holds no memset node: the pass's init kernel clears the barrier words.
"""
import pytest
import torch

from block_draft_model_pass_amd import _lib, synth
from block_draft_model_pass_amd.device import DeviceWeights
from test_device_cycle_gpu import B, K, outputs, setup, stand_in_target, targets
from test_parity_gpu import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev_w():
    return DeviceWeights(synth.make_weights())


def eager_cycles(dev_w, ctx0, cap, cycles, match, offset, tail):
    kv, dr, taps = setup(dev_w, ctx0, cap, cycles * B + B)
    state = torch.tensor([ctx0, synth.anchor_token(0), 0], dtype=torch.int64, device="cuda")
    out = torch.empty(2, dtype=torch.int32, device="cuda")
    res = []
    for t in range(cycles):
        c, lg, hd = outputs(dev_w.vocab)
        dr.draft_commit_dev(taps, ctx0, state, B, cand=c, logits=lg, hidden=hd)
        tgt = stand_in_target(c, t, match, offset, tail, dev_w.vocab)
        dr.verify_advance(c, tgt, K, state, out=out)
        res.append((c, lg, hd, out.clone()))
    torch.cuda.synchronize()
    return kv, state, res


@pytest.mark.parametrize("ctx0,cycles", [(1024, 6), (8192, 5)])
def test_graph_replayed_cycle_equals_eager(dev_w, ctx0, cycles):
    say(f"[graph cycle] ctx0 {ctx0} cycles {cycles}")
    cap = 32768 if ctx0 > 1024 else 2048
    match, offset, tail = targets(cycles)
    kv_e, state_e, ref = eager_cycles(dev_w, ctx0, cap, cycles, match, offset, tail)

    kv, dr, taps = setup(dev_w, ctx0, cap, cycles * B + B)
    state = torch.tensor([ctx0, synth.anchor_token(0), 0], dtype=torch.int64, device="cuda")
    cand, logits, hidden = outputs(dev_w.vocab)
    m_cur = torch.empty_like(match[0])
    o_cur = torch.empty_like(offset[0])
    tail_cur = torch.empty(1, dtype=torch.int32, device="cuda")
    tgt = torch.empty(K + 1, dtype=torch.int32, device="cuda")
    out = torch.empty(2, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dr.draft_commit_dev(taps, ctx0, state, B, cand=cand, logits=logits, hidden=hidden)
        torch.where(m_cur, cand, torch.remainder(cand + o_cur, dev_w.vocab), out=tgt[:K])
        tgt[K:].copy_(tail_cur)
        dr.verify_advance(cand, tgt, K, state, out=out)
    # capturing ran nothing: the state and the ring are as set up
    torch.cuda.synchronize()
    assert state.cpu().tolist() == [ctx0, synth.anchor_token(0), 0]
    st = torch.empty(1, dtype=torch.int32, device="cuda")
    for t in range(cycles):
        m_cur.copy_(match[t])
        o_cur.copy_(offset[t])
        tail_cur.copy_(tail[t:t + 1])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        c, lg, hd, o = ref[t]
        say(f"[graph cycle] replay {t}: state {state.cpu().tolist()} out {out.cpu().tolist()}")
        assert torch.equal(cand, c), f"candidates, replay {t}"
        assert torch.equal(logits, lg), f"logits, replay {t}"
        assert torch.equal(hidden, hd), f"hidden states, replay {t}"
        assert torch.equal(out, o), f"accepted / next token, replay {t}"
        _lib.dflash_draft_status(dr.ws_ptr, dr.ws_bytes, st.data_ptr(), None)
        torch.cuda.synchronize()
        assert int(st.item()) == _lib.DFLASH_OK
    assert torch.equal(state, state_e)
    assert torch.equal(kv.k, kv_e.k) and torch.equal(kv.vt, kv_e.vt)
