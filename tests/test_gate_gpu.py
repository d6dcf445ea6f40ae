"""GPU parity of the confidence-gated proposal pass (dflash_draft_block_gated)
against the oracle's candidate_confidence / gate_candidates.

Bars:
  * cand: bit-equal to dflash_draft_block's on the same inputs (same kernel,
    same fp32 logits), and to the oracle's under the margin rule of the
    other parity tests;
  * conf: log conf = max_v l_v - logsumexp(l).  With d_v a bound on the
    GPU's fp32 logit error (observed |bf16 logit - oracle| plus the bf16
    rounding |l_v| 2^-8), the max moves by at most max(d_c, d_c') over the
    oracle's and the GPU's argmax, and logsumexp by at most
    sum_v p_v d_v + max_v d_v^2 / 2 (first order with the oracle's softmax p,
    plus the bound on its Taylor remainder, whose Hessian diag(p) - p p^T has
    quadratic form <= max d^2); the row's bar is their sum;
  * n_keep: equal to the gate applied to the GPU's own conf (the decision is
    taken in the kernel's fp32) for floors between the GPU's values, and to
    the oracle's gate for floors farther than the largest bar (in log) from
    every oracle conf.
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

MARGIN = 0.05


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def host_w():
    return synth.make_weights()


@pytest.fixture(scope="module")
def dev_w(host_w):
    return DeviceWeights(host_w)


@pytest.fixture(scope="module")
def ow(host_w):
    return O.enable_cache(dict(host_w))


def dec_bf16(t: torch.Tensor) -> np.ndarray:
    u = t.cpu().numpy().astype(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def floors_from(conf_ref, bar):
    """Floors at 0, above 1, and between consecutive oracle confidences
    (log-midpoints), skipping any within the conf bar of an oracle value."""
    out = [0.0, 1.0]
    c = np.sort(np.asarray(conf_ref))
    for lo, hi in zip(c[:-1], c[1:]):
        f = math.exp(0.5 * (math.log(lo) + math.log(hi)))
        if all(abs(math.log(f) - math.log(x)) > bar for x in c):
            out.append(f)
    for x in c:  # just above and below each value, where the bar allows
        for f in (x * math.exp(2 * bar), x * math.exp(-2 * bar)):
            if 0.0 < f <= 1.0 and all(abs(math.log(f) - math.log(y)) > bar for y in c):
                out.append(f)
    return out


@pytest.mark.parametrize("n,block,cap,window", [(0, 2, 256, 256), (40, 5, 1024, 1024),
                                                (1500, 8, 1024, 512), (300, 8, 32768, 32768)])
def test_gated_pass_matches_oracle(dev_w, ow, n, block, cap, window):
    gate_case(dev_w, ow, n, block, cap, window)


def test_gated_pass_with_peaked_distributions(host_w, ow):
    """Synthetic weights give nearly flat next-token distributions (conf near
    3e-4).  Scaling the final-norm gain by 6 on both sides scales every logit
    by 6, so the candidates' probabilities spread over orders of magnitude
    and floors between them cut the proposal part-way."""
    g = (host_w["final_norm"].astype(np.uint32) << 16).view(np.float32)
    hw = dict(host_w)
    hw["final_norm"] = synth.bf16_bits_from_f32(g * 6.0)
    ow2 = dict(ow)  # shares the decoded-matrix cache; the gain is decoded per call
    ow2["final_norm"] = hw["final_norm"]
    dw = DeviceWeights(hw)
    keeps = gate_case(dw, ow2, 40, 8, 1024, 1024)
    say(f"[gate peaked] n_keep over the floors: {sorted(set(keeps))}")


def gate_case(dev_w, ow, n, block, cap, window):
    p = n
    say(f"[gate] n={n} block={block} cap={cap} window={window}")
    g = O.geometry(window=window)
    kv = KVRing(cap, window=window)
    dr = Drafter(dev_w, kv, max_rows=min(n, cap) if n else 16)
    store = O.ContextStore(g)
    step = min(n, cap) if n else 1
    for s in range(0, n, step):
        e = min(n, s + step)
        taps = synth.make_taps(range(s, e))
        dr.commit(to_device(taps), s)
        store.put(*O.project_ctx_kv(ow, O.fuse_context(ow, taps), s), s)
    anchor = synth.anchor_token(p)
    K = block - 1
    # the plain pass, with logits, for cand identity and the logit error
    cand0 = torch.empty(K, dtype=torch.int32, device="cuda")
    logits = torch.empty((K, dev_w.vocab), dtype=torch.int16, device="cuda")
    dr.draft(p, anchor, block, cand=cand0, logits=logits)
    torch.cuda.synchronize()
    ck, cv = store.window(p)
    ref = O.draft_block(ow, ck, cv, p, anchor, synth.MASK_ID, block, g)
    lg = dec_bf16(logits)
    lo = ref["logits"]
    d = np.abs(lg - lo) + np.abs(lg) * 2.0 ** -8
    pr = np.exp(lo - lo.max(axis=1, keepdims=True))
    pr /= pr.sum(axis=1, keepdims=True)
    c0 = cand0.cpu().numpy()
    bars = np.array([max(d[i, ref["cand"][i]], d[i, c0[i]]) + (pr[i] * d[i]).sum()
                     + 0.5 * d[i].max() ** 2 + 1e-5 for i in range(K)])  # + fp32 sums
    bar = float(bars.max())
    floors = floors_from(ref["conf"], bar)
    say(f"[gate] max logit err {np.abs(lg - lo).max():.3e}, conf bars (log) "
        f"{np.array2string(bars, precision=3)}, oracle conf "
        f"{np.array2string(ref['conf'], precision=4)}")
    keeps = []
    for f in floors:
        cand, conf, nk = dr.draft_gated(p, anchor, block, float(f))
        torch.cuda.synchronize()
        c = cand.cpu().numpy()
        cf = conf.cpu().numpy().astype(np.float64)
        k = int(nk.cpu().item())
        assert np.array_equal(c, cand0.cpu().numpy()), (c, cand0)
        sure = ref["margin"] > MARGIN
        assert np.array_equal(c[sure], ref["cand"][sure]), (c, ref["cand"], ref["margin"])
        assert np.all(np.isfinite(cf)) and np.all(cf > 0) and np.all(cf <= 1.0)
        err = np.abs(np.log(cf) - np.log(ref["conf"]))
        assert np.all(err <= bars), (f, cf, ref["conf"], err, bars)
        assert k == O.gate_candidates(cf, f), (f, cf, k)
        assert k == O.gate_candidates(ref["conf"], f), (f, cf, ref["conf"], k)
        keeps.append(k)
    # floors between the GPU's own values: the decision in kernel precision
    cs = np.sort(cf)
    for f in [math.sqrt(a * b) for a, b in zip(cs[:-1], cs[1:]) if b > a]:
        _, conf, nk = dr.draft_gated(p, anchor, block, float(f))
        torch.cuda.synchronize()
        k = int(nk.cpu().item())
        assert k == O.gate_candidates(conf.cpu().numpy().astype(np.float64), f), (f, conf, k)
        keeps.append(k)
    say(f"[gate] {len(floors)} oracle floors and {len(cs) - 1} gpu floors checked, gpu conf "
        f"{np.array2string(cf, precision=4)}")
    return keeps


def test_gated_pass_at_full_context_size(dev_w):
    """Context 8192, block 8, with the launch the decode cycle uses: the
    gated pass gives the plain pass's candidates, and its conf equals the
    softmax probability of the candidate computed on the CPU from the same
    pass's logits within the bf16 rounding of those logits."""
    kv = KVRing(32768)
    dr = Drafter(dev_w, kv, max_rows=8192)
    taps = synth.make_taps(range(0, 8192))
    dr.commit(to_device(taps), 0)
    p, block = 8192, 8
    anchor = synth.anchor_token(p)
    cand0 = torch.empty(block - 1, dtype=torch.int32, device="cuda")
    logits = torch.empty((block - 1, dev_w.vocab), dtype=torch.int16, device="cuda")
    dr.draft(p, anchor, block, cand=cand0, logits=logits)
    cand, conf, nk = dr.draft_gated(p, anchor, block, 0.5)
    torch.cuda.synchronize()
    assert np.array_equal(cand.cpu().numpy(), cand0.cpu().numpy())
    lg = dec_bf16(logits)
    cf = conf.cpu().numpy().astype(np.float64)
    want = np.array([O.candidate_confidence(r) for r in lg])
    bar = 2.0 * np.abs(lg).max() * 2.0 ** -8 + 1e-5  # bf16 rounding, fp32 sums
    err = np.abs(np.log(cf) - np.log(want))
    say(f"[gate 8192] conf {np.array2string(cf, precision=4)} err {err.max():.3e} bar {bar:.3e}")
    assert err.max() <= bar
    assert int(nk.cpu().item()) == O.gate_candidates(cf, 0.5)


def test_gated_timeout_reports_nan_and_zero(dev_w, monkeypatch):
    """A pass whose barriers give up waiting (wall-clock bound forced from the
    host to 0) reports cand -1, conf NaN and n_keep 0; the next pass is whole."""
    kv = KVRing(256)
    dr = Drafter(dev_w, kv)
    monkeypatch.setenv("DFLASH_BARRIER_TIMEOUT_US", "0")
    cand, conf, nk = dr.draft_gated(100, 11, 8, 0.0)
    torch.cuda.synchronize()
    monkeypatch.delenv("DFLASH_BARRIER_TIMEOUT_US")
    c, cf, k = cand.cpu().numpy().copy(), conf.cpu().numpy().copy(), int(nk.cpu().item())
    cand2, conf2, nk2 = dr.draft_gated(100, 11, 8, 0.0)
    torch.cuda.synchronize()
    say(f"[gate timeout] cand {c.tolist()} conf {cf.tolist()} n_keep {k}")
    assert (c == -1).all() and np.isnan(cf).all() and k == 0
    assert (cand2.cpu().numpy() >= 0).all() and int(nk2.cpu().item()) == 7
