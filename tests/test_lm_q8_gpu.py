"""GPU parity of the Q8_0 shared LM head (PR #3322 later snapshot, "How to
enable the pushed optimization options": the Q8_0 shared-head kernel;
"Current implementation and speed comparison": a full shared Q8_0 head)
against the oracle, which decodes every block exactly (scale * q in fp64).

The GPU decodes each block to fp16 in registers (one rounding of q * scale)
and takes the contraction against fp16 final-normed activations on MFMA f16,
accumulating in fp32.  Bars as everywhere: ids exact where the oracle's top-2
margin exceeds 0.05, logits and hidden states within 2e-2 per-row relative
error; the gated pass's conf within the bound its logit error allows.
"""
import numpy as np
import pytest
import torch

from block_draft_model_pass_amd import _lib, synth
from block_draft_model_pass_amd.device import DeviceWeights, Drafter, KVRing, stream_ptr
from oracle import dflash_oracle as O
from test_parity_full_gpu import conf_bars
from test_parity_gpu import TOL, check_cands, dec_bf16, end_to_end, row_rel_err, say

pytestmark = pytest.mark.gpu

H = synth.HIDDEN


@pytest.fixture(scope="module")
def q8lm():
    """bf16 backbone, Q8_0 LM head."""
    host = synth.make_weights(lm_fmt="q8_0")
    dev = DeviceWeights(host)
    ow = O.enable_cache(dict(host))
    yield host, dev, ow
    del dev
    torch.cuda.empty_cache()


def test_q8_lm_head_streaming_copy_layout(q8lm):
    """The LM head's Q8_0 streaming copy: byte j of 64-byte piece kb of row n
    at ((n/16 * 40 + kb) * 64 + n%16 + 16 * (j/16)) * 16 + j%16, the two
    scales of piece kb of row n at ((n/16 * 40 + kb) * 16 + n%16) * 2 + s;
    the layer matrices follow it."""
    host, dev, _ = q8lm
    V = dev.vocab
    raw = host["lm_head"]
    packed = dev.packed.cpu().numpy()
    qb = V * H
    rng = np.random.default_rng(5)
    rows = np.concatenate([rng.integers(0, V, 20000), [0, V - 1]])
    js = np.concatenate([rng.integers(0, H, 20000), [0, H - 1]])
    kb, j = js // 64, js % 64
    idx = ((rows // 16 * 40 + kb) * 64 + rows % 16 + 16 * (j // 16)) * 16 + j % 16
    assert np.array_equal(packed[idx], raw[rows * H + js])
    scales = raw[qb:].view(np.uint16).reshape(V, H // 32)
    gs = packed[qb:qb + V * (H // 32) * 2].view(np.uint16)
    blk = rng.integers(0, H // 32, 20000)
    rows = rng.integers(0, V, 20000)
    assert np.array_equal(gs[((rows // 16 * 40 + blk // 2) * 16 + rows % 16) * 2 + blk % 2],
                          scales[rows, blk])
    assert packed.size == _lib.dflash_packed_size(dev.desc)


@pytest.mark.parametrize("packed", [False, True], ids=["row_major", "streaming_copy"])
def test_q8_lm_head_argmax(q8lm, packed):
    """dflash_lm_head_argmax on 8 rows, from the row-major blocks and from the
    streaming copy (same sums in the same order: identical outputs)."""
    host, dev, ow = q8lm
    outs = []
    for pk in (packed, not packed):
        d = _lib.dflash_weights.from_buffer_copy(dev.desc)
        if not pk:
            d.packed = None
        z_bits = synth.make_rows(8, H, seed=123)
        dr = Drafter(dev, KVRing(256))
        z = torch.from_numpy(z_bits.view(np.int16)).cuda()
        cand = torch.empty(8, dtype=torch.int32, device="cuda")
        logits = torch.empty((8, dev.vocab), dtype=torch.int16, device="cuda")
        _lib.dflash_lm_head_argmax(d, z.data_ptr(), 8, cand.data_ptr(), logits.data_ptr(),
                                   dr.ws.data_ptr(), dr.ws_bytes, stream_ptr())
        torch.cuda.synchronize()
        outs.append((cand.cpu().numpy(), dec_bf16(logits)))
    cand, lg = outs[0]
    ref = O.matvec_rows(ow, "lm_head", (dev.vocab, H), O.bf16_decode(z_bits))
    err = row_rel_err(lg, ref)
    ocand = np.array([O.argmax_lowest(r.astype(np.float32)) for r in ref])
    top2 = np.sort(ref.astype(np.float32), axis=1)[:, -2:]
    margin = top2[:, 1].astype(np.float64) - top2[:, 0]
    say(f"[q8 lm head] packed={packed} logits err {err:.3e} cand {cand.tolist()} ref {ocand.tolist()}")
    assert err <= TOL
    check_cands(cand, ocand, ref.astype(np.float32), margin)
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("n,block", [(0, 2), (40, 8), (300, 5)])
def test_q8_lm_head_draft(q8lm, n, block):
    host, dev, ow = q8lm
    end_to_end(dev, ow, n, block, cap=1024, window=1024, tag=f"q8 lm ctx{n} b{block}")


def test_q8_lm_head_draft_ctx8192_block8_and_gate(q8lm):
    """The timed shape: 8192 cells, block 8, bf16 backbone, Q8_0 LM head;
    the gated pass gives the same ids and conf within its bar."""
    host, dev, ow = q8lm
    (cand, logits, _), ref = end_to_end(dev, ow, 8192, 8, tag="q8 lm ctx8192 b8")
    kv_dr = None
    c = cand.cpu().numpy()
    # the same pass through the gate (the ring built by end_to_end is gone;
    # rebuild it the same way)
    kv = KVRing(32768)
    kv_dr = Drafter(dev, kv, max_rows=8192)
    kv_dr.commit(torch.from_numpy(synth.make_taps(range(8192)).view(np.int16)).cuda(), 0)
    gc, gconf, nk = kv_dr.draft_gated(8192, synth.anchor_token(8192), 8, 0.0)
    torch.cuda.synchronize()
    assert np.array_equal(gc.cpu().numpy(), c)
    bars = conf_bars(dec_bf16(logits), ref, c)
    err = np.abs(np.log(gconf.cpu().numpy().astype(np.float64)) - np.log(ref["conf"]))
    say(f"[q8 lm gate] conf err {err.max():.3e} bars {bars.max():.3e}")
    assert np.all(err <= bars)
    assert int(nk.cpu().item()) == 7


def test_q8_backbone_and_q8_lm_head_ctx8192_block4():
    """Every streamed matrix in Q8_0 (fc, the 35 layer matrices and the LM
    head): 8192 cells, block 4."""
    host = synth.make_weights(fmt="q8_0", lm_fmt="q8_0")
    dev = DeviceWeights(host)
    ow = O.enable_cache(dict(host))
    end_to_end(dev, ow, 8192, 4, tag="q8+q8 lm ctx8192 b4")
    del dev
    torch.cuda.empty_cache()


def test_q8_lm_head_packed_only(q8lm):
    """Row-major LM head released after packing: the pass and the standalone
    argmax read the Q8_0 streaming copy."""
    host, _, ow = q8lm
    dev = DeviceWeights(host, packed_only=True)
    (cand, _, hidden), ref = end_to_end(dev, ow, 40, 8, cap=1024, window=1024,
                                        tag="q8 lm packed-only")
    dr = Drafter(dev, KVRing(256))
    zc = torch.empty(7, dtype=torch.int32, device="cuda")
    dr.lm_head_argmax(hidden[1:].contiguous(), zc)
    torch.cuda.synchronize()
    check_cands(zc.cpu().numpy(), ref["cand"], ref["logits"], ref["margin"])
    del dev
    torch.cuda.empty_cache()
