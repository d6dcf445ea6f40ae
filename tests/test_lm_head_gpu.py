"""GPU parity of the standalone LM-head argmax (the candidate readout of a
block: logits = lm_head . hidden, greedy argmax with the lowest id on ties)
against the oracle, through both layouts the entry point reads: the
row-major bf16 matrix and its streaming copy.  Also checks that the
streaming copy holds exactly the layout the header documents.

Bars as for the draft pass: ids exact where the oracle's top-2 margin exceeds
0.05; bf16 logits within 2e-2 per-row relative error.
"""
import numpy as np
import pytest
import torch

from block_draft_model_pass_amd import _lib, synth
from block_draft_model_pass_amd.device import Drafter, KVRing, stream_ptr
from oracle import dflash_oracle as O
from test_parity_gpu import MARGIN, TOL, check_cands, dec_bf16, dev_w, host_w, ow, row_rel_err, say  # noqa: F401

pytestmark = pytest.mark.gpu

H = synth.HIDDEN


def lm_gpu(dev_w, packed: bool, z_bits: np.ndarray):
    """Run dflash_lm_head_argmax on bf16 rows z_bits with or without the
    streaming copy in the descriptor."""
    d = _lib.dflash_weights.from_buffer_copy(dev_w.desc)
    if not packed:
        d.packed = None
    rows = z_bits.shape[0]
    dr = Drafter(dev_w, KVRing(256))
    z = torch.from_numpy(z_bits.view(np.int16)).cuda()
    cand = torch.empty(rows, dtype=torch.int32, device="cuda")
    logits = torch.empty((rows, dev_w.vocab), dtype=torch.int16, device="cuda")
    _lib.dflash_lm_head_argmax(d, z.data_ptr(), rows, cand.data_ptr(), logits.data_ptr(),
                               dr.ws.data_ptr(), dr.ws_bytes, stream_ptr())
    torch.cuda.synchronize()
    return cand.cpu().numpy(), dec_bf16(logits)


@pytest.mark.parametrize("rows", [1, 5, 8])
@pytest.mark.parametrize("packed", [False, True], ids=["row_major", "streaming_copy"])
def test_lm_head_argmax(dev_w, ow, rows, packed):
    z_bits = synth.make_rows(rows, H, seed=91 + rows)
    cand, logits = lm_gpu(dev_w, packed, z_bits)
    ref = O.matvec_rows(ow, "lm_head", (dev_w.vocab, H), O.bf16_decode(z_bits))
    err = row_rel_err(logits, ref)
    ocand = np.array([O.argmax_lowest(r.astype(np.float32)) for r in ref])
    top2 = np.sort(ref.astype(np.float32), axis=1)[:, -2:]
    margin = top2[:, 1].astype(np.float64) - top2[:, 0]
    say(f"lm head rows={rows} packed={packed} logits err {err:.3e} cand {cand.tolist()} "
        f"ref {ocand.tolist()} margins {np.round(margin, 3).tolist()}")
    assert err <= TOL
    check_cands(cand, ocand, ref.astype(np.float32), margin)


def test_lm_head_layouts_agree_bitwise(dev_w):
    """Same sums in the same order from either layout: identical outputs."""
    z_bits = synth.make_rows(8, H, seed=7)
    c0, l0 = lm_gpu(dev_w, False, z_bits)
    c1, l1 = lm_gpu(dev_w, True, z_bits)
    assert np.array_equal(c0, c1)
    assert np.array_equal(l0, l1)


def packed_index(rows, cols, K):
    """Element index of (row, k) in a streaming copy of a [N][K] matrix."""
    unit = ((rows // 16) * (K // 32) + cols // 32) * 64 + (rows % 16) + 16 * ((cols % 32) // 8)
    return unit * 8 + cols % 8


def check_packed(packed, mat, rng, n_samples=20000):
    N, K = mat.shape
    row = np.concatenate([rng.integers(0, N, n_samples), [0, N - 1]])
    k = np.concatenate([rng.integers(0, K, n_samples), [0, K - 1]])
    assert np.array_equal(packed[packed_index(row, k, K)], mat[row, k])
    # whole first and last tiles
    for t in (0, N // 16 - 1):
        r = np.repeat(np.arange(16) + 16 * t, K)
        kk = np.tile(np.arange(K), 16)
        assert np.array_equal(packed[packed_index(r, kk, K)], mat[r, kk])


def test_streaming_copy_layout(dev_w, host_w):
    """Element (n, k) of each streamed matrix sits at 16-byte unit
    ((n/16) * (K/32) + k/32) * 64 + (n%16) + 16 * ((k%32)/8), element k%8;
    the LM head first, then layer by layer wq, wk, wv, wo, wg, wu, wd, then fc."""
    packed = dev_w.packed.view(torch.int16).cpu().numpy().view(np.uint16)
    rng = np.random.default_rng(3)
    V = dev_w.vocab
    shapes = [("wq", 6144, H), ("wk", 512, H), ("wv", 512, H), ("wo", H, 6144),
              ("wg", 7680, H), ("wu", 7680, H), ("wd", H, 7680)]
    layer_elems = sum(n * k for _, n, k in shapes)
    fc_off = V * H + 5 * layer_elems
    assert packed.size == fc_off + H * 5 * H
    check_packed(packed[:V * H], host_w["lm_head"].reshape(V, H), rng)
    for l in (0, 4):
        off = V * H + l * layer_elems
        for name, n, k in shapes:
            check_packed(packed[off:off + n * k], host_w[f"layers.{l}.{name}"].reshape(n, k), rng,
                         n_samples=4000)
            off += n * k
    check_packed(packed[fc_off:], host_w["fc"].reshape(H, 5 * H), rng, n_samples=4000)
