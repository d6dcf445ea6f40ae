"""GPU parity of the quantized backbone (Q8_0, Q4_0 and Q5_0 storage of fc and the
35 layer matrices; gains, embedding and LM head stay bf16) against the CPU
oracle, which decodes every block exactly (scale * q in fp64).

Same bars as the bf16 cases: ids exact where the oracle's top-2 margin
exceeds 0.05; logits, hidden states, fused context and fp16 K/V within 2e-2
per-row relative error.  The GPU decodes weights to fp16 (one rounding of
q * scale, relative 2^-11) for the MFMA paths and to bf16 for the many-row
GEMM path, well inside that bar.
"""
import numpy as np
import pytest
import torch

from block_draft_model_pass_amd import synth
from block_draft_model_pass_amd.device import DeviceWeights, Drafter, KVRing, to_device
from oracle import dflash_oracle as O
from test_parity_gpu import TOL, dec_bf16, end_to_end, ring_cells, row_rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", params=["q8_0", "q4_0", "q5_0"])
def qset(request):
    fmt = request.param
    say(f"quantized weights {fmt}")
    host = synth.make_weights(fmt=fmt)
    dev = DeviceWeights(host)
    ow = O.enable_cache(dict(host))
    yield fmt, dev, ow
    del dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n", [13, 300])
def test_quant_fuse_context(qset, n):
    """13 rows: skinny GEMV with in-register decode; 300 rows: decode to bf16
    then the MFMA GEMM."""
    fmt, dev, ow = qset
    taps = synth.make_taps(range(500, 500 + n))
    dr = Drafter(dev, KVRing(256), max_rows=n)
    ctx = dr.fuse(to_device(taps))
    torch.cuda.synchronize()
    err = row_rel_err(dec_bf16(ctx), O.bf16_decode(O.fuse_context(ow, taps)))
    say(f"[{fmt}] fuse n={n} rel err {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("n", [40, 300, 2200])  # 2200: cells from the GEMM's epilogue
def test_quant_project_ctx_kv(qset, n):
    fmt, dev, ow = qset
    pos0 = 1000
    ctx = synth.make_rows(n, synth.HIDDEN, seed=79)
    cap = 4096 if n > 2048 else 2048
    kv = KVRing(cap, window=cap)
    dr = Drafter(dev, kv, max_rows=n)
    dr.project(to_device(ctx), pos0)
    torch.cuda.synchronize()
    K, V = O.project_ctx_kv(ow, ctx, pos0)
    gK, gV = ring_cells(kv, range(pos0, pos0 + n))
    ek, ev = row_rel_err(gK, K), row_rel_err(gV, V)
    say(f"[{fmt}] project n={n} K err {ek:.3e} V err {ev:.3e}")
    assert ek <= TOL and ev <= TOL


@pytest.mark.parametrize("n,block", [(40, 4), (300, 8)])
def test_quant_draft(qset, n, block):
    """Context built on each side from its own fusion and projection (skinny
    path for 40 positions, GEMM path for 300), then one block."""
    fmt, dev, ow = qset
    end_to_end(dev, ow, n, block, tag=f"{fmt} ctx{n} b{block}")


def test_quant_draft_no_context(qset):
    fmt, dev, ow = qset
    end_to_end(dev, ow, 0, 8, tag=f"{fmt} ctx0 b8")


def test_quant_streaming_copy_layout(qset):
    """Packed quants and scales of wq and wd (layers 0 and 4) against the
    host bytes, by the layout the header documents: byte j of 64-byte piece
    kb of row n at ((n/16 * P + kb) * 64 + n%16 + 16 * (j/16)) * 16 + j%16;
    the S scales of piece kb of row n at ((n/16 * P + kb) * 16 + n%16) * S + s;
    Q5_0's high-bit words after them at ((n/16 * P + kb) * 16 + n%16) * 4 + s,
    the fifth bit of element 8 a + 4 b + c at bit 2 a + b + 8 c."""
    fmt, dev, _ = qset
    host = synth.make_weights(fmt=fmt)
    packed = dev.packed.cpu().numpy()
    H, V = synth.HIDDEN, dev.vocab
    shapes = [("wq", 6144, H), ("wk", 512, H), ("wv", 512, H), ("wo", H, 6144),
              ("wg", 7680, H), ("wu", 7680, H), ("wd", H, 7680)]
    qb = (lambda n, k: n * k) if fmt == "q8_0" else (lambda n, k: n * k // 2)
    hb = 4 if fmt == "q5_0" else 0  # high-bit word bytes per block
    mat_bytes = {name: qb(n, k) + n * (k // 32) * (2 + hb) for name, n, k in shapes}
    layer_bytes = sum(mat_bytes.values())
    rng = np.random.default_rng(11)
    for l in (0, 4):
        off = 2 * V * H + l * layer_bytes
        for name, n, k in shapes:
            raw = host[f"layers.{l}.{name}"].view(np.uint8)
            mb = mat_bytes[name]
            if name in ("wq", "wd"):
                got = packed[off:off + mb]
                rowb = qb(n, k) // n  # quant bytes per row
                P = rowb // 64
                rows = rng.integers(0, n, 3000)
                js = rng.integers(0, rowb, 3000)
                kb, j = js // 64, js % 64
                idx = ((rows // 16 * P + kb) * 64 + rows % 16 + 16 * (j // 16)) * 16 + j % 16
                assert np.array_equal(got[idx], raw[rows * rowb + js])
                S = 2 if fmt == "q8_0" else 4
                ns = n * (k // 32)
                scales = raw[qb(n, k):qb(n, k) + 2 * ns].view(np.uint16).reshape(n, k // 32)
                gs = got[qb(n, k):qb(n, k) + 2 * ns].view(np.uint16)
                rows = rng.integers(0, n, 3000)
                blk = rng.integers(0, k // 32, 3000)
                kb, sidx = blk // S, blk % S
                assert np.array_equal(gs[((rows // 16 * P + kb) * 16 + rows % 16) * S + sidx],
                                      scales[rows, blk])
                if hb:
                    sq = qb(n, k) + n * (k // 32) * 2
                    words = raw[sq:].view("<u4").reshape(n, k // 32)
                    gw = got[sq:].view("<u4")
                    at = ((rows // 16 * P + kb) * 16 + rows % 16) * S + sidx
                    for e in range(32):
                        a, b, c = e >> 3, (e >> 2) & 1, e & 3
                        assert np.array_equal((gw[at] >> (2 * a + b + 8 * c)) & 1,
                                              (words[rows, blk] >> e) & 1), e
            off += mb
    assert packed.size == 2 * V * H + 5 * layer_bytes + qb(H, 5 * H) + H * (5 * H // 32) * (2 + hb)
