"""dflash_draft_block_static -- the proposal pass with its workspace in the
library's own device array, for callers that cannot allocate -- against
dflash_draft_block with a caller-owned workspace, through the C ABI: the same
kernels run on the same inputs, so candidates, logits and hidden states must
be bit-identical.  Two calls in a row, the second with a smaller input
(shorter context, smaller block), so that the second reuses the array the
first left behind."""
import numpy as np
import pytest
import torch

from block_draft_model_pass_amd import _lib, synth
from block_draft_model_pass_amd.device import (DeviceWeights, Drafter, KVRing, stream_ptr,
                                               to_device)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def outputs(block, vocab):
    return (torch.full((block - 1,), -7, dtype=torch.int32, device="cuda"),
            torch.zeros((block - 1, vocab), dtype=torch.int16, device="cuda"),
            torch.zeros((block, synth.HIDDEN), dtype=torch.int16, device="cuda"))


def test_static_workspace_pass_matches_caller_workspace_pass():
    dev = DeviceWeights(synth.make_weights())
    kv = KVRing(1024)
    dr = Drafter(dev, kv, max_rows=300)
    dr.commit(to_device(synth.make_taps(range(300))), 0)
    torch.cuda.synchronize()
    for p, block in ((300, 8), (40, 4)):  # second call: shorter context, smaller block
        anchor = synth.anchor_token(p)
        say(f"[static scratch] p={p} block={block}")
        c1, l1, h1 = outputs(block, dev.vocab)
        c2, l2, h2 = outputs(block, dev.vocab)
        _lib.dflash_draft_block(dev.desc, kv.desc, p, anchor, synth.MASK_ID, block,
                                c1.data_ptr(), l1.data_ptr(), h1.data_ptr(), dr.ws_ptr,
                                dr.ws_bytes, stream_ptr())
        _lib.dflash_draft_block_static(dev.desc, kv.desc, p, anchor, synth.MASK_ID, block,
                                       c2.data_ptr(), l2.data_ptr(), h2.data_ptr(), stream_ptr())
        torch.cuda.synchronize()
        say(f"[static scratch] cand {c2.cpu().tolist()} vs {c1.cpu().tolist()}")
        assert (c1.cpu().numpy() >= 0).all()
        assert torch.equal(c1, c2)
        assert torch.equal(l1, l2)
        assert torch.equal(h1, h2)
    # arguments are still checked before anything is enqueued
    c, l, h = outputs(8, dev.vocab)
    assert _lib.dflash_draft_block_static(dev.desc, kv.desc, 100, 1, 2, 9, c.data_ptr(), None,
                                          None, stream_ptr(), check=False) == _lib.DFLASH_EINVAL
