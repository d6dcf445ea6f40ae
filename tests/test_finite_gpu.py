"""GPU: the optional finite check (dflash_check_finite) against numpy's
isfinite on the same bytes, for bf16, fp16 and fp32 buffers of ragged length
with NaN / +-inf planted at the first, a middle and the last element (the
last one in the element-wise tail), past the checked range, and not at all."""
import sys

import numpy as np
import pytest
import torch

from block_draft_model_pass_amd import _lib

pytestmark = pytest.mark.gpu

DT = {0: (torch.bfloat16, np.uint16, 16, 7), 1: (torch.float16, np.uint16, 16, 10),
      2: (torch.float32, np.uint32, 32, 23)}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def reference(bits: np.ndarray, dtype: int) -> int:
    """DFLASH_ENONFINITE if any value is NaN or infinite, by decoding the bytes
    with numpy (bf16 widened to fp32 by a 16-bit shift)."""
    if dtype == 0:
        vals = (bits.astype(np.uint32) << 16).view(np.float32)
    elif dtype == 1:
        vals = bits.view(np.float16)
    else:
        vals = bits.view(np.float32)
    return 0 if np.isfinite(vals).all() else _lib.DFLASH_ENONFINITE


def special(dtype: int, kind: str) -> int:
    _, _, width, mant = DT[dtype]
    exp_all = ((1 << (width - 1 - mant)) - 1) << mant
    sign = 1 << (width - 1)
    return {"nan": exp_all | 1, "+inf": exp_all, "-inf": exp_all | sign}[kind]


@pytest.mark.parametrize("dtype", [0, 1, 2])
@pytest.mark.parametrize("count", [0, 1, 7, 8, 1000003])
def test_check_finite(dtype, count):
    tdt, ndt, _, _ = DT[dtype]
    torch.cuda.set_device(0)
    gen = torch.Generator().manual_seed(11 + dtype)
    host = (torch.randn(count + 64, generator=gen) * 1e3).to(tdt)   # 64 spare elements past count
    bits = host.view(torch.int16 if ndt == np.uint16 else torch.int32).numpy().view(ndt).copy()
    status = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    cases = [("none", None, None)]
    if count > 0:
        for kind in ("nan", "+inf", "-inf"):
            for at in sorted({0, count // 2, count - 1}):
                cases.append((kind, at, special(dtype, kind)))
    cases.append(("nan past count", count + 3, special(dtype, "nan")))
    for name, at, val in cases:
        b = bits.copy()
        if at is not None:
            b[at] = val
        dev = torch.from_numpy(b.view(np.int16 if ndt == np.uint16 else np.int32)).cuda()
        say(f"check_finite dtype={dtype} count={count} case={name} at={at}")
        _lib.dflash_check_finite(dev.data_ptr(), count, dtype, status.data_ptr())
        torch.cuda.synchronize()
        assert int(status.item()) == reference(b[:count], dtype), (name, at)
