"""CPU checks of the benchmark's contract: one GPU only, and the algorithmic
bytes its roofline divides by.

Bytes of one draft pass (block B >= 2): the 35 layer matrices in their
storage format, the bf16 LM head (151936 x 2560), the 22 bf16 gains, two
embedding rows and 10,240 bytes of fp16 K and V per context cell (5 layers x
2 KV heads x 256 x K and V).  The expected totals below are that sum written
out per workload."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

LAYERS_BF16 = 5 * (6144 * 2560 + 2 * 512 * 2560 + 2560 * 6144 + 2 * 7680 * 2560 + 2560 * 7680) * 2


def test_layer_matrix_bytes():
    assert LAYERS_BF16 == 930_611_200


@pytest.mark.parametrize("ctx,block,fmt,expected", [
    (8192, 8, "bf16", 1_792_481_280),    # decode loop at ctx 8192 (the headline pass)
    (32768, 8, "bf16", 2_044_139_520),   # 32768 resident cells
    (2432, 8, "bf16", 1_733_498_880),    # short prompt
    (32, 4, "bf16", 1_708_922_880),      # smallest configuration
    (8192, 4, "q8_0", 1_356_257_280),    # 34 bytes per 32 weights
    (8192, 4, "q4_0", 1_123_604_480),    # 18 bytes per 32 weights
    (8192, 4, "q5_0", 1_181_767_680),    # 22 bytes per 32 weights: q4_0 + 465_305_600 / 8
])
def test_pass_bytes(ctx, block, fmt, expected):
    assert bench.pass_bytes(ctx, block, fmt) == expected


def test_pass_bytes_parts():
    lm = 151936 * 2560 * 2
    gains = 2 * (5 * (2 * 2560 + 2 * 256) + 2560)
    assert lm == 777_912_320 and gains == 61_440
    assert bench.pass_bytes(0) == LAYERS_BF16 + lm + gains + 2 * 2560 * 2
    assert bench.pass_bytes(1, 8) - bench.pass_bytes(0, 8) == 10_240


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
