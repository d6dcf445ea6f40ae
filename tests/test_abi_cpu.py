"""The C-ABI library on the host: it loads, exports every entry point the
header declares (and nothing from torch), and its argument checks return the
documented codes before anything reaches a GPU.  Runs without a GPU: every
call below fails validation on the host, so no kernel is launched."""
import ctypes
import os
import re
import subprocess

import pytest

from block_draft_model_pass_amd import _lib, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")


def header_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libdflash.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_header_declares_the_four_operations():
    syms = header_symbols()
    for s in ("dflash_fuse_context", "dflash_project_ctx_kv", "dflash_draft_block",
              "dflash_verify_greedy", "dflash_workspace_size", "dflash_strerror",
              "dflash_lm_head_argmax"):
        assert s in syms


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    for s in header_symbols():
        assert s in exported, s
        assert hasattr(lib, s)


def test_library_exports_only_the_c_abi():
    """Hidden visibility plus a version script: the dynamic symbol table holds
    the header's entry points and nothing else (no C++ internals)."""
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    defined = set(l.split()[-1] for l in out.splitlines() if l.strip())
    assert defined == set(header_symbols()), sorted(defined ^ set(header_symbols()))


def test_library_has_no_torch_dependency():
    out = subprocess.run(["readelf", "-d", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    needed = re.findall(r"NEEDED.*\[(.*)\]", out)
    assert any("amdhip64" in n for n in needed)
    assert not any("torch" in n or "c10" in n or "cuda" in n for n in needed), needed


def fake_weights(**over):
    """A descriptor with the DFlash geometry and non-null dummy pointers; only
    ever used with calls that fail validation on the host."""
    w = _lib.dflash_weights()
    w.hidden, w.n_layers, w.n_q_heads, w.n_kv_heads = 2560, 5, 24, 2
    w.head_dim, w.ffn, w.vocab, w.n_taps = 256, 7680, synth.VOCAB, 5
    w.rope_theta, w.attn_scale, w.rms_eps = 1e7, 1.0 / 16, 1e-6
    w.backbone_type = _lib.DFLASH_W_BF16
    dummy = 0x10000
    w.fc = w.hidden_norm = w.final_norm = w.embed = w.lm_head = dummy
    for l in range(5):
        for f in _lib.LAYER_FIELDS:
            setattr(w.layer[l], f, dummy)
    for k, v in over.items():
        setattr(w, k, v)
    return w


A = 0x40000  # a 16-byte-aligned dummy device pointer (never dereferenced)


def fake_kv(capacity=32768, window=32768):
    return _lib.dflash_kv(0x20000, 0x30000, capacity, window)


def test_workspace_size(lib):
    w = fake_weights()
    base = _lib.dflash_workspace_size(w, 0, 8)
    assert base > 0
    assert _lib.dflash_workspace_size(w, 64, 8) == base       # skinny path
    big = _lib.dflash_workspace_size(w, 32768, 8)
    assert big >= base + 32768 * 5120 * 4
    assert _lib.dflash_workspace_size(w, -1, 8) == 0
    assert _lib.dflash_workspace_size(w, 16, 9) == 0


def test_strerror_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, -99):
        assert isinstance(_lib.dflash_strerror(code), str)
    assert _lib.dflash_strerror(-4) == "workspace too small"
    assert _lib.dflash_strerror(_lib.DFLASH_ENONFINITE) == "non-finite value found"
    assert "gave up" in _lib.dflash_strerror(_lib.DFLASH_ETIMEOUT)


def test_check_finite_arguments(lib):
    """Rejected on the host before anything is enqueued (no device needed)."""
    E = _lib.DFLASH_EINVAL
    assert _lib.dflash_check_finite(A, 16, 0, None, check=False) == E       # no status word
    assert _lib.dflash_check_finite(A, 16, 0, A + 2, check=False) == E      # misaligned status
    assert _lib.dflash_check_finite(None, 16, 0, A, check=False) == E       # no buffer
    assert _lib.dflash_check_finite(A + 8, 16, 2, A, check=False) == E      # misaligned buffer
    assert _lib.dflash_check_finite(A, -1, 0, A, check=False) == E         # negative count
    for dtype in (-1, 3):
        assert _lib.dflash_check_finite(A, 16, dtype, A, check=False) == E


@pytest.mark.parametrize("field,value", [
    ("hidden", 4096), ("n_layers", 4), ("n_q_heads", 32), ("n_kv_heads", 8),
    ("head_dim", 128), ("ffn", 9728), ("n_taps", 4), ("vocab", 151937),
    ("rope_theta", 1e6), ("attn_scale", 0.125), ("rms_eps", 1e-5)])
def test_geometry_mismatch_is_rejected(lib, field, value):
    w = fake_weights(**{field: value})
    rc = _lib.dflash_fuse_context(w, 1, 4, 1, 1, 1 << 40, check=False)
    assert rc == _lib.DFLASH_EGEOMETRY
    rc = _lib.dflash_draft_block(w, fake_kv(), 8192, 1, 2, 8, 1, None, None, 1, 1 << 40,
                                 check=False)
    assert rc == _lib.DFLASH_EGEOMETRY


def test_null_and_bad_arguments(lib):
    w = fake_weights()
    kv = fake_kv()
    big = 1 << 40
    E = _lib.DFLASH_EINVAL
    assert _lib.dflash_fuse_context(None, A, 4, A, A, big, check=False) == E
    assert _lib.dflash_fuse_context(w, None, 4, A, A, big, check=False) == E
    assert _lib.dflash_fuse_context(w, A, -1, A, A, big, check=False) == E
    assert _lib.dflash_fuse_context(w, A, 0, A, A, big, check=False) == 0  # no work
    w2 = fake_weights()
    w2.layer[3].wd = None
    assert _lib.dflash_fuse_context(w2, A, 4, A, A, big, check=False) == E
    w3 = fake_weights(backbone_type=7)
    assert _lib.dflash_fuse_context(w3, A, 4, A, A, big, check=False) == E
    for block in (0, 9, -3):
        assert _lib.dflash_draft_block(w, kv, 100, 1, 2, block, A, None, None, A, big,
                                       check=False) == E
    for anchor, mask in ((-1, 2), (synth.VOCAB, 2), (1, synth.VOCAB)):
        assert _lib.dflash_draft_block(w, kv, 100, anchor, mask, 8, A, None, None, A, big,
                                       check=False) == E
    assert _lib.dflash_draft_block(w, kv, -1, 1, 2, 8, A, None, None, A, big,
                                   check=False) == E
    assert _lib.dflash_draft_block(w, kv, 5, 1, 2, 8, None, None, None, A, big,
                                   check=False) == E
    assert _lib.dflash_project_ctx_kv(w, A, 4, -5, kv, A, big, check=False) == E
    G = _lib.dflash_draft_block_gated
    for block in (0, 1, 9):  # the gate needs at least one candidate
        assert G(w, kv, 100, 1, 2, block, 0.5, A, A, A, A, big, check=False) == E
    for min_p in (-0.1, 1.5, float("nan")):
        assert G(w, kv, 100, 1, 2, 8, min_p, A, A, A, A, big, check=False) == E
    assert G(w, kv, 100, 1, 2, 8, 0.5, A, None, A, A, big, check=False) == E
    assert G(w, kv, 100, 1, 2, 8, 0.5, A, A, None, A, big, check=False) == E
    assert G(w, kv, 100, 1, 2, 8, 0.5, None, A, A, A, big, check=False) == E
    assert G(w, kv, 100, 1, 2, 8, 0.5, A, A + 2, A, A, big, check=False) == E
    assert G(w, kv, 100, -1, 2, 8, 0.5, A, A, A, A, big, check=False) == E
    assert _lib.dflash_lm_head_argmax(w, A, 0, A, None, A, big, check=False) == E
    assert _lib.dflash_lm_head_argmax(w, A, 9, A, None, A, big, check=False) == E
    assert _lib.dflash_lm_head_argmax(w, None, 3, A, None, A, big, check=False) == E
    assert _lib.dflash_verify_greedy(A, A, 8, A, check=False) == E
    assert _lib.dflash_verify_greedy(A, A, -1, A, check=False) == E
    assert _lib.dflash_verify_greedy(A, None, 3, A, check=False) == E


def test_ring_range_violations(lib):
    w = fake_weights()
    big = 1 << 40
    R = _lib.DFLASH_ERANGE
    assert _lib.dflash_draft_block(w, fake_kv(1000, 1000), 10, 1, 2, 8, A, None, None, A, big,
                                   check=False) == R
    assert _lib.dflash_draft_block(w, fake_kv(1024, 2048), 10, 1, 2, 8, A, None, None, A, big,
                                   check=False) == R
    assert _lib.dflash_draft_block(w, fake_kv(1024, 0), 10, 1, 2, 8, A, None, None, A, big,
                                   check=False) == R
    assert _lib.dflash_project_ctx_kv(w, A, 2048, 0, fake_kv(1024, 1024), A, big,
                                      check=False) == R


def test_workspace_too_small(lib):
    w = fake_weights()
    kv = fake_kv()
    need = _lib.dflash_workspace_size(w, 0, 8)
    W = _lib.DFLASH_EWORKSPACE
    assert _lib.dflash_draft_block(w, kv, 10, 1, 2, 8, A, None, None, A, need - 1,
                                   check=False) == W
    need_rows = _lib.dflash_workspace_size(w, 4096, 8)
    assert _lib.dflash_fuse_context(w, A, 4096, A, A, need_rows - 1, check=False) == W
    assert _lib.dflash_project_ctx_kv(w, A, 4096, 0, kv, A, need_rows - 1, check=False) == W


def test_packed_copy_size_and_checks(lib):
    """The streaming copies hold the LM head, the 35 layer matrices and fc in
    the backbone's format; packing needs a buffer and the draft pass needs the
    copies."""
    w = fake_weights()
    lm = 2 * synth.VOCAB * 2560
    weights = 5 * (6144 * 2560 + 2 * 512 * 2560 + 2560 * 6144 + 2 * 7680 * 2560 + 2560 * 7680) \
        + 2560 * 12800
    assert _lib.dflash_packed_size(w) == lm + 2 * weights
    q8 = _lib.dflash_packed_size(fake_weights(backbone_type=_lib.DFLASH_W_Q8_0))
    q4 = _lib.dflash_packed_size(fake_weights(backbone_type=_lib.DFLASH_W_Q4_0))
    q5 = _lib.dflash_packed_size(fake_weights(backbone_type=_lib.DFLASH_W_Q5_0))
    assert q8 == lm + weights * 34 // 32
    assert q4 == lm + weights * 18 // 32
    assert q5 == lm + weights * 22 // 32
    assert _lib.dflash_packed_size(fake_weights(backbone_type=4)) == 0
    assert _lib.dflash_packed_size(fake_weights(hidden=4096)) == 0
    # a Q8_0 LM head: vocab * 2560 weights at 34/32 bytes, ahead of the layers
    assert _lib.dflash_packed_size(fake_weights(lm_head_type=_lib.DFLASH_W_Q8_0)) == \
        synth.VOCAB * 2560 * 34 // 32 + 2 * weights
    for bad in (_lib.DFLASH_W_Q4_0, _lib.DFLASH_W_Q5_0, 4, -1):  # bf16 or Q8_0 only
        assert _lib.dflash_packed_size(fake_weights(lm_head_type=bad)) == 0
    assert _lib.dflash_pack_weights(w, None, check=False) == _lib.DFLASH_EINVAL
    big = 1 << 40
    assert _lib.dflash_draft_block(w, fake_kv(), 10, 1, 2, 8, A, None, None, A, big,
                                   check=False) == _lib.DFLASH_EINVAL


def test_misaligned_pointers_are_rejected(lib):
    """Device buffers are accessed 16 bytes at a time: a misaligned weight,
    ring, workspace, input or output pointer is refused before any launch."""
    big = 1 << 40
    E = _lib.DFLASH_EINVAL
    kv = fake_kv()
    assert _lib.dflash_fuse_context(fake_weights(fc=A + 2), A, 4, A, A, big, check=False) == E
    w = fake_weights()
    w.layer[2].wo = A + 8
    assert _lib.dflash_fuse_context(w, A, 4, A, A, big, check=False) == E
    w = fake_weights()
    assert _lib.dflash_fuse_context(w, A + 2, 4, A, A, big, check=False) == E
    assert _lib.dflash_fuse_context(w, A, 4, A + 4, A, big, check=False) == E
    assert _lib.dflash_project_ctx_kv(w, A, 4, 0, kv, A + 8, big, check=False) == E
    assert _lib.dflash_project_ctx_kv(w, A, 4, 0, _lib.dflash_kv(A + 2, A, 32768, 32768), A,
                                      big, check=False) == E
    w.packed = A
    assert _lib.dflash_draft_block(w, kv, 10, 1, 2, 8, A + 2, None, None, A, big,
                                   check=False) == E
    assert _lib.dflash_draft_block(w, kv, 10, 1, 2, 8, A, A + 8, None, A, big,
                                   check=False) == E
    assert _lib.dflash_lm_head_argmax(w, A + 2, 3, A, None, A, big, check=False) == E
    w.packed = A + 4
    assert _lib.dflash_draft_block(w, kv, 10, 1, 2, 8, A, None, None, A, big,
                                   check=False) == E


def test_gated_verify_and_status_arguments(lib):
    """The verify that reads its count on the device and the pass-status
    readout validate their arguments on the host."""
    E = _lib.DFLASH_EINVAL
    V = _lib.dflash_verify_greedy_gated
    assert V(A, A, 8, A, A, check=False) == E          # k_max > 7
    assert V(A, A, -1, A, A, check=False) == E
    assert V(A, A, 7, None, A, check=False) == E       # no count word
    assert V(A, None, 7, A, A, check=False) == E
    assert V(A, A, 7, A, None, check=False) == E
    assert V(None, A, 3, A, A, check=False) == E       # candidates needed when k_max > 0
    assert V(A, A, 7, A + 2, A, check=False) == E      # misaligned count word
    need = _lib.dflash_workspace_size(fake_weights(), 0, 8)
    S = _lib.dflash_draft_status
    assert S(None, need, A, check=False) == E
    assert S(A, need, None, check=False) == E
    assert S(A, need, A + 1, check=False) == E
    assert S(A + 8, need, A, check=False) == E
    assert S(A, need - 1, A, check=False) == _lib.DFLASH_EWORKSPACE


def test_stage_readout_arguments(lib):
    """dflash_draft_stage checks its stage, index, rows and sizes on the host
    before it enqueues the copy."""
    E = _lib.DFLASH_EINVAL
    need = _lib.dflash_workspace_size(fake_weights(), 0, 8)
    R, Q, T, M = (_lib.DFLASH_STAGE_RESIDUAL, _lib.DFLASH_STAGE_QKV, _lib.DFLASH_STAGE_ATTN,
                  _lib.DFLASH_STAGE_MLP)
    big = 1 << 20

    def S(ws=A, nb=need, st=R, idx=0, rows=8, dst=A, db=big):
        return _lib.dflash_draft_stage(ws, nb, st, idx, rows, dst, db, None, check=False)

    assert S(ws=None) == E and S(dst=None) == E
    assert S(ws=A + 8) == E and S(dst=A + 4) == E
    assert S(rows=0) == E and S(rows=9) == E
    assert S(st=4) == E and S(st=-1) == E
    assert S(st=R, idx=11) == E and S(st=R, idx=-1) == E
    for st in (Q, T, M):
        assert S(st=st, idx=5) == E
    assert S(st=R, rows=8, db=8 * 2560 * 4 - 1) == E
    assert S(st=Q, rows=3, db=3 * 7168 * 2 - 2) == E
    assert S(st=T, rows=1, db=6144 * 2 - 2) == E
    assert S(st=M, rows=2, db=2 * 7680 * 2 - 2) == E
    assert S(nb=need // 4) == _lib.DFLASH_EWORKSPACE


def test_device_cycle_arguments(lib):
    """The device-resident cycle's host checks: state and taps present and
    aligned, taps_pos0 / taps_rows non-negative, block and mask as for
    dflash_draft_block; the advancing verify checks k and its pointers."""
    E = _lib.DFLASH_EINVAL
    w, kv = fake_weights(), fake_kv()
    need = _lib.dflash_workspace_size(w, 0, 8)

    def D(taps=A, pos0=0, rows=64, state=A, mask=2, block=8, cand=A, ws=A, nb=need):
        return _lib.dflash_draft_block_commit_dev(w, kv, taps, pos0, rows, state, mask, block,
                                                  cand, None, None, ws, nb, None, check=False)

    assert D(state=None) == E and D(state=A + 4) == E
    assert D(taps=None) == E and D(taps=A + 8) == E
    assert D(pos0=-1) == E and D(rows=-1) == E
    assert D(block=0) == E and D(block=9) == E and D(mask=-1) == E
    assert D(cand=None) == E and D(ws=None) == E
    assert D(nb=need - 1) == _lib.DFLASH_EWORKSPACE
    V = _lib.dflash_verify_greedy_advance
    assert V(A, A, 8, A, A, check=False) == E
    assert V(A, A, -1, A, A, check=False) == E
    assert V(A, A, 7, None, A, check=False) == E
    assert V(A, A, 7, A + 4, A, check=False) == E       # state: 8-byte words
    assert V(A, None, 7, A, A, check=False) == E
    assert V(A, A, 7, A, None, check=False) == E
    assert V(None, A, 3, A, A, check=False) == E
    assert V(A, A, 7, A, A + 2, check=False) == E


def test_packed_copy_may_stand_in_for_row_major_matrices(lib):
    """With the streaming copies set, the row-major matrices (fc, the layer
    matrices, the LM head) may be null -- the weights are then held once;
    without them, or when packing, they are required.  Gains and the
    embedding are always required."""
    big = 1 << 40
    E = _lib.DFLASH_EINVAL
    w = fake_weights()
    w.packed = A
    w.fc = w.lm_head = None
    for l in range(5):
        for f in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
            setattr(w.layer[l], f, None)
    assert _lib.dflash_fuse_context(w, A, 0, A, A, big, check=False) == 0   # checks pass, no work
    assert _lib.dflash_project_ctx_kv(w, A, 0, 0, fake_kv(), A, big, check=False) == 0
    assert _lib.dflash_packed_size(w) > 0
    assert _lib.dflash_pack_weights(w, None, check=False) == E             # packing reads them
    w.packed = None
    assert _lib.dflash_fuse_context(w, A, 0, A, A, big, check=False) == E
    w.packed = A
    w.layer[2].q_norm = None
    assert _lib.dflash_fuse_context(w, A, 0, A, A, big, check=False) == E
    w.layer[2].q_norm = A
    w.embed = None
    assert _lib.dflash_fuse_context(w, A, 0, A, A, big, check=False) == E


def test_static_workspace_pass_arguments(lib):
    """dflash_draft_block_static checks its arguments like dflash_draft_block
    before it touches a device (no workspace argument)."""
    w = fake_weights()
    w.packed = A
    kv = fake_kv()
    E = _lib.DFLASH_EINVAL
    S = _lib.dflash_draft_block_static
    for block in (0, 9):
        assert S(w, kv, 100, 1, 2, block, A, None, None, check=False) == E
    assert S(w, kv, -1, 1, 2, 8, A, None, None, check=False) == E
    assert S(w, kv, 100, -1, 2, 8, A, None, None, check=False) == E
    assert S(w, kv, 100, 1, 2, 8, None, None, None, check=False) == E
    assert S(w, kv, 100, 1, 2, 8, A + 2, None, None, check=False) == E
    assert S(w, kv, 100, 1, 2, 8, A, A + 8, None, check=False) == E
    assert S(fake_weights(hidden=4096), kv, 100, 1, 2, 8, A, None, None, check=False) == \
        _lib.DFLASH_EGEOMETRY
    assert S(w, fake_kv(1000, 1000), 100, 1, 2, 8, A, None, None, check=False) == \
        _lib.DFLASH_ERANGE


def test_fused_commit_pass_arguments(lib):
    """dflash_draft_block_commit: n_commit in [0, 8], p >= n_commit, taps
    non-null and 16-byte aligned when there are commit rows."""
    w = fake_weights()
    w.packed = A
    kv = fake_kv()
    big = 1 << 40
    E = _lib.DFLASH_EINVAL
    C = _lib.dflash_draft_block_commit
    for nc in (-1, 9):
        assert C(w, kv, A, nc, 100, 1, 2, 8, A, None, None, A, big, check=False) == E
    assert C(w, kv, A, 5, 4, 1, 2, 8, A, None, None, A, big, check=False) == E      # p < n_commit
    assert C(w, kv, None, 3, 100, 1, 2, 8, A, None, None, A, big, check=False) == E  # no taps
    assert C(w, kv, A + 8, 3, 100, 1, 2, 8, A, None, None, A, big, check=False) == E
    assert C(w, kv, A, 3, 100, 1, 2, 9, A, None, None, A, big, check=False) == E    # block
    need = _lib.dflash_workspace_size(w, 0, 8)
    assert C(w, kv, A, 3, 100, 1, 2, 8, A, None, None, A, need - 1, check=False) == \
        _lib.DFLASH_EWORKSPACE
