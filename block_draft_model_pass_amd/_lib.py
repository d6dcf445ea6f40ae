"""ctypes binding of libdflash.so: the C ABI of include/dflash.h with the
same names.  Argument marshalling only -- every step of the pass runs in the
HIP library.  Loading fails loudly when the library has not been built."""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdflash.so")

DFLASH_OK = 0
DFLASH_EINVAL = -1
DFLASH_EGEOMETRY = -2
DFLASH_ERANGE = -3
DFLASH_EWORKSPACE = -4
DFLASH_EHIP = -5
DFLASH_ENONFINITE = -6
DFLASH_ETIMEOUT = -7

DFLASH_STAGE_RESIDUAL = 0
DFLASH_STAGE_QKV = 1
DFLASH_STAGE_ATTN = 2
DFLASH_STAGE_MLP = 3

DFLASH_W_BF16 = 0
DFLASH_W_Q8_0 = 1
DFLASH_W_Q4_0 = 2
DFLASH_W_Q5_0 = 3

LAYER_FIELDS = ("in_norm", "wq", "wk", "wv", "q_norm", "k_norm", "wo",
                "post_norm", "wg", "wu", "wd")


class dflash_layer_weights(ctypes.Structure):
    _fields_ = [(name, c_void_p) for name in LAYER_FIELDS]


class dflash_weights(ctypes.Structure):
    _fields_ = [
        ("hidden", c_int32), ("n_layers", c_int32), ("n_q_heads", c_int32),
        ("n_kv_heads", c_int32), ("head_dim", c_int32), ("ffn", c_int32),
        ("vocab", c_int32), ("n_taps", c_int32),
        ("rope_theta", c_float), ("attn_scale", c_float), ("rms_eps", c_float),
        ("backbone_type", c_int32),
        ("fc", c_void_p), ("hidden_norm", c_void_p),
        ("layer", dflash_layer_weights * 5),
        ("final_norm", c_void_p), ("embed", c_void_p), ("lm_head", c_void_p),
        ("packed", c_void_p),
        ("lm_head_type", c_int32),
    ]


class dflash_kv(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("vt", c_void_p), ("capacity", c_int32),
                ("window", c_int32)]


class DFlashError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {dflash_strerror(code)} ({code})")


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    try:  # let the library bind to the HIP runtime torch already loaded
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m block_draft_model_pass_amd.build` (there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.dflash_workspace_size.argtypes = [P(dflash_weights), c_int32, c_int32]
    lib.dflash_workspace_size.restype = c_size_t
    lib.dflash_packed_size.argtypes = [P(dflash_weights)]
    lib.dflash_packed_size.restype = c_size_t
    lib.dflash_pack_weights.argtypes = [P(dflash_weights), c_void_p]
    lib.dflash_pack_weights.restype = c_int32
    lib.dflash_fuse_context.argtypes = [P(dflash_weights), c_void_p, c_int32, c_void_p,
                                        c_void_p, c_size_t, c_void_p]
    lib.dflash_fuse_context.restype = c_int32
    lib.dflash_project_ctx_kv.argtypes = [P(dflash_weights), c_void_p, c_int32, c_int64,
                                          P(dflash_kv), c_void_p, c_size_t, c_void_p]
    lib.dflash_project_ctx_kv.restype = c_int32
    lib.dflash_draft_block.argtypes = [P(dflash_weights), P(dflash_kv), c_int64, c_int32,
                                       c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_size_t, c_void_p]
    lib.dflash_draft_block.restype = c_int32
    lib.dflash_draft_block_commit.argtypes = [P(dflash_weights), P(dflash_kv), c_void_p,
                                              c_int32, c_int64, c_int32, c_int32, c_int32,
                                              c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                              c_void_p]
    lib.dflash_draft_block_commit.restype = c_int32
    lib.dflash_draft_block_commit_dev.argtypes = [P(dflash_weights), P(dflash_kv), c_void_p,
                                                  c_int64, c_int64, c_void_p, c_int32, c_int32,
                                                  c_void_p, c_void_p, c_void_p, c_void_p,
                                                  c_size_t, c_void_p]
    lib.dflash_draft_block_commit_dev.restype = c_int32
    lib.dflash_verify_greedy_advance.argtypes = [c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                                 c_void_p]
    lib.dflash_verify_greedy_advance.restype = c_int32
    lib.dflash_draft_block_static.argtypes = [P(dflash_weights), P(dflash_kv), c_int64,
                                              c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                              c_void_p, c_void_p]
    lib.dflash_draft_block_static.restype = c_int32
    lib.dflash_draft_block_gated.argtypes = [P(dflash_weights), P(dflash_kv), c_int64,
                                             c_int32, c_int32, c_int32, ctypes.c_float,
                                             c_void_p, c_void_p, c_void_p, c_void_p,
                                             c_size_t, c_void_p]
    lib.dflash_draft_block_gated.restype = c_int32
    lib.dflash_lm_head_argmax.argtypes = [P(dflash_weights), c_void_p, c_int32, c_void_p,
                                          c_void_p, c_void_p, c_size_t, c_void_p]
    lib.dflash_lm_head_argmax.restype = c_int32
    lib.dflash_verify_greedy.argtypes = [c_void_p, c_void_p, c_int32, c_void_p, c_void_p]
    lib.dflash_verify_greedy.restype = c_int32
    lib.dflash_verify_greedy_gated.argtypes = [c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                               c_void_p]
    lib.dflash_verify_greedy_gated.restype = c_int32
    lib.dflash_draft_status.argtypes = [c_void_p, c_size_t, c_void_p, c_void_p]
    lib.dflash_draft_status.restype = c_int32
    lib.dflash_check_finite.argtypes = [c_void_p, c_int64, c_int32, c_void_p, c_void_p]
    lib.dflash_check_finite.restype = c_int32
    lib.dflash_draft_stage.argtypes = [c_void_p, c_size_t, c_int32, c_int32, c_int32, c_void_p,
                                       c_size_t, c_void_p]
    lib.dflash_draft_stage.restype = c_int32
    lib.dflash_strerror.argtypes = [c_int32]
    lib.dflash_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ref(x):
    return ctypes.byref(x) if x is not None else None


def _check(rc: int, where: str) -> int:
    if rc != DFLASH_OK:
        raise DFlashError(rc, where)
    return rc


def dflash_strerror(code: int) -> str:
    return load().dflash_strerror(code).decode()


def dflash_workspace_size(w, max_rows: int, max_block: int) -> int:
    return int(load().dflash_workspace_size(_ref(w), max_rows, max_block))


def dflash_packed_size(w) -> int:
    return int(load().dflash_packed_size(_ref(w)))


def dflash_pack_weights(w, stream=None, check=True):
    rc = load().dflash_pack_weights(_ref(w), stream)
    return _check(rc, "dflash_pack_weights") if check else rc


def dflash_fuse_context(w, taps, n, ctx, ws, ws_bytes, stream=None, check=True):
    rc = load().dflash_fuse_context(_ref(w), taps, n, ctx, ws, ws_bytes, stream)
    return _check(rc, "dflash_fuse_context") if check else rc


def dflash_project_ctx_kv(w, ctx, n, pos0, kv, ws, ws_bytes, stream=None, check=True):
    rc = load().dflash_project_ctx_kv(_ref(w), ctx, n, pos0, _ref(kv), ws, ws_bytes, stream)
    return _check(rc, "dflash_project_ctx_kv") if check else rc


def dflash_draft_block(w, kv, p, anchor_id, mask_id, block, cand, logits_opt,
                       hidden_opt, ws, ws_bytes, stream=None, check=True):
    rc = load().dflash_draft_block(_ref(w), _ref(kv), p, anchor_id, mask_id, block, cand,
                                   logits_opt, hidden_opt, ws, ws_bytes, stream)
    return _check(rc, "dflash_draft_block") if check else rc


def dflash_draft_block_gated(w, kv, p, anchor_id, mask_id, block, min_p, cand, conf,
                             n_keep, ws, ws_bytes, stream=None, check=True):
    rc = load().dflash_draft_block_gated(_ref(w), _ref(kv), p, anchor_id, mask_id, block,
                                         min_p, cand, conf, n_keep, ws, ws_bytes, stream)
    return _check(rc, "dflash_draft_block_gated") if check else rc


def dflash_lm_head_argmax(w, hidden, rows, cand, logits_opt, ws, ws_bytes, stream=None,
                          check=True):
    rc = load().dflash_lm_head_argmax(_ref(w), hidden, rows, cand, logits_opt, ws, ws_bytes,
                                      stream)
    return _check(rc, "dflash_lm_head_argmax") if check else rc


def dflash_verify_greedy(cand, target, k, out, stream=None, check=True):
    rc = load().dflash_verify_greedy(cand, target, k, out, stream)
    return _check(rc, "dflash_verify_greedy") if check else rc


def dflash_check_finite(x, count, dtype, status, stream=None, check=True):
    rc = load().dflash_check_finite(x, count, dtype, status, stream)
    return _check(rc, "dflash_check_finite") if check else rc


def dflash_verify_greedy_gated(cand, target, k_max, n_keep, out, stream=None, check=True):
    rc = load().dflash_verify_greedy_gated(cand, target, k_max, n_keep, out, stream)
    return _check(rc, "dflash_verify_greedy_gated") if check else rc


def dflash_draft_stage(ws, ws_bytes, stage, index, rows, dst, dst_bytes, stream=None, check=True):
    rc = load().dflash_draft_stage(ws, ws_bytes, stage, index, rows, dst, dst_bytes, stream)
    return _check(rc, "dflash_draft_stage") if check else rc


def dflash_draft_status(ws, ws_bytes, status, stream=None, check=True):
    rc = load().dflash_draft_status(ws, ws_bytes, status, stream)
    return _check(rc, "dflash_draft_status") if check else rc


def dflash_draft_block_static(w, kv, p, anchor_id, mask_id, block, cand, logits_opt,
                              hidden_opt, stream=None, check=True):
    rc = load().dflash_draft_block_static(_ref(w), _ref(kv), p, anchor_id, mask_id, block, cand,
                                          logits_opt, hidden_opt, stream)
    return _check(rc, "dflash_draft_block_static") if check else rc


def dflash_draft_block_commit_dev(w, kv, taps, taps_pos0, taps_rows, state, mask_id, block,
                                  cand, logits_opt, hidden_opt, ws, ws_bytes, stream=None,
                                  check=True):
    rc = load().dflash_draft_block_commit_dev(_ref(w), _ref(kv), taps, taps_pos0, taps_rows,
                                              state, mask_id, block, cand, logits_opt,
                                              hidden_opt, ws, ws_bytes, stream)
    return _check(rc, "dflash_draft_block_commit_dev") if check else rc


def dflash_verify_greedy_advance(cand, target, k, state, out, stream=None, check=True):
    rc = load().dflash_verify_greedy_advance(cand, target, k, state, out, stream)
    return _check(rc, "dflash_verify_greedy_advance") if check else rc


def dflash_draft_block_commit(w, kv, taps, n_commit, p, anchor_id, mask_id, block, cand,
                              logits_opt, hidden_opt, ws, ws_bytes, stream=None, check=True):
    rc = load().dflash_draft_block_commit(_ref(w), _ref(kv), taps, n_commit, p, anchor_id,
                                          mask_id, block, cand, logits_opt, hidden_opt, ws,
                                          ws_bytes, stream)
    return _check(rc, "dflash_draft_block_commit") if check else rc
