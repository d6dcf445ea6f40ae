"""Device-memory plumbing over the C ABI: weights resident in HBM with their
descriptor, the fp16 K/V ring, the workspace, and thin methods that pass
pointers to the library on torch's current HIP stream.  PyTorch only
allocates and owns memory here; all computation happens in libdflash.so."""
from __future__ import annotations

import numpy as np
import torch

from . import _lib, synth
from ._lib import (dflash_draft_block, dflash_fuse_context, dflash_kv,
                   dflash_lm_head_argmax, dflash_pack_weights, dflash_packed_size,
                   dflash_project_ctx_kv, dflash_verify_greedy, dflash_weights,
                   dflash_workspace_size)

_FORMATS = {"bf16": _lib.DFLASH_W_BF16, "q8_0": _lib.DFLASH_W_Q8_0,
            "q4_0": _lib.DFLASH_W_Q4_0,
            "q5_0": _lib.DFLASH_W_Q5_0}


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("no HIP device visible: the DFlash library runs on the GPU only")
    _lib.load()


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Copy a host array's bytes to HBM (uint16 arrays travel as int16)."""
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def stream_ptr() -> int:
    return torch.cuda.current_stream().cuda_stream


# Row-major matrices whose streaming copies dflash_pack_weights writes.
MATRICES = ("fc", "lm_head") + tuple(f"layers.{l}.{m}" for l in range(synth.N_LAYERS)
                                     for m in synth.MATRIX_KINDS)


class DeviceWeights:
    """All drafter tensors in HBM plus the dflash_weights descriptor.

    With packed_only=True the row-major matrices are released once their
    streaming copies are written and their descriptor pointers set to NULL:
    every call then reads the copies, so the matrices are held once."""

    def __init__(self, host: dict, device="cuda", packed_only: bool = False):
        require_gpu()
        self.format = host.get("__format__", "bf16")
        self.t = {k: to_device(v, device) for k, v in host.items() if not k.startswith("__")}
        d = dflash_weights()
        d.hidden, d.n_layers, d.n_q_heads = synth.HIDDEN, synth.N_LAYERS, synth.N_Q_HEADS
        d.n_kv_heads, d.head_dim, d.ffn = synth.N_KV_HEADS, synth.HEAD_DIM, synth.FFN
        d.vocab, d.n_taps = self.t["embed"].shape[0], synth.N_TAPS
        d.rope_theta, d.attn_scale, d.rms_eps = synth.ROPE_THETA, synth.ATTN_SCALE, synth.RMS_EPS
        d.backbone_type = _FORMATS[self.format]
        self.lm_format = host.get("__lm_format__", "bf16")
        d.lm_head_type = _FORMATS[self.lm_format]
        d.fc = self.t["fc"].data_ptr()
        d.hidden_norm = self.t["hidden_norm"].data_ptr()
        for l in range(synth.N_LAYERS):
            for f in _lib.LAYER_FIELDS:
                setattr(d.layer[l], f, self.t[f"layers.{l}.{f}"].data_ptr())
        d.final_norm = self.t["final_norm"].data_ptr()
        d.embed = self.t["embed"].data_ptr()
        d.lm_head = self.t["lm_head"].data_ptr()
        # streaming copy of the bf16 matrices the draft pass reads
        self.packed = torch.empty(dflash_packed_size(d), dtype=torch.uint8, device=device)
        d.packed = self.packed.data_ptr()
        dflash_pack_weights(d, stream_ptr())
        self.desc = d
        self.vocab = d.vocab
        self.packed_only = packed_only
        if packed_only:
            torch.cuda.current_stream().synchronize()  # packing has read them
            d.fc = d.lm_head = None
            for l in range(synth.N_LAYERS):
                for m in synth.MATRIX_KINDS:
                    setattr(d.layer[l], m, None)
            for name in MATRICES:
                del self.t[name]

    def repack(self):
        """Rewrite the streaming copies after the row-major tensors changed."""
        if self.packed_only:
            raise RuntimeError("the row-major matrices were released")
        dflash_pack_weights(self.desc, stream_ptr())


class KVRing:
    """fp16 K [5][2][cap][256] and block-transposed V [5][2][cap/32][256][32]."""

    def __init__(self, capacity: int, window: int | None = None, device="cuda"):
        window = min(synth.WINDOW, capacity) if window is None else window
        self.k = torch.zeros((synth.N_LAYERS, synth.N_KV_HEADS, capacity, synth.HEAD_DIM),
                             dtype=torch.float16, device=device)
        self.vt = torch.zeros((synth.N_LAYERS, synth.N_KV_HEADS, capacity // 32,
                               synth.HEAD_DIM, 32), dtype=torch.float16, device=device)
        self.desc = dflash_kv(self.k.data_ptr(), self.vt.data_ptr(), capacity, window)
        self.capacity = capacity
        self.window = window

    def values(self) -> torch.Tensor:
        """V as [5][2][cap][256] (a transposed copy of the ring's values)."""
        L, J, nb, D, c = self.vt.shape
        return self.vt.permute(0, 1, 2, 4, 3).reshape(L, J, nb * c, D)

    def set_values(self, v: torch.Tensor):
        """Fill the ring's values from V [5][2][cap][256]."""
        L, J, nb, D, c = self.vt.shape
        self.vt.copy_(v.reshape(L, J, nb, c, D).permute(0, 1, 2, 4, 3))


class Drafter:
    """Calls of the four entry points with device buffers."""

    def __init__(self, weights: DeviceWeights, kv: KVRing, max_rows: int = 16,
                 max_block: int = synth.MAX_BLOCK, device="cuda"):
        self.w = weights
        self.kv = kv
        self.ws_bytes = dflash_workspace_size(weights.desc, max_rows, max_block)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.ws_ptr = self.ws.data_ptr()
        self.max_rows = max_rows
        self.device = device
        # fused context rows of commit(): reused, so a decode step allocates nothing
        self.ctx_buf = torch.empty((max_rows, synth.HIDDEN), dtype=torch.int16, device=device)

    def fuse(self, taps: torch.Tensor, ctx: torch.Tensor | None = None) -> torch.Tensor:
        n = taps.shape[0]
        if ctx is None:
            ctx = torch.empty((n, synth.HIDDEN), dtype=torch.int16, device=self.device)
        dflash_fuse_context(self.w.desc, taps.data_ptr(), n, ctx.data_ptr(),
                            self.ws.data_ptr(), self.ws_bytes, stream_ptr())
        return ctx

    def project(self, ctx: torch.Tensor, pos0: int):
        dflash_project_ctx_kv(self.w.desc, ctx.data_ptr(), ctx.shape[0], pos0, self.kv.desc,
                              self.ws.data_ptr(), self.ws_bytes, stream_ptr())

    def commit(self, taps: torch.Tensor, pos0: int) -> torch.Tensor:
        """Fuse and project taps [n][12800] (n <= max_rows) into cells
        pos0 .. pos0+n-1; returns the fused rows (a view of the reused
        context buffer, valid until the next commit)."""
        n = taps.shape[0]
        self.commit_ptr(taps.data_ptr(), n, pos0)
        return self.ctx_buf[:n]

    def commit_ptr(self, taps_ptr: int, n: int, pos0: int):
        """commit() on a raw device pointer to n rows of taps: no tensor is
        created or allocated on this path."""
        if not 0 <= n <= self.max_rows:
            raise ValueError(f"commit of {n} rows: this Drafter holds at most {self.max_rows}")
        st = stream_ptr()
        ctx = self.ctx_buf.data_ptr()
        dflash_fuse_context(self.w.desc, taps_ptr, n, ctx, self.ws_ptr, self.ws_bytes, st)
        dflash_project_ctx_kv(self.w.desc, ctx, n, pos0, self.kv.desc, self.ws_ptr,
                              self.ws_bytes, st)

    def draft(self, p: int, anchor: int, block: int, mask_id: int = synth.MASK_ID,
              cand: torch.Tensor | None = None, logits: torch.Tensor | None = None,
              hidden: torch.Tensor | None = None) -> torch.Tensor:
        if cand is None:
            cand = torch.empty(max(block - 1, 1), dtype=torch.int32, device=self.device)
        dflash_draft_block(self.w.desc, self.kv.desc, p, anchor, mask_id, block,
                           cand.data_ptr(),
                           logits.data_ptr() if logits is not None else None,
                           hidden.data_ptr() if hidden is not None else None,
                           self.ws.data_ptr(), self.ws_bytes, stream_ptr())
        return cand

    def draft_commit(self, taps_ptr: int | None, n_commit: int, p: int, anchor: int, block: int,
                     mask_id: int = synth.MASK_ID, cand: torch.Tensor | None = None,
                     logits: torch.Tensor | None = None,
                     hidden: torch.Tensor | None = None) -> torch.Tensor:
        """One pass that commits n_commit rows of taps (a device pointer to
        [n_commit][5][2560] bf16) at positions p-n_commit .. p-1 and drafts
        the block at p (dflash_draft_block_commit)."""
        if cand is None:
            cand = torch.empty(max(block - 1, 1), dtype=torch.int32, device=self.device)
        _lib.dflash_draft_block_commit(self.w.desc, self.kv.desc, taps_ptr, n_commit, p, anchor,
                                       mask_id, block, cand.data_ptr(),
                                       logits.data_ptr() if logits is not None else None,
                                       hidden.data_ptr() if hidden is not None else None,
                                       self.ws_ptr, self.ws_bytes, stream_ptr())
        return cand

    def draft_commit_dev(self, taps: torch.Tensor, taps_pos0: int, state: torch.Tensor,
                         block: int, mask_id: int = synth.MASK_ID,
                         cand: torch.Tensor | None = None, logits: torch.Tensor | None = None,
                         hidden: torch.Tensor | None = None) -> torch.Tensor:
        """draft_commit with p, the anchor and the commit count read from the
        int64 device words state = {p, anchor, n_commit}; taps holds the taps
        of positions taps_pos0 .. taps_pos0 + len(taps) - 1
        (dflash_draft_block_commit_dev)."""
        if cand is None:
            cand = torch.empty(max(block - 1, 1), dtype=torch.int32, device=self.device)
        _lib.dflash_draft_block_commit_dev(self.w.desc, self.kv.desc, taps.data_ptr(), taps_pos0,
                                           taps.shape[0], state.data_ptr(), mask_id, block,
                                           cand.data_ptr(),
                                           logits.data_ptr() if logits is not None else None,
                                           hidden.data_ptr() if hidden is not None else None,
                                           self.ws_ptr, self.ws_bytes, stream_ptr())
        return cand

    def verify_advance(self, cand: torch.Tensor, target: torch.Tensor, k: int,
                       state: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        """verify() that also advances state = {p, anchor, n_commit}
        (dflash_verify_greedy_advance)."""
        if out is None:
            out = torch.empty(2, dtype=torch.int32, device=self.device)
        _lib.dflash_verify_greedy_advance(cand.data_ptr(), target.data_ptr(), k,
                                          state.data_ptr(), out.data_ptr(), stream_ptr())
        return out

    def draft_gated(self, p: int, anchor: int, block: int, min_p: float,
                    mask_id: int = synth.MASK_ID, cand: torch.Tensor | None = None,
                    conf: torch.Tensor | None = None, n_keep: torch.Tensor | None = None):
        """draft() plus each candidate's softmax probability and the number of
        leading candidates at or above the floor min_p; returns
        (cand, conf, n_keep) device tensors."""
        if cand is None:
            cand = torch.empty(block - 1, dtype=torch.int32, device=self.device)
        if conf is None:
            conf = torch.empty(block - 1, dtype=torch.float32, device=self.device)
        if n_keep is None:
            n_keep = torch.empty(1, dtype=torch.int32, device=self.device)
        _lib.dflash_draft_block_gated(self.w.desc, self.kv.desc, p, anchor, mask_id, block,
                                      min_p, cand.data_ptr(), conf.data_ptr(),
                                      n_keep.data_ptr(), self.ws.data_ptr(), self.ws_bytes,
                                      stream_ptr())
        return cand, conf, n_keep

    def lm_head_argmax(self, hidden: torch.Tensor, cand: torch.Tensor,
                       logits: torch.Tensor | None = None) -> torch.Tensor:
        _lib.dflash_lm_head_argmax(self.w.desc, hidden.data_ptr(), hidden.shape[0],
                                   cand.data_ptr(),
                                   logits.data_ptr() if logits is not None else None,
                                   self.ws.data_ptr(), self.ws_bytes, stream_ptr())
        return cand

    def verify_gated(self, cand: torch.Tensor, target: torch.Tensor, k_max: int,
                     n_keep: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
        """Greedy verify of the first min(max(n_keep, 0), k_max) candidates,
        the count read on the device."""
        if out is None:
            out = torch.empty(2, dtype=torch.int32, device=self.device)
        _lib.dflash_verify_greedy_gated(cand.data_ptr(), target.data_ptr(), k_max,
                                        n_keep.data_ptr(), out.data_ptr(), stream_ptr())
        return out

    def status(self, out: torch.Tensor | None = None) -> torch.Tensor:
        """Device word: DFLASH_OK, DFLASH_ETIMEOUT if the last pass gave up
        waiting at a grid barrier, or DFLASH_EINVAL if it found its
        device-resident positions invalid."""
        if out is None:
            out = torch.empty(1, dtype=torch.int32, device=self.device)
        _lib.dflash_draft_status(self.ws_ptr, self.ws_bytes, out.data_ptr(), stream_ptr())
        return out

    def stage(self, stage: int, index: int, rows: int) -> torch.Tensor:
        """Copy of one intermediate of the last pass run in this workspace
        (dflash_draft_stage): fp32 [rows][2560] for the residual stream,
        16-bit [rows][n] otherwise (raw bits as int16)."""
        width = {_lib.DFLASH_STAGE_RESIDUAL: 2560, _lib.DFLASH_STAGE_QKV: 7168,
                 _lib.DFLASH_STAGE_ATTN: 6144, _lib.DFLASH_STAGE_MLP: 7680}[stage]
        dt = torch.float32 if stage == _lib.DFLASH_STAGE_RESIDUAL else torch.int16
        out = torch.empty((rows, width), dtype=dt, device=self.device)
        _lib.dflash_draft_stage(self.ws_ptr, self.ws_bytes, stage, index, rows, out.data_ptr(),
                                out.numel() * out.element_size(), stream_ptr())
        return out

    def verify(self, cand: torch.Tensor, target: torch.Tensor, k: int,
               out: torch.Tensor | None = None) -> torch.Tensor:
        if out is None:
            out = torch.empty(2, dtype=torch.int32, device=self.device)
        dflash_verify_greedy(cand.data_ptr(), target.data_ptr(), k, out.data_ptr(),
                             stream_ptr())
        return out
