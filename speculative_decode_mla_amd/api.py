"""Torch-facing binding of the MLA verify-attention library.

PyTorch supplies device memory and the stream; every step of the computation
runs in the HIP kernels of libmla_verify.so.  Functions here only check shapes
and dtypes on the host and pass raw pointers through the C ABI.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib

D_QK = _lib.D_QK
D_V = _lib.D_V
DEFAULT_SCALE = 1.0 / math.sqrt(192.0)


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, dim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")


class MlaVerify:
    """A handle: shapes fixed at creation, split workspace owned by the library.

    run() enqueues the two kernels on the current (or given) stream and returns
    without synchronising, so it can be captured in a torch.cuda.CUDAGraph.
    `form` picks kernel 1's layout (FORM_AUTO, FORM_128ROW, FORM_TWO_STREAM or FORM_FOUR_STREAM
    from _lib); the result is the same up to rounding, only the speed differs.
    `batch_invariant` makes each request's result bitwise independent of its batchmates
    (MLA_VERIFY_FLAG_BATCH_INVARIANT: no range plan).  `debug` runs the handle on the debug build
    of the library, whose kernels clamp out-of-range slots and lengths and record them
    (debug_flags()).
    """

    def __init__(self, num_heads: int, batch: int, max_q_len: int, max_nsplit: int, num_slots: int,
                 sm_scale: float = DEFAULT_SCALE, form: int = _lib.FORM_AUTO, batch_invariant: bool = False,
                 debug: bool = False):
        lib = self._lib = _lib.load(debug)
        flags = _lib.FLAG_BATCH_INVARIANT if batch_invariant else 0
        self.cfg = _lib.MlaVerifyConfig(num_heads, D_QK, D_V, batch, max_q_len, max_nsplit, num_slots, sm_scale,
                                        form, flags)
        h = ctypes.c_void_p()
        _lib.check("mla_verify_create", lib.mla_verify_create(ctypes.byref(self.cfg), ctypes.byref(h)))
        self._h = h
        self.num_heads, self.batch, self.max_q_len = num_heads, batch, max_q_len
        self.max_nsplit, self.num_slots = max_nsplit, num_slots

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value is not None:
            _lib.check("mla_verify_destroy", self._lib.mla_verify_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def debug_flags(self, clear: bool = True) -> int:
        """The debug build's flag word (MLA_VERIFY_DEBUG_* bits) after a device synchronisation."""
        v = ctypes.c_int32()
        _lib.check("mla_verify_debug_flags", self._lib.mla_verify_debug_flags(self._h, ctypes.byref(v), int(clear)))
        return v.value

    def workspace(self):
        """(o_part pointer, its bytes, lse_part pointer, its bytes) of the handle's split workspace
        (device memory the library owns; see mla_verify_workspace)."""
        op, lp = ctypes.c_void_p(), ctypes.c_void_p()
        ob, lb = ctypes.c_int64(), ctypes.c_int64()
        _lib.check("mla_verify_workspace", self._lib.mla_verify_workspace(
            self._h, ctypes.byref(op), ctypes.byref(ob), ctypes.byref(lp), ctypes.byref(lb)))
        return op.value, ob.value, lp.value, lb.value

    def _check_inputs(self, q, kv_pool, slot_idx, seq_lens, q_lens):
        H = self.num_heads
        _need(q, "q", torch.bfloat16, 3)
        _need(kv_pool, "kv_pool", torch.bfloat16, 2)
        _need(slot_idx, "slot_idx", torch.int32, 1)
        _need(seq_lens, "seq_lens", torch.int32, 1)
        _need(q_lens, "q_lens", torch.int32, 1)
        if q.shape[1:] != (H, D_QK):
            raise ValueError(f"q must be [T_q, {H}, {D_QK}], got {tuple(q.shape)}")
        if kv_pool.shape[1] != D_QK or kv_pool.shape[0] > self.num_slots:
            raise ValueError(f"kv_pool must be [<= {self.num_slots}, {D_QK}], got {tuple(kv_pool.shape)}")
        if seq_lens.shape[0] != self.batch or q_lens.shape[0] != self.batch:
            raise ValueError(f"seq_lens and q_lens must have {self.batch} entries")

    def partials(self, q, kv_pool, slot_idx, seq_lens, q_lens, nsplit: int, stream=None):
        """Kernel 1 only: split partials into the handle's workspace."""
        self._check_inputs(q, kv_pool, slot_idx, seq_lens, q_lens)
        st = self._lib.mla_verify_partials(self._h, _ptr(q), _ptr(kv_pool), _ptr(slot_idx), _ptr(seq_lens),
                                             _ptr(q_lens), int(nsplit), _stream_handle(stream))
        _lib.check("mla_verify_partials", st)

    def run(self, q, kv_pool, slot_idx, seq_lens, q_lens, out, lse, nsplit: int, stream=None):
        """out[T_q, H, 512] (bf16) and lse[T_q, H] (fp32) for one verify step."""
        H = self.num_heads
        _need(q, "q", torch.bfloat16, 3)
        _need(kv_pool, "kv_pool", torch.bfloat16, 2)
        _need(slot_idx, "slot_idx", torch.int32, 1)
        _need(seq_lens, "seq_lens", torch.int32, 1)
        _need(q_lens, "q_lens", torch.int32, 1)
        _need(out, "out", torch.bfloat16, 3)
        _need(lse, "lse", torch.float32, 2)
        if q.shape[1:] != (H, D_QK):
            raise ValueError(f"q must be [T_q, {H}, {D_QK}], got {tuple(q.shape)}")
        if kv_pool.shape[1] != D_QK or kv_pool.shape[0] > self.num_slots:
            raise ValueError(f"kv_pool must be [<= {self.num_slots}, {D_QK}], got {tuple(kv_pool.shape)}")
        if seq_lens.shape[0] != self.batch or q_lens.shape[0] != self.batch:
            raise ValueError(f"seq_lens and q_lens must have {self.batch} entries")
        if out.shape != (q.shape[0], H, D_V):
            raise ValueError(f"out must be [{q.shape[0]}, {H}, {D_V}], got {tuple(out.shape)}")
        if lse.shape != (q.shape[0], H):
            raise ValueError(f"lse must be [{q.shape[0]}, {H}], got {tuple(lse.shape)}")
        st = self._lib.mla_verify_run(self._h, _ptr(q), _ptr(kv_pool), _ptr(slot_idx), _ptr(seq_lens), _ptr(q_lens),
                                        _ptr(out), _ptr(lse), int(nsplit), _stream_handle(stream))
        _lib.check("mla_verify_run", st)
        return out, lse


def run_noalloc(q, kv_pool, slot_idx, seq_lens, q_lens, out, lse, nsplit: int, num_heads: int, batch: int,
                max_q_len: int, max_nsplit: int, num_slots: int, sm_scale: float = DEFAULT_SCALE,
                form: int = _lib.FORM_AUTO, batch_invariant: bool = False, stream=None):
    """mla_verify_run_noalloc: one verify call with no handle and no allocation (the split partials
    live in the library's fixed per-GPU scratch array).  Shapes as for MlaVerify(...).run(...)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(kv_pool, "kv_pool", torch.bfloat16, 2)
    _need(slot_idx, "slot_idx", torch.int32, 1)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(q_lens, "q_lens", torch.int32, 1)
    _need(out, "out", torch.bfloat16, 3)
    _need(lse, "lse", torch.float32, 2)
    if q.shape[1:] != (num_heads, D_QK) or out.shape != (q.shape[0], num_heads, D_V) or \
            lse.shape != (q.shape[0], num_heads):
        raise ValueError("q, out and lse must be [T_q, H, 576], [T_q, H, 512] and [T_q, H]")
    if kv_pool.shape[1] != D_QK or kv_pool.shape[0] > num_slots:
        raise ValueError(f"kv_pool must be [<= {num_slots}, {D_QK}], got {tuple(kv_pool.shape)}")
    if seq_lens.shape[0] != batch or q_lens.shape[0] != batch:
        raise ValueError(f"seq_lens and q_lens must have {batch} entries")
    cfg = _lib.MlaVerifyConfig(num_heads, D_QK, D_V, batch, max_q_len, max_nsplit, num_slots, sm_scale, form,
                               _lib.FLAG_BATCH_INVARIANT if batch_invariant else 0)
    st = _lib.load().mla_verify_run_noalloc(ctypes.byref(cfg), _ptr(q), _ptr(kv_pool), _ptr(slot_idx),
                                            _ptr(seq_lens), _ptr(q_lens), _ptr(out), _ptr(lse), int(nsplit),
                                            _stream_handle(stream))
    _lib.check("mla_verify_run_noalloc", st)
    return out, lse


def compact(kv_pool, slot_idx, dst_pool, dst_first: int, new_slot_idx=None, stream=None):
    """KV compaction: dst_pool[dst_first + j] = kv_pool[slot_idx[j]]; new_slot_idx[j] = dst_first + j.

    kv_pool, dst_pool bf16 [*, 576]; slot_idx int32 [n]; new_slot_idx int32 [n] or None.
    """
    _need(kv_pool, "kv_pool", torch.bfloat16, 2)
    _need(dst_pool, "dst_pool", torch.bfloat16, 2)
    _need(slot_idx, "slot_idx", torch.int32, 1)
    if kv_pool.shape[1] != D_QK or dst_pool.shape[1] != D_QK:
        raise ValueError(f"pools must be [*, {D_QK}]")
    n = slot_idx.shape[0]
    if new_slot_idx is not None:
        _need(new_slot_idx, "new_slot_idx", torch.int32, 1)
        if new_slot_idx.shape[0] != n:
            raise ValueError("new_slot_idx must have one entry per slot")
    st = _lib.load().mla_verify_compact(_ptr(kv_pool), _ptr(slot_idx), n, _ptr(dst_pool), dst_pool.shape[0],
                                        int(dst_first), _ptr(new_slot_idx) if new_slot_idx is not None else None,
                                        _stream_handle(stream))
    _lib.check("mla_verify_compact", st)
    return dst_pool, new_slot_idx


def build_metadata(req_to_token, req_ids, prefix_lens, draft_lens, slot_idx, seq_lens, q_lens, status,
                   table_width=None, stream=None):
    """Step metadata on the device (see mla_verify_build_metadata): all int32 device tensors;
    req_to_token [rows, stride], slot_idx [capacity], status [1]."""
    for t, name in ((req_ids, "req_ids"), (prefix_lens, "prefix_lens"), (draft_lens, "draft_lens"),
                    (slot_idx, "slot_idx"), (seq_lens, "seq_lens"), (q_lens, "q_lens"), (status, "status")):
        _need(t, name, torch.int32, 1)
    _need(req_to_token, "req_to_token", torch.int32, 2)
    batch = req_ids.shape[0]
    if prefix_lens.shape[0] != batch or draft_lens.shape[0] != batch or seq_lens.shape[0] < batch \
            or q_lens.shape[0] < batch or status.shape[0] < 1:
        raise ValueError("inconsistent metadata shapes")
    rows, stride = req_to_token.shape
    st = _lib.load().mla_verify_build_metadata(
        _ptr(req_to_token), rows, stride if table_width is None else int(table_width), stride, _ptr(req_ids),
        _ptr(prefix_lens), _ptr(draft_lens), batch, _ptr(slot_idx), slot_idx.shape[0], _ptr(seq_lens), _ptr(q_lens),
        _ptr(status), _stream_handle(stream))
    _lib.check("mla_verify_build_metadata", st)


def merge(o_part, lse_part, q_lens, out, lse, stream=None):
    """Kernel 2 alone: reduce caller-provided split partials.

    o_part fp32 [B, S, max_q_len*H, 512], lse_part fp32 [B, S, max_q_len*H] (natural log).
    """
    _need(o_part, "o_part", torch.float32, 4)
    _need(lse_part, "lse_part", torch.float32, 3)
    _need(q_lens, "q_lens", torch.int32, 1)
    _need(out, "out", torch.bfloat16, 3)
    _need(lse, "lse", torch.float32, 2)
    B, S, rows, dv = o_part.shape
    H = out.shape[1]
    if dv != D_V or rows % H or lse_part.shape != (B, S, rows) or q_lens.shape[0] != B:
        raise ValueError("inconsistent partial shapes")
    st = _lib.load().mla_verify_merge(_ptr(o_part), _ptr(lse_part), _ptr(q_lens), B, H, rows // H, S,
                                      _ptr(out), _ptr(lse), _stream_handle(stream))
    _lib.check("mla_verify_merge", st)
    return out, lse
