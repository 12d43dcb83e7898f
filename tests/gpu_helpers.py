"""Shared set-up for the GPU tests: move seeded inputs to the device and call the library."""
from __future__ import annotations

import numpy as np
import torch

from speculative_decode_mla_amd import inputs as I

OUT_TOL = 1e-2   # max |err| on the bf16 output
LSE_TOL = 1e-3   # max |err| on the fp32 log-sum-exp


def bits_to_bf16(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


class DeviceInputs:
    """Device copies of a VerifyInputs: the pool is NaN except at the referenced slots."""

    def __init__(self, x: I.VerifyInputs, device="cuda"):
        self.x = x
        self.q = bits_to_bf16(x.q, device)
        self.pool = torch.full((x.num_slots, I.D_QK), I.BF16_QNAN, dtype=torch.int16, device=device)
        slots = torch.from_numpy(x.slot_idx.astype(np.int64)).to(device)
        self.pool[slots] = torch.from_numpy(x.kv_rows.view(np.int16)).to(device)
        self.pool = self.pool.view(torch.bfloat16)
        self.slot_idx = torch.from_numpy(x.slot_idx).to(device)
        self.seq_lens = torch.from_numpy(x.seq_lens).to(device)
        self.q_lens = torch.from_numpy(x.q_lens).to(device)
        t_q = x.q.shape[0]
        self.out = torch.empty((t_q, x.heads, I.D_V), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((t_q, x.heads), dtype=torch.float32, device=device)

    def run(self, handle, nsplit):
        handle.run(self.q, self.pool, self.slot_idx, self.seq_lens, self.q_lens, self.out, self.lse, nsplit)
        return self.out, self.lse


def max_errors(out_gpu: torch.Tensor, lse_gpu: torch.Tensor, out_ref: np.ndarray, lse_ref: np.ndarray):
    o = bf16_to_f64(out_gpu)
    l = lse_gpu.cpu().numpy().astype(np.float64)
    finite = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(l), finite), "-inf pattern of lse differs"
    return float(np.max(np.abs(o - out_ref))), float(np.max(np.abs(l[finite] - lse_ref[finite]), initial=0.0))


class _DeviceArray:
    """A raw device allocation seen through __cuda_array_interface__ (torch wraps it without a copy)."""

    def __init__(self, ptr: int, nbytes: int, typestr: str, itemsize: int):
        self.__cuda_array_interface__ = {"shape": (nbytes // itemsize,), "typestr": typestr,
                                         "data": (ptr, False), "version": 2, "strides": None}


def workspace_tensors(handle):
    """The handle's split workspace as torch tensors sharing its memory: (o_part int16, lse_part fp32)."""
    op, ob, lp, lb = handle.workspace()
    o = torch.as_tensor(_DeviceArray(op, ob, "<i2", 2), device="cuda")
    l = torch.as_tensor(_DeviceArray(lp, lb, "<f4", 4), device="cuda")
    assert o.data_ptr() == op and l.data_ptr() == lp
    return o, l


def poison_workspace(handle):
    """Fill the workspace with NaN: bf16 0x7FC0 in every partial, fp32 NaN in every LSE."""
    o, l = workspace_tensors(handle)
    o.fill_(I.BF16_QNAN)
    l.fill_(float("nan"))
    torch.cuda.synchronize()
