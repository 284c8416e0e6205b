"""Runs the HIP layer through the C ABI on seeded inputs and fetches its results.

Shared by the GPU tests, the smoke check and the benchmark.  Uses torch only to
allocate device memory, copy host arrays in and out, and supply the stream.
"""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_layer_31_amd as moe
import moe_inputs as mi


def desc_of(cfg: mi.LayerConfig, flags: int = 0) -> moe.moe_desc:
    return moe.make_desc(cfg.T, cfg.D, cfg.F, cfg.E, cfg.K, cfg.mode, flags)


def to_dev(a: np.ndarray, bf16: bool, device="cuda") -> torch.Tensor:
    if bf16:
        bits = mi.bf16_bits(np.ascontiguousarray(a, dtype=np.float32))
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return mi.from_bf16_bits(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


class Layer:
    """Device buffers of one layer workload and the calls that run it."""

    def __init__(self, cfg: mi.LayerConfig, inp: dict, flags: int = 0, device="cuda"):
        self.cfg = cfg
        self.desc = desc_of(cfg, flags)
        bf = cfg.io_is_bf16
        self.bf16 = bf
        self.x = to_dev(inp["x"], bf, device)
        self.w1 = to_dev(inp["w1"], bf, device)
        self.w2 = to_dev(inp["w2"], bf, device)
        self.dy = to_dev(inp["dy"], bf, device) if "dy" in inp else None
        self.idx = torch.from_numpy(np.ascontiguousarray(inp["topk_idx"])).to(device)
        self.w = torch.from_numpy(np.ascontiguousarray(inp["topk_w"])).to(device)
        dt = torch.bfloat16 if bf else torch.float32
        T, D = cfg.T, cfg.D
        self.y = torch.empty((T, D), dtype=dt, device=device)
        self.dx = torch.empty((T, D), dtype=dt, device=device)
        self.dw1 = torch.empty_like(self.w1)
        self.dw2 = torch.empty_like(self.w2)
        self.dprob = torch.empty((T, cfg.K), dtype=torch.float32, device=device)
        nb = moe.moe_scratch_bytes(self.desc)
        assert nb > 0
        self.scratch = torch.empty(nb, dtype=torch.uint8, device=device)
        wp = moe.moe_wprep_bytes(self.desc)
        self.wprep = torch.empty(wp, dtype=torch.uint8, device=device) if wp else None

    def prepare(self):
        moe.check(moe.moe_prepare_weights(self.desc, self.w1, self.w2, self.wprep), "prepare")

    def fwd(self):
        moe.check(moe.moe_fwd(self.desc, self.x, self.idx, self.w, self.w1, self.w2, self.wprep,
                              self.y, self.scratch), "moe_fwd")

    def bwd(self):
        moe.check(moe.moe_bwd(self.desc, self.dy, self.w, self.w1, self.w2, self.wprep, self.dx,
                              self.dw1, self.dw2, self.dprob, self.scratch), "moe_bwd")

    def check(self) -> int:
        return moe.moe_check(self.desc, self.scratch)

    def routing(self) -> dict:
        rc, counts, offsets, pos, src = moe.moe_routing_view(self.desc, self.scratch)
        moe.check(rc, "routing_view")
        base = self.scratch.data_ptr()
        E, N = self.cfg.E, self.cfg.N

        def grab(addr, n):
            off = addr - base
            return self.scratch[off:off + 4 * n].view(torch.int32).cpu().numpy().astype(np.int64)

        return dict(counts=grab(counts, E), offsets=grab(offsets, E + 1), pos=grab(pos, N),
                    src=grab(src, N))

    def view(self, which: int, cols: int, dtype=torch.bfloat16) -> np.ndarray:
        rc, addr, nbytes = moe.moe_scratch_view(self.desc, self.scratch, which)
        moe.check(rc, "scratch_view")
        off = addr - self.scratch.data_ptr()
        t = self.scratch[off:off + nbytes].view(dtype)
        return to_host(t).reshape(-1, cols) if cols else to_host(t)

    def view_dev(self, which: int, cols: int, dtype=None) -> torch.Tensor:
        """Device tensor over an intermediate inside the scratch (no copy)."""
        rc, addr, nbytes = moe.moe_scratch_view(self.desc, self.scratch, which)
        moe.check(rc, "scratch_view")
        off = addr - self.scratch.data_ptr()
        t = self.scratch[off:off + nbytes].view(dtype or torch.bfloat16)
        return t.reshape(-1, cols) if cols else t

    def outputs(self) -> dict:
        return dict(y=to_host(self.y), dx=to_host(self.dx), dw1=to_host(self.dw1),
                    dw2=to_host(self.dw2), dprob=to_host(self.dprob))


def rel_err(got, ref) -> float:
    """max|got - ref| / max|ref| (the parity metric)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))
