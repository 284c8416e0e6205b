"""The overlapped forward (dispatch + W1 + SwiGLU + W2 in one launch over ticket
queues) against the one-kernel-per-step forward, through the C ABI.

Both paths run the same tile code in the same accumulation order, so every
forward output and intermediate must agree bit for bit; the per-step path is
itself checked against the oracle in test_gpu_parity.py.  Also: the bounded
waits report MOE_ETIMEOUT (forced from the host with the diagnostics flag,
so every kernel still exits normally).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_layer_31_amd as moe
import moe_inputs as mi
from tests.layer_harness import Layer

pytestmark = pytest.mark.gpu

QUEUE_CASES = ["mid_bf16", "wide_bf16", "mid_f32io", "zipf_bf16", "fp8bwd_small"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    moe.lib()


def _views(L):
    cfg = L.cfg
    D, F = cfg.D, cfg.F
    out = {"y": L.y.clone()}
    for name, which, cols, dt in (("xperm", moe.MOE_VIEW_XPERM, D, None),
                                  ("wperm", moe.MOE_VIEW_WPERM, 0, torch.float32),
                                  ("h", moe.MOE_VIEW_H, 2 * F, None),
                                  ("a", moe.MOE_VIEW_A, F, None),
                                  ("o", moe.MOE_VIEW_O, D, None)):
        out[name] = L.view_dev(which, cols, dt).clone()
    return out


def _fwd(cfg, inp, flags):
    L = Layer(cfg, inp, flags=flags)
    L.prepare()
    L.fwd()
    rc = L.check()
    torch.cuda.synchronize()
    return L, rc


def _assert_same(a, b, n_rows):
    for k in a:
        x, y = a[k], b[k]
        if k not in ("y",):
            x, y = x[:n_rows], y[:n_rows]
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), k


@pytest.mark.parametrize("name", QUEUE_CASES)
def test_queue_forward_is_bitwise_the_per_step_forward(name):
    cfg = mi.CONFIGS[name]
    inp = mi.make_inputs(cfg)
    print(f"[case] {name} T={cfg.T} D={cfg.D} F={cfg.F} E={cfg.E} K={cfg.K} mode={cfg.mode}",
          flush=True)
    Lq, rcq = _fwd(cfg, inp, moe.MOE_FLAG_OVERLAP)
    Ls, rcs = _fwd(cfg, inp, 0)
    assert rcq == moe.MOE_OK and rcs == moe.MOE_OK
    nv = int(np.bincount(inp["topk_idx"].ravel(), minlength=cfg.E).sum())
    _assert_same(_views(Lq), _views(Ls), nv)
    # the backward on the persistent forward's saved state matches too
    Lq.bwd()
    Ls.bwd()
    torch.cuda.synchronize()
    for k in ("dx", "dw1", "dw2", "dprob"):
        assert torch.equal(getattr(Lq, k).view(torch.uint8), getattr(Ls, k).view(torch.uint8)), k


def test_queue_forward_with_out_of_range_indices():
    cfg = mi.CONFIGS["mid_bf16"]
    inp = mi.make_inputs(cfg)
    idx = inp["topk_idx"].copy()
    idx[5, 0] = cfg.E + 3
    idx[611, 1] = -1
    inp = dict(inp, topk_idx=idx)
    Lq, rcq = _fwd(cfg, inp, moe.MOE_FLAG_OVERLAP)
    Ls, rcs = _fwd(cfg, inp, 0)
    assert rcq == moe.MOE_EINDEX and rcs == moe.MOE_EINDEX
    nv = int(((idx >= 0) & (idx < cfg.E)).sum())
    _assert_same(_views(Lq), _views(Ls), nv)


def test_queue_timeout_is_reported_then_cleared():
    cfg = mi.CONFIGS["mid_bf16"]
    inp = mi.make_inputs(cfg)
    L, rc = _fwd(cfg, inp, moe.MOE_FLAG_OVERLAP | moe.MOE_FLAG_QUEUE_TIMEOUT_TEST)
    assert rc == moe.MOE_ETIMEOUT
    assert L.check() == moe.MOE_OK  # cleared by the read
    L2, rc2 = _fwd(cfg, inp, moe.MOE_FLAG_OVERLAP)
    assert rc2 == moe.MOE_OK


@pytest.mark.timeout(600)
def test_queue_forward_full_size_30b_bitwise():
    cfg = mi.CONFIGS["30b"]
    inp = mi.make_inputs(cfg)
    print("[case] 30b queue vs per-step forward", flush=True)
    Lq, rcq = _fwd(cfg, inp, moe.MOE_FLAG_OVERLAP)
    vq = _views(Lq)
    del Lq
    torch.cuda.empty_cache()
    Ls, rcs = _fwd(cfg, inp, 0)
    assert rcq == moe.MOE_OK and rcs == moe.MOE_OK
    _assert_same(vq, _views(Ls), cfg.N)
