"""The overlapped forward (dispatch + W1 + SwiGLU + W2 in one launch over ticket
queues) against the one-kernel-per-step forward, through the C ABI.

Both paths run the same tile code in the same accumulation order, so every
forward output and intermediate must agree bit for bit.  The overlapped path
is also checked against the CPU oracle directly, as the per-step path is:
every output and intermediate within 1e-2 (1e-4 with fp32 I/O is not used:
the overlapped forward runs only bf16 GEMMs), on the small shapes and on
sampled tokens and weight-gradient rows of the full 30B layer.  Also: the
bounded waits report MOE_ETIMEOUT (forced from the host with the diagnostics
flag, so every kernel still exits normally).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_layer_31_amd as moe
import moe_inputs as mi
from tests.layer_harness import Layer
from tests.oracle_parity import full_size_vs_oracle, layer_vs_oracle

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


@pytest.mark.parametrize("name", QUEUE_CASES)
def test_queue_forward_matches_oracle(name):
    cfg = mi.CONFIGS[name]
    print(f"[case] overlapped forward vs oracle {name}", flush=True)
    if cfg.mode == mi.MODE_FP8_BWD:
        pytest.skip("FP8 backward: held to the FP8-recipe oracle (test_gpu_fp8.py); the "
                    "bitwise test above ties this path to that one")
    layer_vs_oracle(cfg, mi.make_inputs(cfg), moe.MOE_FLAG_OVERLAP)


@pytest.mark.timeout(600)
def test_queue_forward_full_size_30b_matches_oracle():
    full_size_vs_oracle("30b", ntok=24, nexp=2, flags=moe.MOE_FLAG_OVERLAP)


@pytest.mark.parametrize("name", QUEUE_CASES + ["30b"])
def test_queue_tables_equal_the_host_mirror(name):
    """The schedule queue_build_kernel writes (row bounds, dispatch-item and
    ticket-table bases, every table entry) equals the host mirror's, whose
    properties (bijection, same-queue smaller-ticket waits, capacities) the
    CPU tests check (tests/test_queue_tables.py)."""
    from oracle import moe_oracle as orc
    from tests import queue_tables as qt
    cfg = mi.CONFIGS[name]
    idx, w = mi.make_routing(cfg)
    inp = mi.make_inputs(cfg) if cfg.T < 5000 else None
    print(f"[case] queue tables {name}", flush=True)
    if inp is None:  # full size: only the forward's schedule matters, inputs of that routing
        inp = dict(x=np.zeros((cfg.T, cfg.D), np.float32), w1=np.zeros((cfg.E, 2 * cfg.F, cfg.D), np.float32),
                   w2=np.zeros((cfg.E, cfg.D, cfg.F), np.float32), topk_idx=idx, topk_w=w)
    L, rc = _fwd(cfg, inp, moe.MOE_FLAG_OVERLAP)
    assert rc == moe.MOE_OK
    ntn2, ntn3 = 2 * cfg.F // 256, cfg.D // 256
    ref = qt.build(orc.route(inp["topk_idx"], cfg.E)["offsets"], ntn2, ntn3)
    qt.check(ref, cfg.N)
    region = L.view_dev(moe.MOE_VIEW_QUEUE, 0, torch.uint8).cpu().numpy()
    off = qt.region_offsets(cfg.N, cfg.E, ntn2, ntn3)
    ctrl = region[off["ctrl"]:off["ctrl"] + 4 * qt.CTRL_WORDS].view(np.int32)
    X = qt.XCDS
    np.testing.assert_array_equal(ctrl[qt.CTRL_ROWS:qt.CTRL_ROWS + X + 1], ref["R"])
    np.testing.assert_array_equal(ctrl[qt.CTRL_CHUNK_BASE:qt.CTRL_CHUNK_BASE + X + 1], ref["CB"])
    np.testing.assert_array_equal(ctrl[qt.CTRL_BASES:qt.CTRL_BASES + X], ref["BASE"][:X])
    np.testing.assert_array_equal(ctrl[qt.CTRL_TOTALS:qt.CTRL_TOTALS + X], np.diff(ref["BASE"]))
    # every ticket taken: each queue's counter ran past its total
    assert np.all(ctrl[qt.CTRL_TICKETS:qt.CTRL_TICKETS + X] >= np.diff(ref["BASE"]))
    nt = ref["BASE"][X]
    table = region[off["table"]:off["table"] + 4 * nt].view(np.int32)
    np.testing.assert_array_equal(table, ref["table"])
