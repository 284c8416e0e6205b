"""Activation recompute (MOE_FLAG_RECOMPUTE) against the default path, through
the C ABI.

With the flag the forward keeps no H and the backward rebuilds it with the
forward's own W1 GEMM (same kernel, operands and accumulation order), so every
output and every saved or backward intermediate must agree bit for bit with
the default path.  The recompute path is also checked against the CPU oracle
directly: every output and intermediate within 1e-2 (1e-4 in the fp32 mode)
on the small shapes, and sampled tokens and weight-gradient rows of the full
30B layer.
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

CASES = ["tiny", "tiny_bf16gemm", "mid_bf16", "wide_bf16", "zipf_bf16", "fp8bwd_small",
         "mxfp8_small", "fp8_small"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    moe.lib()


def _run(cfg, inp, flags):
    L = Layer(cfg, inp, flags=flags)
    L.prepare()
    L.fwd()
    dt = torch.float32 if cfg.mode == moe.MOE_FP32 else torch.bfloat16  # intermediates' dtype
    fwd_views = {"a": L.view_dev(moe.MOE_VIEW_A, cfg.F, dt).clone(),
                 "o": L.view_dev(moe.MOE_VIEW_O, cfg.D, dt).clone(),
                 "y": L.y.clone()}
    L.bwd()
    rc = L.check()
    torch.cuda.synchronize()
    out = {k: getattr(L, k).clone() for k in ("dx", "dw1", "dw2", "dprob")}
    out.update(fwd_views)
    out["dh"] = L.view_dev(moe.MOE_VIEW_DH, 2 * cfg.F, dt).clone()
    return rc, out


def _same(a, b, n_rows):
    for k in a:
        x, y = a[k], b[k]
        if k in ("a", "o", "dh"):
            x, y = x[:n_rows], y[:n_rows]
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), k


@pytest.mark.parametrize("name", CASES)
def test_recompute_is_bitwise_the_default(name):
    cfg = mi.CONFIGS[name]
    inp = mi.make_inputs(cfg)
    print(f"[case] recompute {name} T={cfg.T} D={cfg.D} F={cfg.F} E={cfg.E} K={cfg.K} "
          f"mode={cfg.mode}", flush=True)
    rc0, base = _run(cfg, inp, 0)
    rc1, rec = _run(cfg, inp, moe.MOE_FLAG_RECOMPUTE)
    assert rc0 == moe.MOE_OK and rc1 == moe.MOE_OK
    nv = int(np.bincount(inp["topk_idx"].ravel(), minlength=cfg.E).sum())
    _same(base, rec, nv)


def test_recompute_with_the_overlapped_forward():
    cfg = mi.CONFIGS["mid_bf16"]
    inp = mi.make_inputs(cfg)
    print("[case] recompute + overlap mid_bf16", flush=True)
    rc0, base = _run(cfg, inp, 0)
    rc1, rec = _run(cfg, inp, moe.MOE_FLAG_RECOMPUTE | moe.MOE_FLAG_OVERLAP)
    assert rc0 == moe.MOE_OK and rc1 == moe.MOE_OK
    _same(base, rec, cfg.N)


@pytest.mark.timeout(600)
def test_recompute_full_size_30b():
    cfg = mi.CONFIGS["30b"]
    inp = mi.make_inputs(cfg)
    print("[case] recompute 30b", flush=True)
    rc1, rec = _run(cfg, inp, moe.MOE_FLAG_RECOMPUTE)
    rec = {k: v.cpu() for k, v in rec.items()}
    torch.cuda.empty_cache()
    rc0, base = _run(cfg, inp, 0)
    base = {k: v.cpu() for k, v in base.items()}
    assert rc0 == moe.MOE_OK and rc1 == moe.MOE_OK
    _same(base, rec, cfg.N)


@pytest.mark.parametrize("name", [c for c in CASES if mi.CONFIGS[c].mode in
                                  (mi.MODE_FP32, mi.MODE_FP32_BF16GEMM, mi.MODE_BF16)])
def test_recompute_matches_oracle(name):
    cfg = mi.CONFIGS[name]
    print(f"[case] recompute vs oracle {name}", flush=True)
    layer_vs_oracle(cfg, mi.make_inputs(cfg), moe.MOE_FLAG_RECOMPUTE)


def test_recompute_with_overlap_matches_oracle():
    cfg = mi.CONFIGS["mid_bf16"]
    print("[case] recompute + overlap vs oracle mid_bf16", flush=True)
    layer_vs_oracle(cfg, mi.make_inputs(cfg), moe.MOE_FLAG_RECOMPUTE | moe.MOE_FLAG_OVERLAP)


@pytest.mark.timeout(600)
def test_recompute_full_size_30b_matches_oracle():
    full_size_vs_oracle("30b", ntok=24, nexp=2, flags=moe.MOE_FLAG_RECOMPUTE)
