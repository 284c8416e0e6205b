"""The paired backward (each dgrad beside its weight gradient in one launch:
the default in bf16, MOE_FLAG_OVERLAP_BWD in the FP8 modes) against the
one-kernel-per-GEMM backward (MOE_FLAG_SERIAL_BWD) and against the CPU oracle,
through the C ABI.

Both backwards run the same tile code in the same accumulation order, so every
backward output and intermediate must agree bit for bit; the paired path is
also held to the oracle directly (1e-2 per output and intermediate).  Cases:
uniform and Zipf-skewed routing with dead experts, a run of out-of-range ids,
and the full 30B layer.
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

CASES = ["mid_bf16", "wide_bf16", "zipf_wide_bf16", "deep_bf16"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    moe.lib()


def _run(cfg, inp, flags):
    L = Layer(cfg, inp, flags=flags)
    L.prepare()
    L.fwd()
    L.bwd()
    rc = L.check()
    torch.cuda.synchronize()
    out = {k: getattr(L, k).clone() for k in ("dx", "dw1", "dw2", "dprob")}
    out["dh"] = L.view_dev(moe.MOE_VIEW_DH, 2 * cfg.F).clone()
    out["dxp"] = L.view_dev(moe.MOE_VIEW_DXPERM, cfg.D).clone()
    return rc, out


def _same(a, b, n_rows):
    for k in a:
        x, y = a[k], b[k]
        if k in ("dh", "dxp"):
            x, y = x[:n_rows], y[:n_rows]
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), k


@pytest.mark.parametrize("name", CASES)
def test_paired_backward_is_bitwise_the_default(name):
    cfg = mi.CONFIGS[name]
    inp = mi.make_inputs(cfg)
    print(f"[case] paired backward {name}", flush=True)
    rc0, base = _run(cfg, inp, moe.MOE_FLAG_SERIAL_BWD)
    rc1, pair = _run(cfg, inp, moe.MOE_FLAG_OVERLAP_BWD)
    assert rc0 == moe.MOE_OK and rc1 == moe.MOE_OK
    nv = int(np.bincount(inp["topk_idx"].ravel(), minlength=cfg.E).sum())
    _same(base, pair, nv)


@pytest.mark.parametrize("name", CASES)
def test_paired_backward_matches_oracle(name):
    cfg = mi.CONFIGS[name]
    print(f"[case] paired backward vs oracle {name}", flush=True)
    layer_vs_oracle(cfg, mi.make_inputs(cfg), moe.MOE_FLAG_OVERLAP_BWD)


def test_paired_backward_with_out_of_range_ids():
    cfg = mi.CONFIGS["mid_bf16"]
    inp = mi.make_inputs(cfg)
    idx = inp["topk_idx"].copy()
    idx[:37, 0] = cfg.E + 2
    idx[100, 1] = -1
    inp = dict(inp, topk_idx=idx)
    print("[case] paired backward, out-of-range ids", flush=True)
    rc0, base = _run(cfg, inp, moe.MOE_FLAG_SERIAL_BWD)
    rc1, pair = _run(cfg, inp, moe.MOE_FLAG_OVERLAP_BWD)
    assert rc0 == moe.MOE_EINDEX and rc1 == moe.MOE_EINDEX
    _same(base, pair, int(((idx >= 0) & (idx < cfg.E)).sum()))


def test_paired_backward_twice_on_one_forward():
    """The ticket counters start from zero on every backward."""
    cfg = mi.CONFIGS["wide_bf16"]
    inp = mi.make_inputs(cfg)
    L = Layer(cfg, inp, flags=moe.MOE_FLAG_OVERLAP_BWD)
    L.fwd()
    L.bwd()
    first = {k: getattr(L, k).clone() for k in ("dx", "dw1", "dw2", "dprob")}
    L.bwd()
    assert L.check() == moe.MOE_OK
    torch.cuda.synchronize()
    for k, v in first.items():
        assert torch.equal(getattr(L, k).view(torch.uint8), v.view(torch.uint8)), k


@pytest.mark.timeout(600)
def test_paired_backward_full_size_30b():
    cfg = mi.CONFIGS["30b"]
    inp = mi.make_inputs(cfg, threads=16)
    print("[case] paired backward 30b bitwise", flush=True)
    rc1, pair = _run(cfg, inp, moe.MOE_FLAG_OVERLAP_BWD)
    pair = {k: v.cpu() for k, v in pair.items()}
    torch.cuda.empty_cache()
    rc0, base = _run(cfg, inp, moe.MOE_FLAG_SERIAL_BWD)
    base = {k: v.cpu() for k, v in base.items()}
    assert rc0 == moe.MOE_OK and rc1 == moe.MOE_OK
    _same(base, pair, cfg.N)


@pytest.mark.timeout(600)
def test_paired_backward_full_size_30b_matches_oracle():
    full_size_vs_oracle("30b", ntok=24, nexp=2, flags=moe.MOE_FLAG_OVERLAP_BWD)


FP8_CASES = ["fp8bwd_small", "mxfp8_small", "fp8_small", "mxfp8_zipf_small"]


@pytest.mark.parametrize("name", FP8_CASES)
def test_paired_fp8_backward_is_bitwise_the_default_and_the_recipe(name):
    """FP8 modes: the paired backward quantises dYw over tokens into a third
    buffer (the W2 dgrad still reads dYw's row codes) and runs the same tiles:
    bit-identical to the default, and within 2e-2 of the FP8-recipe oracle."""
    from oracle import fp8_layer_oracle as fl
    from tests.layer_harness import rel_err, to_host
    cfg = mi.CONFIGS[name]
    inp = mi.make_inputs(cfg)
    print(f"[case] paired FP8 backward {name}", flush=True)
    rc0, base = _run(cfg, inp, moe.MOE_FLAG_SERIAL_BWD)
    rc1, pair = _run(cfg, inp, moe.MOE_FLAG_OVERLAP_BWD)
    assert rc0 == moe.MOE_OK and rc1 == moe.MOE_OK
    nv = int(np.bincount(inp["topk_idx"].ravel(), minlength=cfg.E).sum())
    _same(base, pair, nv)
    recipe = {mi.MODE_FP8_BWD: "fp8_bwd", mi.MODE_FP8: "fp8", mi.MODE_MXFP8: "mxfp8"}[cfg.mode]
    ref = fl.layer(recipe, inp["x"], inp["topk_idx"], inp["topk_w"], inp["dy"], inp["w1"], inp["w2"])
    for k in ("dx", "dw1", "dw2", "dprob"):
        e = rel_err(to_host(pair[k]), ref[k])
        assert e <= 2e-2, (k, e)


@pytest.mark.parametrize("name,paired", [("mid_bf16", True), ("deep_bf16", False),
                                         ("fp8bwd_small", False), ("mxfp8_small", False)])
def test_default_backward_schedule(name, paired):
    """bf16 pairs its backward GEMMs by default while experts average at most
    4096 routed rows; larger experts and the FP8 modes launch one kernel per
    GEMM unless asked (the kernels the opt-in profiler saw)."""
    cfg = mi.CONFIGS[name]
    L = Layer(cfg, mi.make_inputs(cfg))
    L.prepare()
    L.fwd()
    torch.cuda.synchronize()
    moe.moe_profile_reset()
    moe.moe_profile_enable(True)
    L.bwd()
    torch.cuda.synchronize()
    moe.moe_profile_enable(False)
    names = set(moe.moe_profile_collect())
    moe.moe_profile_reset()
    assert L.check() == moe.MOE_OK
    assert ("pair_w2" in names and "pair_w1" in names) == paired, names
    assert ("gemm_w2_wgrad" in names) == (not paired), names
