"""Can any FP8 kernel meet max|err|/max|ref| <= 5e-2 against the plain oracle?

The FP8-recipe oracle (oracle/fp8_layer_oracle.py) computes the layer with
every FP8 GEMM operand quantised exactly (e4m3 codes and scales from the
oracle's codecs, float64 products) and the stored intermediates rounded once
to bf16.  Its distance from the unquantised oracle is the error of the number
format itself, before any kernel: a kernel that reproduced the recipe exactly
would show the same distance.  These CPU tests measure it, on the small FP8
parity workloads whole and on sampled experts of the full Qwen3 shapes, and
pin which bound the recipe can meet:

* MXFP8 and blockwise FP8 in both passes: the recipe itself exceeds 5e-2 on
  several outputs (0.055-0.08), so the literal bound is out of reach for these
  modes and the GPU test of it is an expected failure;
* fp8_bwd (bf16 forward): the forward outputs stay at bf16 accuracy, and the
  backward ones sit at the bound (0.03-0.054): dW1 exceeds it on the small
  parity workload and on the sampled 235B experts (0.052-0.054), while dX
  stays just under it (0.046-0.050).

With `experts`, the oracle keeps only the rows routed to those experts (every
quantiser works per row, per weight or per expert segment, so they are the
full layer's rows), and y, dx and dprob hold those experts' contributions.
"""
import numpy as np
import pytest

import moe_inputs as mi
from oracle import fp8_layer_oracle as fl

RECIPE = {mi.MODE_FP8_BWD: "fp8_bwd", mi.MODE_FP8: "fp8", mi.MODE_MXFP8: "mxfp8"}
FWD = ("y", "h", "a", "o", "dprob")
BWD = ("dx", "dw1", "dw2", "dh", "dxp")
TOL_FP8 = 5e-2


def _rel(a, b):
    return float(np.abs(a - b).max() / np.abs(b).max())


def recipe_errors(name, experts=None):
    cfg = mi.CONFIGS[name]
    inp = mi.make_inputs(cfg, experts=experts)
    args = (inp["x"], inp["topk_idx"], inp["topk_w"], inp["dy"], inp["w1"], inp["w2"])
    q = fl.layer(RECIPE[cfg.mode], *args, experts=experts)
    plain = fl.layer(RECIPE[cfg.mode], *args, quantiser=fl.identity_quantiser,
                     store_bf16=False, experts=experts)
    errs = {k: _rel(q[k], plain[k]) for k in FWD + BWD}
    print(name, experts, {k: round(v, 4) for k, v in errs.items()}, flush=True)
    return cfg, errs


def _sampled_experts(cfg):
    """The least-routed live expert and the median-routed one."""
    idx, _ = mi.make_routing(cfg)
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    live = np.nonzero(counts)[0]
    order = live[np.argsort(counts[live], kind="stable")]
    return sorted({int(order[0]), int(order[len(order) // 2])})


def _check(cfg, errs):
    if cfg.mode == mi.MODE_FP8_BWD:
        # bf16 forward: only the storage rounding of the intermediates
        for k in FWD:
            assert errs[k] <= 1e-2, (k, errs[k])
        # the FP8 backward alone takes the weight gradient over the bound
        assert TOL_FP8 < max(errs[k] for k in BWD) < 0.06
    else:
        # every GEMM quantised: the format error alone exceeds the bound
        assert max(errs.values()) > TOL_FP8 + 5e-3
        assert max(errs.values()) < 0.1


@pytest.mark.parametrize("name", ["fp8bwd_small", "mxfp8_small", "fp8_small", "mxfp8_zipf_small"])
def test_recipe_error_on_the_small_fp8_workloads(name):
    cfg, errs = recipe_errors(name)
    _check(cfg, errs)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["30b_mxfp8", "30b_fp8", "235b_fp8bwd"])
def test_recipe_error_at_full_size(name):
    cfg = mi.CONFIGS[name]
    _, errs = recipe_errors(name, _sampled_experts(cfg))
    _check(cfg, errs)
