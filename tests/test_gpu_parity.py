"""Parity of the HIP layer (through the C ABI) against the CPU oracle.

Integer routing arrays must be bit-exact; floating-point outputs and
intermediates must meet max|err| / max|ref| <= 1e-2 (bf16 GEMM operands and
bf16 storage, fp32 accumulation) against the fp64 oracle on the same inputs.
Dispatch copies (x_perm, dY_perm) and the permuted routing weights are
bit-exact copies.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_31_amd as moe
import moe_inputs as mi
from oracle import moe_oracle as orc
from tests.layer_harness import Layer
from tests.oracle_parity import full_size_vs_oracle, layer_vs_oracle, routing_bitexact, run

pytestmark = pytest.mark.gpu

SMALL = ["tiny", "tiny_bf16gemm", "small_bf16", "dead_bf16", "mid_bf16", "wide_bf16", "mid_f32io",
         "zipf_bf16", "rows4k_bf16", "rows8k_f32io", "deep_bf16"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    moe.lib()


@pytest.mark.parametrize("name", SMALL)
def test_layer_matches_oracle(name):
    cfg = mi.CONFIGS[name]
    inp = mi.make_inputs(cfg)
    print(f"[case] {name} T={cfg.T} D={cfg.D} F={cfg.F} E={cfg.E} K={cfg.K} mode={cfg.mode}",
          flush=True)
    layer_vs_oracle(cfg, inp)


def test_zero_token_experts_get_zero_wgrad():
    cfg = mi.CONFIGS["dead_bf16"]
    inp = mi.make_inputs(cfg)
    L = run(cfg, inp)
    counts = np.bincount(inp["topk_idx"].ravel(), minlength=cfg.E)
    dead = np.nonzero(counts == 0)[0]
    assert len(dead) == 4
    out = L.outputs()
    for e in dead:
        assert np.all(out["dw1"][e] == 0) and np.all(out["dw2"][e] == 0)


def test_run_to_run_bitwise_determinism():
    cfg = mi.CONFIGS["mid_bf16"]
    inp = mi.make_inputs(cfg)
    L = run(cfg, inp)
    first = L.outputs()
    for _ in range(3):
        L.fwd()
        L.bwd()
        torch.cuda.synchronize()
        again = L.outputs()
        for k in first:
            np.testing.assert_array_equal(again[k], first[k], err_msg=k)


def test_out_of_range_index_is_reported_and_skipped():
    cfg = mi.CONFIGS["small_bf16"]
    inp = mi.make_inputs(cfg)
    idx = inp["topk_idx"].copy()
    idx[3, 1] = cfg.E + 5
    idx[150, 0] = -2
    L = Layer(cfg, dict(inp, topk_idx=idx))
    moe.check(moe.moe_route(L.desc, L.idx, L.scratch), "route")
    assert L.check() == moe.MOE_EINDEX
    assert L.check() == moe.MOE_OK  # cleared
    got = L.routing()
    ref = orc.route(idx, cfg.E)
    assert ref["invalid"] == 2
    np.testing.assert_array_equal(got["pos"], ref["pos"])
    np.testing.assert_array_equal(got["counts"], ref["counts"])
    nv = int(ref["offsets"][-1])
    np.testing.assert_array_equal(got["src"][:nv], ref["src"])


@pytest.mark.parametrize("name", ["30b", "30b_mxfp8"])
def test_routing_full_size_bitexact(name):
    cfg = mi.CONFIGS[name]
    idx, w = mi.make_routing(cfg)
    d = moe.make_desc(cfg.T, cfg.D, cfg.F, cfg.E, cfg.K, mi.MODE_BF16)
    scratch = torch.empty(moe.moe_scratch_bytes(d), dtype=torch.uint8, device="cuda")
    tidx = torch.from_numpy(idx).cuda()
    moe.check(moe.moe_route(d, tidx, scratch), "route")
    assert moe.moe_check(d, scratch) == moe.MOE_OK

    L = Layer.__new__(Layer)
    L.cfg, L.desc, L.scratch = cfg, d, scratch
    routing_bitexact(L, idx)


@pytest.mark.timeout(600)
def test_full_size_30b_sampled():
    full_size_vs_oracle("30b", ntok=24, nexp=2)


@pytest.mark.timeout(900)
def test_full_size_235b_sampled():
    full_size_vs_oracle("235b", ntok=12, nexp=1)


@pytest.mark.timeout(600)
def test_full_size_30b_ep_share_sampled():
    # one expert-parallel rank's share: 16 experts with about 8192 rows each
    full_size_vs_oracle("30b_ep_share", ntok=24, nexp=1)


@pytest.mark.parametrize("name", ["one_token", "one_expert", "all_experts"])
def test_degenerate_shapes(name):
    cfg = mi.CONFIGS[name]
    print(f"[case] {name} T={cfg.T} D={cfg.D} F={cfg.F} E={cfg.E} K={cfg.K}", flush=True)
    layer_vs_oracle(cfg, mi.make_inputs(cfg))


def test_all_pairs_on_two_experts():
    # maximal skew: every token picks experts 0 and 1 (in either slot order);
    # the other six get no rows and must get exactly zero weight gradients
    cfg = mi.CONFIGS["mid_bf16"]
    inp = mi.make_inputs(cfg)
    idx = np.zeros_like(inp["topk_idx"])
    idx[:, 1] = 1
    idx[::3] = idx[::3, ::-1]
    print("[case] mid_bf16 with all pairs on experts 0 and 1", flush=True)
    L, out, b = layer_vs_oracle(cfg, dict(inp, topk_idx=idx))
    for e in range(2, cfg.E):
        assert np.all(out["dw1"][e] == 0) and np.all(out["dw2"][e] == 0)


@pytest.mark.parametrize("name", ["mid_bf16", "mid_f32io"])
def test_zero_routing_weights(name):
    # a third of the tokens give their second expert weight 0: those pairs add nothing to y,
    # dx or the weight gradients, yet their routing-weight gradient <dy, o> is not zero (with
    # the weights in the GEMMs, dProb's partials use the unweighted A, never dividing by w)
    cfg = mi.CONFIGS[name]
    inp = mi.make_inputs(cfg)
    w = inp["topk_w"].copy()
    w[::3, 1] = 0.0
    print(f"[case] {name} with zero routing weights", flush=True)
    L, out, b = layer_vs_oracle(cfg, dict(inp, topk_w=w))
    assert np.all(out["dprob"][::3, 1] != 0)


@pytest.mark.parametrize("name", ["small_bf16", "mid_bf16"])
def test_saturated_gates(name):
    # W1 scaled by 200: about one gate value in ten lies beyond +-88, where exp(-g) is 0 or
    # overflows to inf and the logistic function is exactly 1 or 0 in fp32; the SwiGLU and
    # SwiGLU-backward epilogues must give the oracle's values there, without NaN or inf
    cfg = mi.CONFIGS[name]
    inp = mi.make_inputs(cfg)
    w1 = inp["w1"] * np.float32(200.0)
    mi.bf16_round(w1)
    f = orc.forward(inp["x"], inp["topk_idx"], inp["topk_w"], w1, inp["w2"])
    g = f["h"][..., :cfg.F]
    assert (g < -88).mean() > 0.02 and (g > 88).mean() > 0.02
    print(f"[case] {name} with W1 x 200", flush=True)
    L, out, b = layer_vs_oracle(cfg, dict(inp, w1=w1))
    for k, v in out.items():
        assert np.all(np.isfinite(v)), k


@pytest.mark.parametrize("mode", [moe.MOE_FP32, moe.MOE_FP32_BF16GEMM, moe.MOE_BF16,
                                  moe.MOE_FP8_BWD, moe.MOE_MXFP8, moe.MOE_FP8])
def test_empty_layer(mode):
    """No tokens (T = 0): null token buffers are accepted, the routing metadata
    is all zeros even in a scratch full of garbage, and the backward writes zero
    weight gradients (every expert has no tokens, as the oracle's empty sums)."""
    T, D, F, E, K = 0, 256, 256, 4, 2
    d = moe.make_desc(T, D, F, E, K, mode)
    dt = torch.float32 if mode in (moe.MOE_FP32, moe.MOE_FP32_BF16GEMM) else torch.bfloat16
    g = torch.Generator().manual_seed(2200 + mode)
    w1 = (torch.randn(E, 2 * F, D, generator=g) * 0.02).to(dt).cuda()
    w2 = (torch.randn(E, D, F, generator=g) * 0.02).to(dt).cuda()
    nwp = moe.moe_wprep_bytes(d)
    wprep = torch.empty(nwp, dtype=torch.uint8, device="cuda") if nwp else None
    if wprep is not None:
        moe.check(moe.moe_prepare_weights(d, w1, w2, wprep), "moe_prepare_weights")
    scratch = torch.full((moe.moe_scratch_bytes(d),), 0xAB, dtype=torch.uint8, device="cuda")
    dw1 = torch.full_like(w1, float("nan"))
    dw2 = torch.full_like(w2, float("nan"))
    moe.check(moe.moe_fwd(d, None, None, None, w1, w2, wprep, None, scratch), "moe_fwd")
    moe.check(moe.moe_bwd(d, None, None, w1, w2, wprep, None, dw1, dw2, None, scratch), "moe_bwd")
    assert moe.moe_check(d, scratch) == moe.MOE_OK
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(dw1)) == 0 and int(torch.count_nonzero(dw2)) == 0
    rc, counts, offsets, _, _ = moe.moe_routing_view(d, scratch)
    moe.check(rc, "moe_routing_view")
    base = scratch.data_ptr()
    got_c = scratch[counts - base:counts - base + 4 * E].view(torch.int32).cpu().numpy()
    got_o = scratch[offsets - base:offsets - base + 4 * (E + 1)].view(torch.int32).cpu().numpy()
    ref = orc.route(np.zeros((0, K), np.int32), E)
    np.testing.assert_array_equal(got_c, ref["counts"])
    np.testing.assert_array_equal(got_o, ref["offsets"])
