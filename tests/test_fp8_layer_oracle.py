"""Pins of the FP8-recipe layer oracle (oracle/fp8_layer_oracle.py), CPU only.

* With the identity as the quantiser it is the plain layer: it must equal the
  per-token float64 oracle (itself pinned by closed forms, autograd and finite
  differences), which checks the permutation, gathers, sums and SwiGLU
  backward of the segment formulation.
* Data flow: zeroing one named operand may change exactly the outputs that
  operand feeds (and in fp8_bwd the forward operands are never quantised).
* Orientation: every quantised operand reaches the quantiser as
  [rows, contraction] with the contraction of its GEMM last.
* bf16 storage: rounding the stored intermediates moves the outputs a little,
  but not by much.
* Expert subsets: restricted to some experts, their rows and weight gradients
  are bit-identical to the full run's.
* Format bound: a product of two e4m3-quantised operands differs from the exact
  product by at most sum |a||eb| + |ea||b| + |ea||eb|, where an element's
  encoding error is at most 2^-4 of it (3 mantissa bits) plus half a subnormal
  step (2^-10 of the group's scale unit, at most 2^-9 amax / 448).
"""
import numpy as np
import pytest

import moe_inputs as mi
from oracle import fp8_layer_oracle as fl
from oracle import moe_oracle as orc

CFG = mi.LayerConfig("fp8_recipe_pin", T=96, D=256, F=128, E=4, K=2, seed=4101)
OUTS = ("y", "dx", "dw1", "dw2", "dprob")


@pytest.fixture(scope="module")
def inp():
    return mi.make_inputs(CFG)


def _run(inp, mode, q=None, store_bf16=False):
    return fl.layer(mode, inp["x"], inp["topk_idx"], inp["topk_w"], inp["dy"], inp["w1"],
                    inp["w2"], quantiser=q, store_bf16=store_bf16)


def test_identity_quantiser_is_the_plain_layer(inp):
    f = orc.forward(inp["x"], inp["topk_idx"], inp["topk_w"], inp["w1"], inp["w2"])
    b = orc.backward(inp["dy"], inp["x"], inp["topk_idx"], inp["topk_w"], inp["w1"], inp["w2"], f)
    ref = dict(y=f["y"], dx=b["dx"], dw1=b["dw1"], dw2=b["dw2"], dprob=b["dprob"])
    for mode in fl.MODES:
        r = _run(inp, mode, fl.identity_quantiser)
        for k in OUTS:
            np.testing.assert_allclose(r[k], ref[k], rtol=0, atol=1e-10 * np.abs(ref[k]).max(),
                                       err_msg=f"{mode} {k}")


# outputs a zeroed operand must change (all others must stay bit-identical)
FEEDS = {
    "fwd_x": OUTS, "fwd_w1": OUTS,
    "fwd_a": ("y", "dprob"), "fwd_w2": ("y", "dprob"),
    "dgrad_dyw": ("dx", "dw1"), "dgrad_w2": ("dx", "dw1"),
    "dgrad_dh": ("dx",), "dgrad_w1": ("dx",),
    "wgrad_dyw": ("dw2",), "wgrad_a": ("dw2",),
    "wgrad_dh": ("dw1",), "wgrad_x": ("dw1",),
}


@pytest.mark.parametrize("mode", fl.MODES)
def test_each_operand_feeds_its_outputs(inp, mode):
    base = _run(inp, mode, fl.identity_quantiser)
    assert set(FEEDS) == set(fl.OPERANDS)
    for name, feeds in FEEDS.items():
        def zero_one(n, a, kind, offsets=None, name=name):
            a = np.asarray(a, np.float64)
            return a * 0.0 if n == name else a
        r = _run(inp, mode, zero_one)
        quantised = mode != "fp8_bwd" or not name.startswith("fwd_")
        for k in OUTS:
            same = np.array_equal(r[k], base[k])
            if quantised and k in feeds:
                assert not same, (mode, name, k)
            else:
                assert same, (mode, name, k)


def test_operands_reach_the_quantiser_contraction_last(inp):
    D, F, N = CFG.D, CFG.F, CFG.T * CFG.K
    want = {"fwd_x": ("rows", (N, D)), "fwd_w1": ("weight", (2 * F, D)),
            "fwd_a": ("rows", (N, F)), "fwd_w2": ("weight", (D, F)),
            "dgrad_dyw": ("rows", (N, D)), "dgrad_w2": ("weight", (F, D)),
            "dgrad_dh": ("rows", (N, 2 * F)), "dgrad_w1": ("weight", (D, 2 * F)),
            "wgrad_dyw": ("tokens", (N, D)), "wgrad_a": ("tokens", (N, F)),
            "wgrad_dh": ("tokens", (N, 2 * F)), "wgrad_x": ("tokens", (N, D))}
    seen = {}

    def spy(n, a, kind, offsets=None):
        a = np.asarray(a, np.float64)
        if kind == "weight":
            seen.setdefault(n, (kind, a.shape))
        else:
            seen[n] = (kind, a.shape)
            assert (offsets is not None) == (kind == "tokens"), n
        return a

    _run(inp, "fp8", spy)
    assert seen == want


def _product_bound(a, b, amax_a, amax_b):
    """Bound on |Q(a) Q(b) - a b| for a [M, C] times b [C, N] (see module doc)."""
    u = 2.0 ** -4
    ea = u * np.abs(a) + 2.0 ** -9 * amax_a / 448
    eb = u * np.abs(b) + 2.0 ** -9 * amax_b / 448
    return ea @ np.abs(b) + np.abs(a) @ eb + ea @ eb


@pytest.mark.parametrize("mode", ["fp8", "mxfp8"])
def test_quantised_products_within_the_e4m3_bound(inp, mode):
    r = _run(inp, mode)
    off, src = r["offsets"], r["src"]
    xp = np.asarray(inp["x"], np.float64)[src // CFG.K]
    for e in range(CFG.E):
        s = slice(off[e], off[e + 1])
        if off[e + 1] == off[e]:
            continue
        W1 = np.asarray(inp["w1"][e], np.float64)
        # forward W1: rows of x_perm times W1[e]^T
        exact = xp[s] @ W1.T
        err = np.abs(r["h"][s] - exact)
        bnd = _product_bound(xp[s], W1.T, np.abs(xp).max(), np.abs(W1).max())
        assert np.all(err <= bnd * (1 + 1e-6) + 1e-12), (mode, e, "h")
        assert err.max() > 0  # it was quantised
        # W1 dgrad: the recipe's dH rows times W1[e]
        dh = r["dh"][s]
        err = np.abs(r["dxp"][s] - dh @ W1)
        bnd = _product_bound(dh, W1, np.abs(r["dh"]).max(), np.abs(W1).max())
        assert np.all(err <= bnd * (1 + 1e-6) + 1e-12), (mode, e, "dxp")
        # W1 wgrad: over the segment's tokens, dH^T x_perm
        err = np.abs(r["dw1"][e] - dh.T @ xp[s])
        bnd = _product_bound(dh.T, xp[s], np.abs(r["dh"]).max(), np.abs(xp).max())
        assert np.all(err <= bnd * (1 + 1e-6) + 1e-12), (mode, e, "dw1")


@pytest.mark.parametrize("mode", fl.MODES)
def test_recipe_stays_near_the_unquantised_layer(inp, mode):
    """e4m3 keeps about 2^-4 relative error per operand: the recipe's outputs stay
    within a few percent of the plain layer, and fp8_bwd's forward is exact."""
    plain = _run(inp, mode, fl.identity_quantiser)
    r = _run(inp, mode)
    rb = _run(inp, mode, store_bf16=True)  # e4m3 codes of bf16-rounded values flip now and then
    for k in OUTS:
        rel = np.abs(rb[k] - r[k]).max() / np.abs(r[k]).max()
        assert 0 < rel < 0.1, (mode, k, rel)
    for k in OUTS:
        rel = np.abs(r[k] - plain[k]).max() / np.abs(plain[k]).max()
        if mode == "fp8_bwd" and k in ("y", "dprob"):
            assert rel == 0.0, (mode, k)
        else:
            assert 1e-4 < rel < 0.2, (mode, k, rel)


def test_expert_subset_keeps_those_rows_unchanged(inp):
    full = _run(inp, "mxfp8", store_bf16=True)
    sub = fl.layer("mxfp8", inp["x"], inp["topk_idx"], inp["topk_w"], inp["dy"], inp["w1"],
                   inp["w2"], experts=[2, 0])
    off = full["offsets"]
    rows = np.r_[off[0]:off[1], off[2]:off[3]]
    for k in ("h", "a", "o", "dh", "dxp"):
        np.testing.assert_array_equal(sub[k], full[k][rows], err_msg=k)
    np.testing.assert_array_equal(sub["dw1"], full["dw1"][[2, 0]])
    np.testing.assert_array_equal(sub["dw2"], full["dw2"][[2, 0]])


def test_bf16_storage_points_are_the_stored_intermediates(inp, monkeypatch):
    """The recipe rounds to bf16 exactly where the layer stores (A, H, O, y, w dy,
    dH, dX_perm, dx, in that order), and every later step consumes the rounded
    value: each rounding's argument is recomputed here, in float64 from the
    previous rounded values, by the layer's definition, and must equal what the
    oracle rounded.  A dropped, added or moved storage point changes the count,
    the order or one of the arguments."""
    seen = []
    round_bf16 = fl.bf16

    def spy(a):
        seen.append(np.array(a, np.float64, copy=True))
        return round_bf16(a)

    monkeypatch.setattr(fl, "bf16", spy)
    r = _run(inp, "fp8", fl.identity_quantiser, store_bf16=True)
    monkeypatch.undo()
    T, D, F, K = CFG.T, CFG.D, CFG.F, CFG.K
    off, src = r["offsets"], r["src"]
    N = len(src)
    assert [a.shape for a in seen] == [(N, F), (N, 2 * F), (N, D), (T, D), (N, D), (N, 2 * F),
                                        (N, D), (T, D)]
    pre = dict(zip(("a", "h", "o", "y", "dyw", "dh", "dxp", "dx"), seen))
    st = {k: fl.bf16(v) for k, v in pre.items()}
    for k in ("a", "h", "o", "y", "dh", "dxp", "dx"):  # the returned values are the rounded ones
        np.testing.assert_array_equal(r[k], st[k], err_msg=k)
    tok = src // K
    wp = np.asarray(inp["topk_w"], np.float64).reshape(-1)[src]
    x = np.asarray(inp["x"], np.float64)
    dy = np.asarray(inp["dy"], np.float64)
    h_raw = np.zeros((N, 2 * F))
    o_raw = np.zeros((N, D))
    dA = np.zeros((N, F))
    dxp_raw = np.zeros((N, D))
    for e in range(CFG.E):
        s = slice(off[e], off[e + 1])
        W1 = np.asarray(inp["w1"][e], np.float64)
        W2 = np.asarray(inp["w2"][e], np.float64)
        h_raw[s] = x[tok[s]] @ W1.T
        o_raw[s] = st["a"][s] @ W2.T            # O from the stored A
        dA[s] = st["dyw"][s] @ W2                # dgrad from the stored w dy
        dxp_raw[s] = st["dh"][s] @ W1            # dgrad from the stored dH
    g, u = h_raw[:, :F], h_raw[:, F:]
    a_raw = g / (1 + np.exp(-g)) * u             # A from the unrounded H
    y_raw = np.zeros((T, D))
    np.add.at(y_raw, tok, wp[:, None] * st["o"])  # y from the stored O
    dyw_raw = wp[:, None] * dy[tok]
    gs, us = st["h"][:, :F], st["h"][:, F:]      # SwiGLU backward at the stored H
    sg = 1 / (1 + np.exp(-gs))
    dh_raw = np.concatenate([dA * us * sg * (1 + gs * (1 - sg)), dA * gs * sg], axis=1)
    dx_raw = np.zeros((T, D))
    np.add.at(dx_raw, tok, st["dxp"])            # dx from the stored dX_perm
    for k, want in (("a", a_raw), ("h", h_raw), ("o", o_raw), ("y", y_raw), ("dyw", dyw_raw),
                    ("dh", dh_raw), ("dxp", dxp_raw), ("dx", dx_raw)):
        np.testing.assert_allclose(pre[k], want, rtol=0, atol=1e-12 * np.abs(want).max(),
                                   err_msg=k)
    # the weight gradients contract the stored w dy, A, dH and the inputs
    for e in range(CFG.E):
        s = slice(off[e], off[e + 1])
        np.testing.assert_allclose(r["dw2"][e], st["dyw"][s].T @ st["a"][s], rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["dw1"][e], st["dh"][s].T @ x[tok[s]], rtol=0, atol=1e-12)
