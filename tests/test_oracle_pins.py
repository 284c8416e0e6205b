"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Closed-form hand-derived example, a special case that reduces to library
routines (torch.nn.functional), finite differences, torch autograd on a dense
all-experts formulation, invariants (token permutation, slot order, zero-token
experts, linearity in the routing weights) and the routing arrays against
numpy's stable argsort.
"""
import json
import os
import re

import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_layer(seed, T, D, F, E, K, dead=()):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, D))
    w1 = rng.standard_normal((E, 2 * F, D)) * 0.3
    w2 = rng.standard_normal((E, D, F)) * 0.3
    dy = rng.standard_normal((T, D))
    live = np.array([e for e in range(E) if e not in dead])
    idx = np.stack([rng.choice(live, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, K)) + 0.1
    w = w / w.sum(axis=1, keepdims=True)
    return x, w1, w2, dy, idx, w


def _eval_expr(s, L3):
    if isinstance(s, (int, float)):
        return float(s)
    assert re.fullmatch(r"[0-9L3+\-*/(). ]+", s), s
    return float(eval(s, {"__builtins__": {}}, {"L3": L3}))


def _tree(v, L3):
    if isinstance(v, list):
        return [_tree(u, L3) for u in v]
    return _eval_expr(v, L3)


def test_closed_form_two_experts():
    line = [l for l in open(os.path.join(GOLDEN, "closed_form_two_experts.txt")) if l.startswith("{")][0]
    g = json.loads(line)
    L3 = float(np.log(3.0))
    x = np.array(g["x"], float)
    idx = np.array(g["idx"], np.int32)
    w = np.array(g["w"], float)
    dy = np.array(g["dy"], float)
    w1 = np.array(_tree(g["w1"], L3))
    w2 = np.array(_tree(g["w2"], L3), float)
    f = orc.forward(x, idx, w, w1, w2)
    b = orc.backward(dy, x, idx, w, w1, w2, f)
    np.testing.assert_allclose(f["y"], _tree(g["y"], L3), rtol=1e-13, atol=1e-14)
    for key in ("dprob", "dx", "dw1", "dw2"):
        np.testing.assert_allclose(b[key], np.array(_tree(g[key], L3)), rtol=1e-13, atol=1e-14,
                                   err_msg=key)


def test_single_expert_is_dense_swiglu_ffn():
    """E=1, top-1, weight 1: the layer is a dense SwiGLU FFN (torch.nn.functional)."""
    x, w1, w2, dy, _, _ = _rand_layer(1, T=7, D=12, F=5, E=1, K=1)
    idx = np.zeros((7, 1), np.int32)
    w = np.ones((7, 1))
    y = orc.forward(x, idx, w, w1, w2)["y"]
    tx = torch.tensor(x, dtype=torch.float64)
    g = torch.nn.functional.linear(tx, torch.tensor(w1[0, :5]))
    u = torch.nn.functional.linear(tx, torch.tensor(w1[0, 5:]))
    ref = torch.nn.functional.linear(torch.nn.functional.silu(g) * u, torch.tensor(w2[0]))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_silu_against_torch():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(orc.silu(z), torch.nn.functional.silu(torch.tensor(z)).numpy(),
                               rtol=1e-13, atol=1e-300)


def _dense_autograd(x, idx, w, w1, w2, dy):
    """Brute force: every expert on every token, masked by the routing weights."""
    T, K = idx.shape
    E, F2, D = w1.shape
    F = F2 // 2
    tx = torch.tensor(x, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    t1 = torch.tensor(w1, requires_grad=True)
    t2 = torch.tensor(w2, requires_grad=True)
    onehot = torch.nn.functional.one_hot(torch.tensor(idx, dtype=torch.long), E).double()
    c = (onehot * tw[:, :, None]).sum(dim=1)  # [T, E]
    y = torch.zeros(T, D, dtype=torch.float64)
    for e in range(E):
        h = tx @ t1[e].T
        a = torch.nn.functional.silu(h[:, :F]) * h[:, F:]
        y = y + c[:, e:e + 1] * (a @ t2[e].T)
    (y * torch.tensor(dy)).sum().backward()
    return y.detach().numpy(), tx.grad.numpy(), t1.grad.numpy(), t2.grad.numpy(), tw.grad.numpy()


def test_against_dense_autograd():
    x, w1, w2, dy, idx, w = _rand_layer(2, T=9, D=8, F=6, E=5, K=3)
    f = orc.forward(x, idx, w, w1, w2)
    b = orc.backward(dy, x, idx, w, w1, w2, f)
    y, dx, dw1, dw2, dw = _dense_autograd(x, idx, w, w1, w2, dy)
    np.testing.assert_allclose(f["y"], y, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(b["dx"], dx, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(b["dw1"], dw1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(b["dw2"], dw2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(b["dprob"], dw, rtol=1e-11, atol=1e-12)


def test_finite_differences():
    x, w1, w2, dy, idx, w = _rand_layer(3, T=5, D=6, F=4, E=4, K=2)
    b = orc.backward(dy, x, idx, w, w1, w2)

    def loss(x_, w1_, w2_, w_):
        return float((orc.forward(x_, idx, w_, w1_, w2_)["y"] * dy).sum())

    rng = np.random.default_rng(7)
    h = 1e-5
    for name, grad in (("x", b["dx"]), ("w1", b["dw1"]), ("w2", b["dw2"]), ("w", b["dprob"])):
        args = dict(x=x, w1=w1, w2=w2, w=w)
        base = args[name]
        for _ in range(6):
            i = tuple(int(rng.integers(s)) for s in base.shape)
            p = base.copy(); p[i] += h
            m = base.copy(); m[i] -= h
            ap = dict(args); ap[name] = p
            am = dict(args); am[name] = m
            fd = (loss(ap["x"], ap["w1"], ap["w2"], ap["w"]) -
                  loss(am["x"], am["w1"], am["w2"], am["w"])) / (2 * h)
            assert abs(fd - grad[i]) <= 1e-6 * max(1.0, abs(fd)), (name, i, fd, grad[i])


def test_token_permutation_invariance():
    x, w1, w2, dy, idx, w = _rand_layer(4, T=11, D=8, F=4, E=6, K=2)
    pi = np.random.default_rng(5).permutation(11)
    f = orc.forward(x, idx, w, w1, w2)
    b = orc.backward(dy, x, idx, w, w1, w2, f)
    fp = orc.forward(x[pi], idx[pi], w[pi], w1, w2)
    bp = orc.backward(dy[pi], x[pi], idx[pi], w[pi], w1, w2, fp)
    np.testing.assert_allclose(fp["y"], f["y"][pi], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(bp["dx"], b["dx"][pi], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(bp["dprob"], b["dprob"][pi], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(bp["dw1"], b["dw1"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(bp["dw2"], b["dw2"], rtol=1e-10, atol=1e-12)


def test_slot_order_invariance():
    x, w1, w2, dy, idx, w = _rand_layer(6, T=7, D=6, F=4, E=5, K=3)
    sigma = np.array([2, 0, 1])
    f = orc.forward(x, idx, w, w1, w2)
    b = orc.backward(dy, x, idx, w, w1, w2, f)
    fs = orc.forward(x, idx[:, sigma], w[:, sigma], w1, w2)
    bs = orc.backward(dy, x, idx[:, sigma], w[:, sigma], w1, w2, fs)
    np.testing.assert_allclose(fs["y"], f["y"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(bs["dx"], b["dx"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(bs["dw1"], b["dw1"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(bs["dw2"], b["dw2"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(bs["dprob"], b["dprob"][:, sigma], rtol=1e-12, atol=1e-14)


def test_zero_token_expert_has_zero_wgrad():
    x, w1, w2, dy, idx, w = _rand_layer(8, T=10, D=6, F=4, E=5, K=2, dead=(1, 3))
    b = orc.backward(dy, x, idx, w, w1, w2)
    for e in (1, 3):
        assert np.all(b["dw1"][e] == 0.0) and np.all(b["dw2"][e] == 0.0)
    for e in (0, 2, 4):
        assert np.any(b["dw1"][e] != 0.0)
    r = orc.route(idx, 5)
    assert r["counts"][1] == 0 and r["counts"][3] == 0
    assert r["counts"].sum() == idx.size and r["offsets"][-1] == idx.size


def test_no_tokens_gives_zero_weight_gradients():
    # T = 0: every expert receives no tokens, so each weight gradient is an empty
    # sum (zero), the routing has zero counts and the token outputs are empty
    _, w1, w2, _, _, _ = _rand_layer(9, T=3, D=6, F=4, E=5, K=2)
    x, dy = np.zeros((0, 6)), np.zeros((0, 6))
    idx, w = np.zeros((0, 2), np.int32), np.zeros((0, 2))
    f = orc.forward(x, idx, w, w1, w2)
    b = orc.backward(dy, x, idx, w, w1, w2, f)
    assert f["y"].shape == (0, 6) and b["dx"].shape == (0, 6) and b["dprob"].shape == (0, 2)
    assert b["dw1"].shape == w1.shape and not np.any(b["dw1"])
    assert b["dw2"].shape == w2.shape and not np.any(b["dw2"])
    r = orc.route(idx, 5)
    assert not np.any(r["counts"]) and not np.any(r["offsets"]) and r["pos"].size == 0


def test_linear_in_routing_weights():
    x, w1, w2, dy, idx, w = _rand_layer(9, T=6, D=5, F=3, E=4, K=2)
    y1 = orc.forward(x, idx, w, w1, w2)["y"]
    y3 = orc.forward(x, idx, 2.5 * w, w1, w2)["y"]
    np.testing.assert_allclose(y3, 2.5 * y1, rtol=1e-13, atol=1e-14)


def test_route_against_stable_argsort():
    rng = np.random.default_rng(10)
    for E, T, K in ((8, 64, 2), (128, 333, 8), (5, 17, 3)):
        idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
        r = orc.route(idx, E)
        flat = idx.reshape(-1)
        src = np.argsort(flat, kind="stable")
        np.testing.assert_array_equal(r["src"], src)
        pos = np.empty_like(src)
        pos[src] = np.arange(src.size)
        np.testing.assert_array_equal(r["pos"], pos)
        np.testing.assert_array_equal(r["counts"], np.bincount(flat, minlength=E))
        np.testing.assert_array_equal(r["offsets"][1:], np.cumsum(np.bincount(flat, minlength=E)))
        assert r["offsets"][0] == 0


def test_route_skips_out_of_range_ids():
    idx = np.array([[0, 3], [5, 1], [-1, 2]], np.int32)
    r = orc.route(idx, 4)
    assert r["invalid"] == 2
    assert r["pos"][2] == -1 and r["pos"][4] == -1
    np.testing.assert_array_equal(r["counts"], [1, 1, 1, 1])
    np.testing.assert_array_equal(r["src"], [0, 3, 5, 1])


def test_sampled_helpers_match_full_backward():
    x, w1, w2, dy, idx, w = _rand_layer(11, T=13, D=8, F=6, E=4, K=2)
    b = orc.backward(dy, x, idx, w, w1, w2)
    f = orc.forward(x, idx, w, w1, w2)
    tok = np.array([3, 0, 12, 7])
    bt = orc.backward_tokens(dy, x, idx, w, w1, w2, tok)
    np.testing.assert_allclose(bt["y"], f["y"][tok], rtol=1e-13)
    np.testing.assert_allclose(bt["dx"], b["dx"][tok], rtol=1e-13)
    np.testing.assert_allclose(bt["dprob"], b["dprob"][tok], rtol=1e-13)
    for e in range(4):
        r1, r2 = np.array([0, 5, 11]), np.array([1, 7])
        wr = orc.wgrad_rows(dy, x, idx, w, w1, w2, e, r1, r2)
        np.testing.assert_allclose(wr["dw1"], b["dw1"][e][r1], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(wr["dw2"], b["dw2"][e][r2], rtol=1e-11, atol=1e-13)
