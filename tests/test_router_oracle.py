"""Pins of the router oracle against facts that do not come from the oracle itself.

A hand-derived example, the renormalised weights as a softmax over the selected
logits alone, finite differences, torch autograd through torch.softmax and
gather, the closed-form gradient w_j (dw_j - <w, dw>), K = E as the textbook
softmax, ties to the lower index, -inf logits, and the selection against an
ordering of the float32 logits themselves.
"""
import math

import numpy as np
import torch

from oracle import router_oracle as ro


def test_hand_example():
    # p is proportional to (1, 2, 3, 0): top-2 is (2, 1) with weights 3/5, 2/5.
    z = np.array([[0.0, math.log(2.0), math.log(3.0), -np.inf]])
    f = ro.router_forward(z, 2)
    assert f["idx"].tolist() == [[2, 1]]
    np.testing.assert_allclose(f["w"], [[3 / 5, 2 / 5]], rtol=1e-15)
    np.testing.assert_allclose(f["P"], [5 / 6], rtol=1e-15)
    # dw = (1, 0): <w, dw> = 3/5, dz_2 = 3/5 * 2/5, dz_1 = 2/5 * (-3/5), the rest 0.
    dz = ro.router_backward(z, 2, np.array([[1.0, 0.0]]), f)
    np.testing.assert_allclose(dz, [[0.0, -6 / 25, 6 / 25, 0.0]], atol=1e-15)


def _logits(seed, T, E, spread=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, E)) * spread).astype(np.float32)


def test_weights_are_softmax_of_selected_logits():
    z = _logits(1, 64, 128).astype(np.float64)
    f = ro.router_forward(z, 8)
    zs = np.take_along_axis(z, f["idx"], axis=1)
    e = np.exp(zs - zs[:, :1])
    np.testing.assert_allclose(f["w"], e / e.sum(axis=1, keepdims=True), rtol=1e-13)
    assert np.all(np.diff(f["w"], axis=1) <= 0)


def test_selection_orders_the_float32_logits():
    z = _logits(2, 256, 128)
    # neighbours one float32 step apart must still be ordered
    z[:, 5] = np.nextafter(z[:, 9], np.float32(np.inf))
    f = ro.router_forward(z, 8)
    expect = np.argsort(-z, axis=1, kind="stable")[:, :8]
    assert np.array_equal(f["idx"], expect)


def test_ties_go_to_the_lower_index():
    z = np.array([[1.0, 3.0, 3.0, 0.0, 3.0], [2.0, 2.0, 2.0, 2.0, 2.0]])
    f = ro.router_forward(z, 2)
    assert f["idx"].tolist() == [[1, 2], [0, 1]]
    np.testing.assert_allclose(f["w"], [[0.5, 0.5], [0.5, 0.5]], rtol=1e-15)


def test_neg_inf_logits():
    z = np.array([[-np.inf, 0.5, -np.inf, -1.0, -np.inf]])
    f = ro.router_forward(z, 4)
    assert f["idx"].tolist() == [[1, 3, 0, 2]]
    w = f["w"][0]
    assert w[2] == 0.0 and w[3] == 0.0
    np.testing.assert_allclose(w[0] + w[1], 1.0, rtol=1e-15)
    np.testing.assert_allclose(w[0] / w[1], math.exp(1.5), rtol=1e-13)
    dz = ro.router_backward(z, 4, np.array([[0.3, -0.2, 5.0, 7.0]]), f)
    assert dz[0, 0] == 0.0 and dz[0, 2] == 0.0 and dz[0, 4] == 0.0


def test_closed_form_gradient_and_zero_sum():
    z = _logits(3, 32, 64)
    dw = np.random.default_rng(4).standard_normal((32, 8))
    f = ro.router_forward(z, 8)
    dz = ro.router_backward(z, 8, dw, f)
    c = (f["w"] * dw).sum(axis=1, keepdims=True)
    expect = np.zeros_like(dz)
    np.put_along_axis(expect, f["idx"], f["w"] * (dw - c), axis=1)
    np.testing.assert_allclose(dz, expect, atol=1e-15)
    np.testing.assert_allclose(dz.sum(axis=1), 0.0, atol=1e-15)


def test_backward_finite_differences():
    rng = np.random.default_rng(5)
    T, E, K = 3, 10, 3
    # well separated logits so a step of h never changes the selection
    z = np.stack([rng.permutation(E) * 0.37 + rng.random(E) * 0.01 for _ in range(T)])
    dw = rng.standard_normal((T, K))

    def loss(zz):
        return float((ro.router_forward(zz, K)["w"] * dw).sum())

    dz = ro.router_backward(z, K, dw)
    h = 1e-6
    num = np.zeros_like(z)
    for t in range(T):
        for j in range(E):
            zp, zm = z.copy(), z.copy()
            zp[t, j] += h
            zm[t, j] -= h
            num[t, j] = (loss(zp) - loss(zm)) / (2 * h)
    np.testing.assert_allclose(dz, num, atol=1e-8)


def test_against_torch_autograd():
    z = _logits(6, 48, 128).astype(np.float64)
    dw = np.random.default_rng(7).standard_normal((48, 8))
    f = ro.router_forward(z, 8)
    zt = torch.tensor(z, requires_grad=True)
    p = torch.softmax(zt, dim=1)
    top = torch.topk(p, 8, dim=1)  # the logits have no ties: torch's order is unique
    assert np.array_equal(top.indices.numpy(), f["idx"])
    ps = p.gather(1, top.indices)
    w = ps / ps.sum(dim=1, keepdim=True)
    (w * torch.tensor(dw)).sum().backward()
    np.testing.assert_allclose(f["w"], w.detach().numpy(), rtol=1e-13)
    np.testing.assert_allclose(ro.router_backward(z, 8, dw, f), zt.grad.numpy(), atol=1e-14)


def test_k_equals_e_is_the_softmax():
    z = _logits(8, 16, 12).astype(np.float64)
    dw = np.random.default_rng(9).standard_normal((16, 12))
    f = ro.router_forward(z, 12)
    zt = torch.tensor(z, requires_grad=True)
    p = torch.softmax(zt, dim=1)
    # weights in expert order are the softmax itself
    w_e = np.zeros_like(z)
    np.put_along_axis(w_e, f["idx"], f["w"], axis=1)
    np.testing.assert_allclose(w_e, p.detach().numpy(), rtol=1e-13)
    dw_e = np.zeros_like(z)
    np.put_along_axis(dw_e, f["idx"], dw, axis=1)
    (p * torch.tensor(dw_e)).sum().backward()
    np.testing.assert_allclose(ro.router_backward(z, 12, dw, f), zt.grad.numpy(), atol=1e-14)


def _brute_topk(row, K):
    """Pure-Python selection: K times take the largest remaining entry, the lowest
    index among equals."""
    left = list(range(len(row)))
    out = []
    for _ in range(K):
        best = left[0]
        for j in left[1:]:
            if row[j] > row[best]:
                best = j
        out.append(best)
        left.remove(best)
    return out


def test_many_ties_against_brute_force():
    rng = np.random.default_rng(10)
    z = rng.integers(0, 4, size=(64, 128)).astype(np.float64)  # four levels: ties everywhere
    f = ro.router_forward(z, 8)
    for t in range(64):
        assert f["idx"][t].tolist() == _brute_topk(z[t].tolist(), 8)


def test_shift_invariance_with_large_logits():
    z = _logits(11, 16, 128).astype(np.float64)
    f0 = ro.router_forward(z, 8)
    f1 = ro.router_forward(z + 1000.0, 8)
    assert np.array_equal(f0["idx"], f1["idx"])
    np.testing.assert_allclose(f1["w"], f0["w"], rtol=1e-10)
    dw = np.random.default_rng(12).standard_normal((16, 8))
    np.testing.assert_allclose(ro.router_backward(z + 1000.0, 8, dw),
                               ro.router_backward(z, 8, dw), atol=1e-12)


def test_workload_routing_is_the_routers_decision():
    # the layer workloads draw their routing decision from the same logits
    import moe_inputs as mi
    for name in ("mid_bf16", "zipf_bf16", "dead_bf16"):
        cfg = mi.CONFIGS[name]
        idx, w = mi.make_routing(cfg)
        f = ro.router_forward(mi.make_router_inputs(cfg)["logits"], cfg.K)
        assert np.array_equal(f["idx"], idx), name
        np.testing.assert_allclose(f["w"], w, atol=1e-6)
