"""Comparisons of the HIP layer (through the C ABI) with the CPU oracle, shared by
the GPU parity tests of every schedule: the default one-kernel-per-step path,
the overlapped forward (MOE_FLAG_OVERLAP) and activation recompute
(MOE_FLAG_RECOMPUTE).  Test infrastructure: only the tests import this module.

Integer routing arrays must be bit-exact; floating-point outputs and
intermediates must meet max|err| / max|ref| <= tol against the float64 oracle
on the same inputs.  Dispatch copies (x_perm, dY_perm) and the permuted
routing weights are bit-exact copies.

In bf16 at the shapes whose GEMMs carry the routing weights (2F % 256 == 0,
D % 64 == 0) the saved A and O rows are w * A and w * O, and the dispatched
upstream gradient is dy itself (w enters in the W2 dgrad); elsewhere A and O
are unweighted and the dispatched gradient is w * dy.
"""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_layer_31_amd as moe
import moe_inputs as mi
from oracle import moe_oracle as orc
from tests.layer_harness import Layer, rel_err, to_host

TOL_BF16 = 1e-2
# fp32 storage and arithmetic against the float64 oracle: rounding of fp32 sums
# over at most a few thousand terms stays orders of magnitude below this
TOL_F32 = 1e-4


def weights_in_gemms(cfg):
    """Whether the library applies the routing weights inside the GEMMs."""
    return cfg.mode == mi.MODE_BF16 and (2 * cfg.F) % 256 == 0 and cfg.D % 64 == 0


def run(cfg, inp, flags=0):
    L = Layer(cfg, inp, flags=flags)
    L.prepare()
    L.fwd()
    L.bwd()
    assert L.check() == moe.MOE_OK
    torch.cuda.synchronize()
    return L


def routing_bitexact(L, idx):
    got = L.routing()
    ref = orc.route(idx, L.cfg.E)
    np.testing.assert_array_equal(got["counts"], ref["counts"])
    np.testing.assert_array_equal(got["offsets"], ref["offsets"])
    np.testing.assert_array_equal(got["pos"], ref["pos"])
    nv = int(ref["offsets"][-1])
    np.testing.assert_array_equal(got["src"][:nv], ref["src"])
    return ref


def layer_vs_oracle(cfg, inp, flags=0):
    """Whole layer, every output and every saved or backward intermediate."""
    L = run(cfg, inp, flags)
    r = routing_bitexact(L, inp["topk_idx"])
    f = orc.forward(inp["x"], inp["topk_idx"], inp["topk_w"], inp["w1"], inp["w2"])
    b = orc.backward(inp["dy"], inp["x"], inp["topk_idx"], inp["topk_w"], inp["w1"], inp["w2"], f)
    out = L.outputs()
    errs = {k: rel_err(out[k], ref) for k, ref in
            (("y", f["y"]), ("dx", b["dx"]), ("dw1", b["dw1"]), ("dw2", b["dw2"]),
             ("dprob", b["dprob"]))}
    tol = TOL_F32 if cfg.mode == mi.MODE_FP32 else TOL_BF16

    # intermediates, row r of a view is pair src[r]; fp32 in the fp32 mode, else bf16
    K, F, D = cfg.K, cfg.F, cfg.D
    act = torch.float32 if cfg.mode == mi.MODE_FP32 else torch.bfloat16
    rnd = (lambda a: a) if cfg.mode == mi.MODE_FP32 else mi.bf16_round
    src = r["src"]
    t_of, k_of = src // K, src % K
    xp = L.view(moe.MOE_VIEW_XPERM, D, act)
    dyp = L.view(moe.MOE_VIEW_DYPERM, D, act)
    wp = L.view(moe.MOE_VIEW_WPERM, 0, torch.float32)
    w = inp["topk_w"][t_of, k_of]
    if weights_in_gemms(cfg):
        # dy itself; the saved A and O carry the weights
        np.testing.assert_array_equal(dyp[:len(src)], rnd(inp["dy"][t_of].copy()))
        a_ref, o_ref = f["a"] * inp["topk_w"][..., None], f["o"] * inp["topk_w"][..., None]
    else:
        # the dispatched gradient is w * dy (fp32 product, stored once)
        dyw = rnd((w[:, None] * inp["dy"][t_of]).astype(np.float32))
        np.testing.assert_array_equal(dyp[:len(src)], dyw)
        a_ref, o_ref = f["a"], f["o"]
    np.testing.assert_array_equal(xp[:len(src)], rnd(inp["x"][t_of].copy()))
    np.testing.assert_array_equal(wp[:len(src)], w)
    views = [(moe.MOE_VIEW_A, F, a_ref, "a"), (moe.MOE_VIEW_O, D, o_ref, "o"),
             (moe.MOE_VIEW_DH, 2 * F, b["dh"], "dh")]
    if not flags & moe.MOE_FLAG_RECOMPUTE:  # the forward keeps no H under recompute
        views.append((moe.MOE_VIEW_H, 2 * F, f["h"], "h"))
    for which, cols, ref, name in views:
        got = L.view(which, cols, act)[:len(src)]
        errs[name] = rel_err(got, ref[t_of, k_of])
    print(cfg.name, f"flags={flags}", {k: round(v, 5) for k, v in errs.items()}, flush=True)
    for k, e in errs.items():
        assert e <= tol, (k, e)
    return L, out, b


def full_size_vs_oracle(name, ntok, nexp, flags=0):
    """A full-size workload on sampled tokens (y, dx, dprob) and sampled rows of
    the weight gradients of sampled experts; routing bit-exact in full."""
    cfg = mi.CONFIGS[name]
    print(f"[case] full-size {name} flags={flags}", flush=True)
    inp = mi.make_inputs(cfg, threads=16)
    L = run(cfg, inp, flags)
    routing_bitexact(L, inp["topk_idx"])
    rng = np.random.default_rng(0)
    tok = np.sort(rng.choice(cfg.T, size=ntok, replace=False))
    tok[0], tok[-1] = 0, cfg.T - 1
    ref = orc.backward_tokens(inp["dy"], inp["x"], inp["topk_idx"], inp["topk_w"], inp["w1"],
                              inp["w2"], tok)
    tt = torch.from_numpy(tok).cuda()
    out = dict(y=L.y[tt], dx=L.dx[tt], dprob=L.dprob[tt])
    errs = {k: rel_err(to_host(v), ref[k]) for k, v in out.items()}
    counts = np.bincount(inp["topk_idx"].ravel(), minlength=cfg.E)
    for e in rng.choice(np.nonzero(counts)[0], size=nexp, replace=False):
        r1 = np.sort(rng.choice(2 * cfg.F, size=6, replace=False))
        r2 = np.sort(rng.choice(cfg.D, size=6, replace=False))
        wr = orc.wgrad_rows(inp["dy"], inp["x"], inp["topk_idx"], inp["topk_w"], inp["w1"],
                            inp["w2"], int(e), r1, r2)
        errs[f"dw1[{e}]"] = rel_err(to_host(L.dw1[int(e)][torch.from_numpy(r1).cuda()]), wr["dw1"])
        errs[f"dw2[{e}]"] = rel_err(to_host(L.dw2[int(e)][torch.from_numpy(r2).cuda()]), wr["dw2"])
    print(name, f"flags={flags}", errs, flush=True)
    for k, e in errs.items():
        assert e <= TOL_BF16, (k, e)
