"""The whole layer under an FP8 recipe, in float64.  TEST INFRASTRUCTURE ONLY.

Only the tests may import this module; the HIP library never calls it and
shares no code with it.

The pages name three FP8 uses of the fused layer: blockwise FP8, MXFP8, and an
fp8_bwd mode with a BF16 forward and an FP8 backward (Prime Mega MoE news item,
"How does the fused kernel work?" and "How do developers use it?").  They do
not say which operands are quantised; the reading taken here is the plainest
one: both operands of every FP8 GEMM, each quantised along its contraction
index, and nothing else.  Concretely, per expert segment of the stable
by-expert order:

  forward (modes fp8 and mxfp8; fp8_bwd keeps it unquantised)
    H  = Q(x_perm) Q(W1[e])^T           x_perm rows along D, W1[e] along D
    A  = silu(H_gate) * H_up
    O  = Q(A) Q(W2[e])^T                A rows along F, W2[e] along F
    y_t = sum_k w O
  backward (every FP8 mode)
    dYw = w dy_t (one row per pair), dprob[t,k] = <dy_t, O>   (unquantised)
    dA  = Q(dYw) Q(W2[e]^T)^T           dYw rows along D, W2[e] along D
    dH  = SwiGLU backward of dA at H
    dX_perm = Q(dH) Q(W1[e]^T)^T        dH rows along 2F, W1[e] along 2F
    dx_t = sum_k dX_perm
    dW2[e] = Qt(dYw)^T Qt(A)            both along the tokens of segment e
    dW1[e] = Qt(dH)^T Qt(x_perm)

Q along a row is `fp8_oracle.quant_rows` (groups of 128 with an fp32 scale, or
MX groups of 32 with an e8m0 scale); Q of a weight is the 128 x 128 block
quantiser (blockwise) or quant_rows along the contraction index (MX); Qt is
`fp8_oracle.quant_tokens` (groups run along the tokens of a segment from its
first token).  Each Q is quantise-then-dequantise, so the GEMMs are plain
float64 products of the dequantised operands.  Between quantisation points
everything stays float64.

With `store_bf16` (the default) every intermediate the layer stores is rounded
once to bfloat16 where it is stored, as in the layer's precision rule (fp32
accumulators rounded once when stored; intermediates and outputs stay bf16):
H, A, O, w dy, dH and dX_perm, and the outputs y and dx.  The quantisers then
see the same bf16 values the layer stores.  The rounding is torch's float to
bfloat16 conversion (nearest, ties to even), used as a library primitive.

`quantiser` may be replaced (the pins use the identity, and one that zeroes a
named operand) so that the data flow can be checked apart from the encodings.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import fp8_oracle as f8
from oracle import moe_oracle as orc

MODES = ("fp8_bwd", "fp8", "mxfp8")

# operand names, in the order the recipe above lists them
OPERANDS = ("fwd_x", "fwd_w1", "fwd_a", "fwd_w2",
            "dgrad_dyw", "dgrad_w2", "dgrad_dh", "dgrad_w1",
            "wgrad_dyw", "wgrad_a", "wgrad_dh", "wgrad_x")


def fp8_quantiser(mx: bool):
    """Q for the recipe: quantise then dequantise `a` with the given kind.

    kind "rows": a [R, C] along C;  "weight": a [out, contraction] along the
    contraction;  "tokens": a [N, C] along N inside the segments `offsets`.
    """
    group = 32 if mx else 128

    def q(name, a, kind, offsets=None):
        if kind == "rows":
            c, s = f8.quant_rows(a, group, mx)
            return f8.dequant_rows(c, s, group, mx)
        if kind == "weight":
            if mx:
                c, s = f8.quant_rows(a, 32, True)
                return f8.dequant_rows(c, s, 32, True)
            c, s = f8.quant_weight_blocks(a)
            return f8.dequant_weight_blocks(c, s)
        # tokens: quantise [C, Npad] in padded segments, then take each segment back
        c, s, poff = f8.quant_tokens(a, offsets, group, mx)
        if mx:
            d = f8.dequant_rows(c, s, 32, True)
        else:
            d = f8.e4m3_decode(c) * np.repeat(np.asarray(s, np.float64).T, 128, axis=1)
        out = np.zeros(np.shape(a))
        for e in range(len(offsets) - 1):
            n = offsets[e + 1] - offsets[e]
            out[offsets[e]:offsets[e + 1]] = d[:, poff[e]:poff[e] + n].T
        return out

    return q


def identity_quantiser(name, a, kind, offsets=None):
    return np.asarray(a, np.float64)


def bf16(a) -> np.ndarray:
    """Nearest bfloat16 value of each element (ties to even), as float64."""
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def layer(mode, x, topk_idx, topk_w, dy, w1, w2, quantiser=None, store_bf16=True,
          experts=None) -> dict:
    """Forward and backward of the layer under `mode`'s FP8 recipe.

    Returns y [T, D], dx [T, D], dw1 [E, 2F, D], dw2 [E, D, F], dprob [T, K],
    and the permuted-order intermediates h, a, o, dh, dxp with the routing
    (offsets, src) they are ordered by.

    `experts` (a list of expert ids) keeps only the rows routed to those experts
    (checks at large sizes): every quantiser here works per row, per weight or
    per expert segment, so those rows are unchanged; y, dx and dprob then hold
    only those experts' contributions, and dw1, dw2 are [len(experts), ...] in
    the order given.
    """
    if mode not in MODES:
        raise ValueError(f"mode must be one of {MODES}")
    q = quantiser if quantiser is not None else fp8_quantiser(mode == "mxfp8")
    fwd_q = mode != "fp8_bwd"
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    T, D = x.shape
    E, F2, _ = w1.shape
    F = F2 // 2
    K = topk_idx.shape[1]
    r = orc.route(topk_idx, E)
    off, src = r["offsets"], r["src"]
    sel = list(range(E)) if experts is None else [int(e) for e in experts]
    if experts is not None:
        keep = np.zeros(E, bool)
        keep[sel] = True
        cnt = np.diff(off)
        src = src[np.repeat(keep, cnt)]
        off = np.concatenate([[0], np.cumsum(np.where(keep, cnt, 0))])
    tok = src // K
    wp = np.asarray(topk_w, np.float64).reshape(-1)[src]      # routing weight of each row
    N = len(src)
    st = bf16 if store_bf16 else (lambda a: a)

    def per_expert(fn, width):
        out = np.zeros((N, width))
        for e in range(E):
            if off[e + 1] > off[e]:
                out[off[e]:off[e + 1]] = fn(e, slice(off[e], off[e + 1]))
        return out

    W1 = {e: np.asarray(w1[e], np.float64) for e in sel}
    W2 = {e: np.asarray(w2[e], np.float64) for e in sel}
    # forward
    xp = x[tok]
    xq = q("fwd_x", xp, "rows") if fwd_q else xp
    H = per_expert(lambda e, s: xq[s] @ (q("fwd_w1", W1[e], "weight") if fwd_q else W1[e]).T, F2)
    A = st(orc.silu(H[:, :F]) * H[:, F:])  # from the unrounded gate and up
    H = st(H)
    g, u = H[:, :F], H[:, F:]
    Aq = q("fwd_a", A, "rows") if fwd_q else A
    O = st(per_expert(lambda e, s: Aq[s] @ (q("fwd_w2", W2[e], "weight") if fwd_q else W2[e]).T, D))
    y = np.zeros((T, D))
    np.add.at(y, tok, wp[:, None] * O)
    y = st(y)
    # backward
    dprob = np.zeros(T * K)
    dprob[src] = np.einsum("nd,nd->n", dy[tok], O)
    dYw = st(wp[:, None] * dy[tok])
    dYq = q("dgrad_dyw", dYw, "rows")
    dA = per_expert(lambda e, s: dYq[s] @ q("dgrad_w2", W2[e].T, "weight").T, F)
    sg = orc.sigmoid(g)
    dH = st(np.concatenate([dA * u * sg * (1.0 + g * (1.0 - sg)), dA * g * sg], axis=1))
    dHq = q("dgrad_dh", dH, "rows")
    dXp = st(per_expert(lambda e, s: dHq[s] @ q("dgrad_w1", W1[e].T, "weight").T, D))
    dx = np.zeros((T, D))
    np.add.at(dx, tok, dXp)
    dx = st(dx)
    dYt = q("wgrad_dyw", dYw, "tokens", off)
    At = q("wgrad_a", A, "tokens", off)
    dHt = q("wgrad_dh", dH, "tokens", off)
    xt = q("wgrad_x", xp, "tokens", off)
    dw1 = np.zeros((len(sel), F2, D))
    dw2 = np.zeros((len(sel), D, F))
    for i, e in enumerate(sel):
        s = slice(off[e], off[e + 1])
        dw2[i] = dYt[s].T @ At[s]
        dw1[i] = dHt[s].T @ xt[s]
    return dict(y=y, dx=dx, dw1=dw1, dw2=dw2, dprob=dprob.reshape(T, K),
                h=H, a=A, o=O, dh=dH, dxp=dXp, offsets=off, src=src)
