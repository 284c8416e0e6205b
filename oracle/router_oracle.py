"""CPU oracle of the top-k router ahead of the MoE layer.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The product path (the HIP library and its binding) never calls
it, and this module shares no code with that path.

The router is the step just before the layer: every token's expert scores are
turned into a top-k routing decision, which the layer then dispatches on (Prime
Mega MoE news item, "TL;DR": Qwen3 MoE models with 128 experts and top-8
routing; "Why is MoE training communication-bound?": each token goes to a
small subset of experts).  The pages do not spell the router out; this module
takes the plain Qwen3-style reading, in float64:

  forward, per token t with logits z_t [E]:
    p = softmax(z_t)                                   (over all E experts)
    S = the K experts of largest p, in descending order of p, ties to the
        lower expert index
    w_k = p[S_k] / sum_{k'} p[S_k']                    (renormalised top-k)

  backward of a loss L with upstream gradient dw = dL/dw [K]:
    dp_j = (dw_k - sum_k' w_k' dw_k') / P  for j = S_k,  0 for j not in S
           (P = sum_k p[S_k]; the renormalisation's chain rule)
    dz   = p * (dp - <p, dp>)                              (softmax's chain rule)

The selection compares the probabilities of float32 logits in float64, which
orders them exactly as the logits themselves (exp is strictly increasing and
its float64 rounding is far below a float32 step), so the indices are a
function of the logits alone.  -inf logits get probability 0 and, if selected
(fewer than K finite logits), weight 0.

Parity pins (tests marked "not gpu"): the renormalised weights equal a
softmax over the selected logits only; the backward equals finite differences,
torch autograd through torch.softmax/gather, and the closed form
w_j (dw_j - <w, dw>); K = E reduces to the textbook softmax; ties and -inf
logits; the gradient sums to zero per token.
"""
from __future__ import annotations

import numpy as np


def softmax(z: np.ndarray) -> np.ndarray:
    """Row softmax in float64 (max subtracted first)."""
    z = np.asarray(z, np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=-1, keepdims=True)


def select_topk(p: np.ndarray, K: int) -> np.ndarray:
    """Indices [T, K] of the K largest entries of each row, descending, ties to the
    lower index (numpy's stable sort of -p)."""
    return np.argsort(-p, axis=1, kind="stable")[:, :K].astype(np.int32)


def router_forward(logits: np.ndarray, K: int) -> dict:
    """Softmax -> top-K -> renormalise, per token.

    logits: [T, E] (float32 values).  Returns idx int32 [T, K], w float64 [T, K],
    and the intermediates p [T, E] and P [T] (sum of the selected p) that the
    backward reuses.
    """
    z = np.asarray(logits, np.float64)
    p = softmax(z)
    idx = select_topk(p, K)
    ps = np.take_along_axis(p, idx, axis=1)
    P = ps.sum(axis=1)
    w = ps / P[:, None]
    return {"idx": idx, "w": w, "p": p, "P": P}


def router_backward(logits: np.ndarray, K: int, dw: np.ndarray, fwd: dict | None = None) -> np.ndarray:
    """dL/dlogits [T, E] for an upstream gradient dw = dL/dw [T, K], by the chain rule
    through the renormalisation and then the softmax (float64)."""
    if fwd is None:
        fwd = router_forward(logits, K)
    idx, w, p, P = fwd["idx"], fwd["w"], fwd["p"], fwd["P"]
    dw = np.asarray(dw, np.float64)
    T, E = p.shape
    # renormalisation: w_k = p_{S_k} / P
    c = (w * dw).sum(axis=1)
    dp = np.zeros((T, E))
    np.put_along_axis(dp, idx, (dw - c[:, None]) / P[:, None], axis=1)
    # softmax: dz = p * (dp - <p, dp>)
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))
