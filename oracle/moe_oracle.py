"""CPU oracle of one GPU's trainable MoE layer.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The product path (the HIP library and its binding) never calls
it, and this module shares no code with that path.

Everything here is plain numpy in float64, written from the definition of the
layer on the pages (Prime Mega MoE news item, section "How does the fused kernel
work?": expert-parallel dispatch, the two expert linear layers, SwiGLU and the
combine, plus the backward pass Prime Intellect added).  The layer itself is
the textbook top-k mixture-of-experts FFN:

  forward, per token t and slot k (expert e = idx[t,k], weight w = w[t,k]):
    h = W1[e] x_t                       (W1[e] is [2F, D]; rows 0..F-1 gate, F..2F-1 up)
    a = silu(h[:F]) * h[F:]             (SwiGLU, silu(z) = z * sigmoid(z))
    o = W2[e] a                         (W2[e] is [D, F])
    y_t = sum_k w * o

  backward of L = sum_t <dy_t, y_t> (analytic):
    dprob[t,k] = <dy_t, o>
    da = w * W2[e]^T dy_t
    dg = da * u * s * (1 + g (1 - s)),  du = da * silu(g),  s = sigmoid(g)
    dx_t += W1[e]^T [dg; du]
    dW2[e] += (w dy_t) a^T,   dW1[e] += [dg; du] x_t^T

The routing metadata is a stable counting sort of the flat pair index
p = t*K + k by expert (the "sort tokens" step the pages describe in "Why is MoE
training communication-bound?").  Readings where the pages are silent:
gate/up stacked in that order inside W1; SwiGLU without bias or clamp; the
order inside an expert segment is ascending p; out-of-range expert ids are
skipped.  The matrix-vector products use numpy's `@` as a library primitive;
there is no blocking or fusion beyond the definition.

Parity pins (tests marked "not gpu"): closed-form hand-derived example, the
E=1/K=1/w=1 dense SwiGLU FFN against torch.nn.functional, finite differences,
torch autograd on a dense all-experts formulation, permutation and slot-order
invariance, zero-token experts, linearity in the routing weights, and the
routing arrays against numpy's stable argsort.
"""
from __future__ import annotations

import numpy as np


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    return z * sigmoid(z)


def route(topk_idx: np.ndarray, E: int) -> dict:
    """Stable counting sort of the routed pairs by expert.

    counts[e]  = number of pairs p with idx_p == e
    offsets    = exclusive prefix sum of counts, offsets[E] = number of valid pairs
    pos[p]     = offsets[e] + #{p' < p : idx_p' == e}   (-1 for an out-of-range id)
    src[pos[p]] = p
    Returns int64 arrays and the number of invalid ids.
    """
    idx = np.asarray(topk_idx).reshape(-1)
    N = idx.size
    counts = np.zeros(E, np.int64)
    invalid = 0
    for p in range(N):
        e = int(idx[p])
        if 0 <= e < E:
            counts[e] += 1
        else:
            invalid += 1
    offsets = np.zeros(E + 1, np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    nxt = offsets[:E].copy()
    pos = np.full(N, -1, np.int64)
    src = np.full(int(offsets[E]), -1, np.int64)
    for p in range(N):
        e = int(idx[p])
        if 0 <= e < E:
            pos[p] = nxt[e]
            src[nxt[e]] = p
            nxt[e] += 1
    return dict(counts=counts, offsets=offsets, pos=pos, src=src, invalid=invalid)


class _Weights:
    """Lazily converts one expert's weights to float64 (keeps a small cache)."""

    def __init__(self, w1, w2, cache: int = 16):
        self.w1, self.w2 = w1, w2
        self.cache = {}
        self.order = []
        self.limit = cache

    def get(self, e: int):
        if e not in self.cache:
            if len(self.order) >= self.limit:
                del self.cache[self.order.pop(0)]
            self.cache[e] = (np.asarray(self.w1[e], np.float64),
                             np.asarray(self.w2[e], np.float64))
            self.order.append(e)
        return self.cache[e]


def _pair_forward(W1e, W2e, xt, F):
    h = W1e @ xt
    g, u = h[:F], h[F:]
    a = silu(g) * u
    o = W2e @ a
    return h, a, o


def forward(x, topk_idx, topk_w, w1, w2, tokens=None) -> dict:
    """Per-token forward loop.  Returns y [T or len(tokens), D] and per-pair h, a, o.

    `tokens` restricts the loop to a subset of tokens (sampled checks at large
    sizes); rows of the result follow the order of `tokens`.
    """
    x = np.asarray(x)
    T, D = x.shape
    E, F2, _ = w1.shape
    F = F2 // 2
    K = topk_idx.shape[1]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    W = _Weights(w1, w2, cache=E if tokens is None else 16)
    y = np.zeros((len(tok), D))
    h = np.zeros((len(tok), K, 2 * F))
    a = np.zeros((len(tok), K, F))
    o = np.zeros((len(tok), K, D))
    for i, t in enumerate(tok):
        xt = x[t].astype(np.float64)
        for k in range(K):
            e = int(topk_idx[t, k])
            if not 0 <= e < E:
                continue
            W1e, W2e = W.get(e)
            h[i, k], a[i, k], o[i, k] = _pair_forward(W1e, W2e, xt, F)
            y[i] += float(topk_w[t, k]) * o[i, k]
    return dict(y=y, h=h, a=a, o=o)


def _pair_backward(W1e, W2e, dyt, h, w, F):
    g, u = h[:F], h[F:]
    s = sigmoid(g)
    da = w * (W2e.T @ dyt)
    dg = da * u * s * (1.0 + g * (1.0 - s))
    du = da * (g * s)
    dh = np.concatenate([dg, du])
    return dh, W1e.T @ dh


def backward(dy, x, topk_idx, topk_w, w1, w2, fwd=None) -> dict:
    """Analytic backward of L = sum_t <dy_t, y_t> over all tokens.

    Returns dx [T,D], dw1 [E,2F,D], dw2 [E,D,F], dprob [T,K] and per-pair dh.
    dW accumulates pairs in ascending t, then k (ascending p).
    """
    x = np.asarray(x)
    dy = np.asarray(dy)
    T, D = x.shape
    E, F2, _ = w1.shape
    F = F2 // 2
    K = topk_idx.shape[1]
    if fwd is None:
        fwd = forward(x, topk_idx, topk_w, w1, w2)
    W = _Weights(w1, w2, cache=E)
    dx = np.zeros((T, D))
    dw1 = np.zeros((E, 2 * F, D))
    dw2 = np.zeros((E, D, F))
    dprob = np.zeros((T, K))
    dh = np.zeros((T, K, 2 * F))
    for t in range(T):
        xt = x[t].astype(np.float64)
        dyt = dy[t].astype(np.float64)
        for k in range(K):
            e = int(topk_idx[t, k])
            if not 0 <= e < E:
                continue
            w = float(topk_w[t, k])
            W1e, W2e = W.get(e)
            dprob[t, k] = dyt @ fwd["o"][t, k]
            dh[t, k], dxc = _pair_backward(W1e, W2e, dyt, fwd["h"][t, k], w, F)
            dx[t] += dxc
            dw2[e] += np.outer(w * dyt, fwd["a"][t, k])
            dw1[e] += np.outer(dh[t, k], xt)
    return dict(dx=dx, dw1=dw1, dw2=dw2, dprob=dprob, dh=dh)


def backward_tokens(dy, x, topk_idx, topk_w, w1, w2, tokens) -> dict:
    """dx rows, dprob rows and per-pair dh of the selected tokens only."""
    x = np.asarray(x)
    D = x.shape[1]
    E, F2, _ = w1.shape
    F = F2 // 2
    K = topk_idx.shape[1]
    tok = np.asarray(tokens)
    fwd = forward(x, topk_idx, topk_w, w1, w2, tokens=tok)
    W = _Weights(w1, w2)
    dx = np.zeros((len(tok), D))
    dprob = np.zeros((len(tok), K))
    dh = np.zeros((len(tok), K, 2 * F))
    for i, t in enumerate(tok):
        dyt = np.asarray(dy[t], np.float64)
        for k in range(K):
            e = int(topk_idx[t, k])
            if not 0 <= e < E:
                continue
            W1e, W2e = W.get(e)
            dprob[i, k] = dyt @ fwd["o"][i, k]
            dh[i, k], dxc = _pair_backward(W1e, W2e, dyt, fwd["h"][i, k],
                                           float(topk_w[t, k]), F)
            dx[i] += dxc
    return dict(y=fwd["y"], h=fwd["h"], a=fwd["a"], o=fwd["o"],
                dx=dx, dprob=dprob, dh=dh)


def wgrad_rows(dy, x, topk_idx, topk_w, w1, w2, e, rows_w1, rows_w2) -> dict:
    """Selected rows of dW1[e] and dW2[e] (sum over that expert's pairs).

    rows_w1 index the 2F rows of dW1[e]; rows_w2 index the D rows of dW2[e].
    The pairs of expert e are stacked in ascending p and the per-pair products
    of the definition are taken as matrix products over that stack (a library
    matmul as one step); the sums over pairs are the same definition.
    """
    x = np.asarray(x)
    dy = np.asarray(dy)
    E, F2, D = w1.shape
    F = F2 // 2
    K = topk_idx.shape[1]
    W1e = np.asarray(w1[e], np.float64)
    W2e = np.asarray(w2[e], np.float64)
    rows_w1 = np.asarray(rows_w1)
    rows_w2 = np.asarray(rows_w2)
    p = np.nonzero(np.asarray(topk_idx).reshape(-1) == e)[0]
    t = p // K
    w = np.asarray(topk_w, np.float64).reshape(-1)[p][:, None]
    X = x[t].astype(np.float64)            # [n_e, D]
    dY = dy[t].astype(np.float64)          # [n_e, D]
    H = X @ W1e.T                          # h of every pair
    g, u = H[:, :F], H[:, F:]
    A = silu(g) * u
    s = sigmoid(g)
    dA = w * (dY @ W2e)                    # w * W2^T dy, per pair
    dH = np.concatenate([dA * u * s * (1.0 + g * (1.0 - s)), dA * (g * s)], axis=1)
    dw2 = (w * dY[:, rows_w2]).T @ A       # sum_p (w dy)[rows] a^T
    dw1 = dH[:, rows_w1].T @ X             # sum_p dh[rows] x^T
    return dict(dw1=dw1, dw2=dw2, n_pairs=len(p))
