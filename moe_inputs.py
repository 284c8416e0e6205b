"""Seeded synthetic inputs for the single-GPU trainable MoE layer.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds no arithmetic of the layer itself: it only draws the
tensors the layer consumes (activations, expert weights, upstream gradient and
a top-k routing decision) and rounds them to the storage precision.

Workload shapes follow the pages' layer benchmark (Prime Mega MoE news item,
section "How fast is Prime Mega MoE?": Qwen3-30B-A3B and Qwen3-235B-A22B MoE
layers, 128 experts, top-8, random routing, 16,384-token sequences).  The model
dim D and expert FFN dim F of each shape, the value distributions and the skewed
routing variant are this project's readings (the pages do not state them):

* x, dY ~ N(0, 1); W1 = [E, 2F, D] and W2 = [E, D, F] ~ N(0, 0.02) (std 0.02).
* Router logits ~ N(0, 1) -> softmax over experts -> top-k by descending
  probability (ties to the lower expert index) -> the k weights renormalised to
  sum to 1, all in fp32.
* Skewed routing: a seeded permutation pi of the experts; the last 8 entries of
  pi are dead (bias -inf), the others get a finite Zipf(s=1.2) rank-frequency
  bias ln(r^-s / sum_r' r'^-s) with rank r = 1.. in pi's order, added to the
  logits before the softmax.

Every tensor gets its own numpy PCG64 child stream spawned from one
SeedSequence, in a fixed order (logits, permutation, x, W1, W2, dY, then the
router's upstream gradient dtopk_w), so a tensor does not change when another is
resized.  Expert weights take one child per expert so they can be drawn in
parallel threads.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Storage modes of the layer (mirrors the C descriptor's mode field).
MODE_FP32 = 0            # fp32 storage and fp32 GEMMs
MODE_FP32_BF16GEMM = 1   # fp32 storage, GEMM operands rounded to bf16
MODE_BF16 = 2            # bf16 storage, bf16 GEMMs with fp32 accumulation
MODE_FP8_BWD = 3         # bf16 forward, blockwise-FP8 backward GEMMs
MODE_MXFP8 = 4           # MXFP8 GEMMs forward and backward
MODE_FP8 = 5             # blockwise FP8 forward and backward


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    D: int
    F: int
    E: int
    K: int
    mode: int = MODE_BF16
    routing: str = "uniform"   # "uniform" | "zipf" | "dead<k>" (k experts get no tokens)
    seed: int = 1000

    @property
    def N(self) -> int:
        return self.T * self.K

    @property
    def io_is_bf16(self) -> bool:
        return self.mode >= MODE_BF16

    def fwd_flops(self) -> float:
        # two GEMMs: W1 (2F x D) and W2 (D x F) per routed pair, 2 flops per MAC
        return 6.0 * self.T * self.K * self.D * self.F

    def bwd_flops(self) -> float:
        # four GEMMs: dgrad and wgrad of both linear layers
        return 12.0 * self.T * self.K * self.D * self.F


# The five layer workloads (tiny parity case, then the two Qwen3 shapes in three
# precisions), followed by extra parity shapes that span several tiles and
# ragged per-expert tails.
CONFIGS = {
    "tiny": LayerConfig("tiny", T=64, D=128, F=64, E=8, K=2, mode=MODE_FP32, seed=1000),
    "tiny_bf16gemm": LayerConfig("tiny_bf16gemm", T=64, D=128, F=64, E=8, K=2,
                                 mode=MODE_FP32_BF16GEMM, seed=1000),
    "30b": LayerConfig("30b", T=16384, D=2048, F=768, E=128, K=8, seed=1001),
    "235b": LayerConfig("235b", T=16384, D=4096, F=1536, E=128, K=8, seed=1002),
    "235b_fp8bwd": LayerConfig("235b_fp8bwd", T=16384, D=4096, F=1536, E=128, K=8,
                               mode=MODE_FP8_BWD, seed=1003),
    "30b_mxfp8": LayerConfig("30b_mxfp8", T=16384, D=2048, F=768, E=128, K=8,
                             mode=MODE_MXFP8, routing="zipf", seed=1004),
    # blockwise FP8 in both passes (the pages' "fp8" precision) at the 30B shape
    "30b_fp8": LayerConfig("30b_fp8", T=16384, D=2048, F=768, E=128, K=8, mode=MODE_FP8,
                           seed=1007),
    # one expert-parallel rank's share (EP = 8): 16 local experts receiving the
    # 131072 routed rows of the 30B/235B layers, one row per received pair
    # (top-1 over the local experts), so n_e is about 8192 and N, D, F and the
    # flop count are those of the whole-layer workloads
    "30b_ep_share": LayerConfig("30b_ep_share", T=131072, D=2048, F=768, E=16, K=1, seed=1005),
    "235b_ep_share": LayerConfig("235b_ep_share", T=131072, D=4096, F=1536, E=16, K=1,
                                 seed=1006),
    # parity shapes
    "small_bf16": LayerConfig("small_bf16", T=200, D=192, F=128, E=16, K=4, seed=2001),
    "mid_bf16": LayerConfig("mid_bf16", T=700, D=512, F=256, E=8, K=2, seed=2002),
    "dead_bf16": LayerConfig("dead_bf16", T=300, D=256, F=192, E=12, K=3,
                             routing="dead4", seed=2003),
    "wide_bf16": LayerConfig("wide_bf16", T=1100, D=1024, F=512, E=8, K=2, seed=2004),
    # fp32 I/O with bf16 GEMMs, and skewed routing with dead experts, at shapes
    # the persistent forward takes (D % 256 == 0, F % 128 == 0)
    "mid_f32io": LayerConfig("mid_f32io", T=700, D=512, F=256, E=8, K=2,
                             mode=MODE_FP32_BF16GEMM, seed=2005),
    "zipf_bf16": LayerConfig("zipf_bf16", T=900, D=256, F=128, E=16, K=4, routing="zipf",
                             seed=2006),
    # skewed routing with dead experts at a shape the paired backward takes
    # (D % 256 == 0, F % 256 == 0)
    "zipf_wide_bf16": LayerConfig("zipf_wide_bf16", T=1500, D=512, F=256, E=16, K=4,
                                  routing="zipf", seed=2009),
    # two experts of about 4200 rows each (above the mean expert size up to
    # which bf16 pairs its backward GEMMs by default)
    "deep_bf16": LayerConfig("deep_bf16", T=8400, D=256, F=256, E=2, K=1, seed=2010),
    # token rows of 512 and 1024 16-byte chunks (the row movers give each thread
    # several chunks of a row), top-8, bf16 I/O and fp32 I/O
    "rows4k_bf16": LayerConfig("rows4k_bf16", T=96, D=4096, F=128, E=12, K=8, seed=2007),
    "rows8k_f32io": LayerConfig("rows8k_f32io", T=40, D=8192, F=128, E=8, K=8,
                                mode=MODE_FP32_BF16GEMM, seed=2008),
    # degenerate shapes: one token; one expert; every expert chosen (K = E)
    "one_token": LayerConfig("one_token", T=1, D=128, F=64, E=4, K=2, seed=2101),
    "one_expert": LayerConfig("one_expert", T=100, D=128, F=64, E=1, K=1, seed=2102),
    "all_experts": LayerConfig("all_experts", T=50, D=128, F=128, E=8, K=8, seed=2103),
    # FP8 parity shapes (D, F multiples of 256): experts with several 256-row
    # tiles and 128-token steps, experts with fewer than 128 tokens, dead experts
    "fp8bwd_small": LayerConfig("fp8bwd_small", T=600, D=512, F=256, E=4, K=2,
                                mode=MODE_FP8_BWD, seed=3001),
    "mxfp8_small": LayerConfig("mxfp8_small", T=600, D=512, F=256, E=4, K=2,
                               mode=MODE_MXFP8, seed=3002),
    "fp8_small": LayerConfig("fp8_small", T=600, D=512, F=256, E=4, K=2,
                             mode=MODE_FP8, seed=3003),
    "mxfp8_zipf_small": LayerConfig("mxfp8_zipf_small", T=512, D=256, F=256, E=16, K=4,
                                    mode=MODE_MXFP8, routing="zipf", seed=3004),
}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round a float32 array to the nearest bfloat16 value (ties to even), in place.

    Returns the same array, whose float32 values are now exactly representable
    in bfloat16.  Inputs must be finite.
    """
    assert a.dtype == np.float32
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF) + lsb
    u &= np.uint32(0xFFFF0000)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The upper 16 bits of bf16-representable float32 values, as uint16."""
    assert a.dtype == np.float32
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """float32 values of bfloat16 bit patterns."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _router_logits(rng_logits: np.random.Generator, rng_perm: np.random.Generator,
                   cfg: LayerConfig) -> np.ndarray:
    """Router logits [T, E] float32: N(0, 1) draws plus the routing variant's
    per-expert bias (-inf for dead experts)."""
    T, E = cfg.T, cfg.E
    logits = rng_logits.standard_normal((T, E), dtype=np.float32)
    bias = np.zeros(E, np.float32)
    if cfg.routing == "zipf":
        perm = rng_perm.permutation(E)
        live = E - 8
        s = 1.2
        r = np.arange(1, live + 1, dtype=np.float64)
        freq = r ** -s
        b = np.log(freq / freq.sum())
        bias[perm[:live]] = b.astype(np.float32)
        bias[perm[live:]] = -np.inf
    elif cfg.routing.startswith("dead"):
        ndead = int(cfg.routing[4:])
        perm = rng_perm.permutation(E)
        bias[perm[E - ndead:]] = -np.inf
    elif cfg.routing != "uniform":
        raise ValueError(cfg.routing)
    return logits + bias[None, :]


def _route(rng_logits: np.random.Generator, rng_perm: np.random.Generator,
           cfg: LayerConfig):
    """Draw logits and turn them into a top-k routing decision (input generation:
    the layer consumes a routing decision; the router step itself is checked
    against its own oracle, never against this draw)."""
    K = cfg.K
    z = _router_logits(rng_logits, rng_perm, cfg)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z, dtype=np.float32)
    p /= p.sum(axis=1, keepdims=True)
    # top-k by descending probability, ties to the lower expert index
    order = np.argsort(-p, axis=1, kind="stable")[:, :K]
    idx = order.astype(np.int32)
    pw = np.take_along_axis(p, order, axis=1)
    w = (pw / pw.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx, w


def make_routing(cfg: LayerConfig):
    """Only the routing decision (topk_idx, topk_w) of a workload."""
    ss = np.random.SeedSequence(cfg.seed)
    c_logits, c_perm = ss.spawn(6)[:2]
    return _route(np.random.Generator(np.random.PCG64(c_logits)),
                  np.random.Generator(np.random.PCG64(c_perm)), cfg)


def make_router_inputs(cfg: LayerConfig) -> dict:
    """Inputs of the router step of a workload: the float32 logits [T, E] the
    workload's routing decision is drawn from, and an upstream gradient
    dtopk_w [T, K] ~ N(0, 1) float32 (its own child stream)."""
    ss = np.random.SeedSequence(cfg.seed)
    kids = ss.spawn(7)
    c_logits, c_perm, c_dw = kids[0], kids[1], kids[6]
    z = _router_logits(np.random.Generator(np.random.PCG64(c_logits)),
                       np.random.Generator(np.random.PCG64(c_perm)), cfg)
    dw = np.random.Generator(np.random.PCG64(c_dw)).standard_normal((cfg.T, cfg.K), dtype=np.float32)
    return {"logits": np.ascontiguousarray(z, np.float32), "dtopk_w": dw}


def make_inputs(cfg: LayerConfig, threads: int = 8, with_dy: bool = True,
                experts=None) -> dict:
    """Seeded inputs of one layer workload.

    Returns float32 arrays x [T,D], w1 [E,2F,D], w2 [E,D,F], dy [T,D]; int32
    topk_idx [T,K]; float32 topk_w [T,K].  In bf16 storage modes the float
    tensors hold bf16-representable values (rounded once, ties to even), and
    both the GPU and the oracle consume exactly these values.

    `experts` (a list of expert ids) draws only those experts' weights, each
    equal to its draw in the full set (one child stream per expert); the other
    experts' weights are left zero and their pages untouched, so checks of a
    few experts at the full Qwen3 shapes stay cheap on the host.
    """
    ss = np.random.SeedSequence(cfg.seed)
    c_logits, c_perm, c_x, c_w1, c_w2, c_dy = ss.spawn(6)
    idx, w = _route(np.random.Generator(np.random.PCG64(c_logits)),
                    np.random.Generator(np.random.PCG64(c_perm)), cfg)
    rnd = cfg.mode != MODE_FP32 and cfg.mode != MODE_FP32_BF16GEMM

    x = _normal(np.random.Generator(np.random.PCG64(c_x)), (cfg.T, cfg.D), 1.0)
    alloc = np.empty if experts is None else np.zeros
    w1 = alloc((cfg.E, 2 * cfg.F, cfg.D), np.float32)
    w2 = alloc((cfg.E, cfg.D, cfg.F), np.float32)
    keep = set(range(cfg.E)) if experts is None else {int(e) for e in experts}

    def fill(args):
        arr, child, e = args
        arr[e] = _normal(np.random.Generator(np.random.PCG64(child)), arr.shape[1:], 0.02)
        if rnd:
            bf16_round(arr[e])

    jobs = [(w1, c, e) for e, c in enumerate(c_w1.spawn(cfg.E)) if e in keep]
    jobs += [(w2, c, e) for e, c in enumerate(c_w2.spawn(cfg.E)) if e in keep]
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(fill, jobs))
    out = dict(x=x, w1=w1, w2=w2, topk_idx=idx, topk_w=w)
    if with_dy:
        out["dy"] = _normal(np.random.Generator(np.random.PCG64(c_dy)), (cfg.T, cfg.D), 1.0)
    if rnd:
        bf16_round(out["x"])
        if with_dy:
            bf16_round(out["dy"])
    return out
