"""A seeded sweep of small layer shapes against the CPU oracle, through the C ABI.

The named parity shapes pick particular cases; this sweep draws twenty more
(plus four fixed edge cases listed with them) from fixed ranges (D and F multiples of 64, one to 33 experts, top-1 to top-8,
one to 700 tokens, uniform, dead-expert and skewed routing, bf16 and fp32-I/O
modes, each backward schedule and activation recompute), so that both the
path where the bf16 GEMMs carry the routing weights and the dispatch (2F a
multiple of 256) and the one where the row movers do are met at many ragged
tile counts.  Each case is held to the oracle at the same bound as the named
shapes (1e-2 per output and intermediate; routing bit-exact).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_layer_31_amd as moe
import moe_inputs as mi
from tests.oracle_parity import layer_vs_oracle

pytestmark = pytest.mark.gpu


def _cases(n=20, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([64, 128, 192, 256, 384, 512]))
        F = int(rng.choice([64, 128, 192, 256, 384]))
        E = int(rng.choice([1, 2, 5, 8, 16, 33]))
        K = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([1, 64, 150, 333, 700]))
        kinds = ["uniform"] + (["dead"] if E - K >= 1 else []) + (["zipf"] if E >= K + 8 else [])
        kind = kinds[int(rng.integers(len(kinds)))]
        routing = kind if kind != "dead" else f"dead{int(rng.integers(1, E - K + 1))}"
        mode = mi.MODE_FP32_BF16GEMM if rng.random() < 0.25 else mi.MODE_BF16
        flags = [0, moe.MOE_FLAG_SERIAL_BWD, moe.MOE_FLAG_RECOMPUTE]
        if mode == mi.MODE_BF16 and D % 256 == 0 and F % 256 == 0:
            flags.append(moe.MOE_FLAG_OVERLAP_BWD)
        flag = flags[int(rng.integers(len(flags)))]
        cfg = mi.LayerConfig(f"sweep{i}", T=T, D=D, F=F, E=E, K=K, mode=mode, routing=routing,
                             seed=5000 + i)
        out.append((cfg, flag))
    return out


# and the expert counts past the paired backward's limit (256) up to the
# descriptor's (1024), where the routing blocks loop over experts; and weight-
# gradient tile grids that end in partial blocks of the 4 x 8 tile order (W1:
# 2 x 9 tiles of 256, W2: 9 x 1), one kernel per GEMM and paired
CASES = _cases() + [
    (mi.LayerConfig("many_experts", T=200, D=128, F=128, E=300, K=8, seed=5100), 0),
    (mi.LayerConfig("max_experts", T=500, D=64, F=64, E=1024, K=4, routing="dead100", seed=5101), 0),
    (mi.LayerConfig("wgrad_grid", T=96, D=2304, F=256, E=3, K=2, seed=5102), moe.MOE_FLAG_SERIAL_BWD),
    (mi.LayerConfig("wgrad_grid_pair", T=96, D=2304, F=256, E=3, K=2, seed=5103), 0),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    moe.lib()


@pytest.mark.parametrize("cfg,flags", CASES,
                         ids=[f"{c.name}-T{c.T}-D{c.D}-F{c.F}-E{c.E}-K{c.K}-{c.routing}-m{c.mode}-f{f}"
                              for c, f in CASES])
def test_swept_shape_matches_oracle(cfg, flags):
    print(f"[case] {cfg.name} T={cfg.T} D={cfg.D} F={cfg.F} E={cfg.E} K={cfg.K} "
          f"routing={cfg.routing} mode={cfg.mode} flags={flags}", flush=True)
    layer_vs_oracle(cfg, mi.make_inputs(cfg), flags)
