"""The overlapped forward's ticket schedule, checked on the CPU (host mirror of
its table construction, tests/queue_tables.py).

For routings with uniform, Zipf-skewed, dead-expert, all-on-two-experts,
one-expert and out-of-range expert ids: the tickets are a bijection onto the
dispatch items, W1 tiles and W2 tiles; every wait targets an item of the same
queue with a smaller ticket (the property that makes the one-item-per-
workgroup launch free of deadlock whether or not its workgroups are
co-resident); each queue's dispatch items copy exactly the rows its W1 tiles
read; the table fits its scratch region and every queue has a workgroup for
every ticket.  The earlier looped variant's tables fail the same-queue
property (its W1 tiles wait on other queues' dispatch items).
"""
import numpy as np
import pytest

import moe_inputs as mi
from oracle import moe_oracle as orc
from tests import queue_tables as qt


def _routings():
    out = []
    for name in ("mid_bf16", "zipf_bf16", "dead_bf16", "wide_bf16", "30b", "30b_mxfp8"):
        cfg = mi.CONFIGS[name]
        idx, _ = mi.make_routing(cfg)
        out.append((name, cfg, idx))
    cfg = mi.CONFIGS["mid_bf16"]
    idx, _ = mi.make_routing(cfg)
    two = np.zeros_like(idx)
    two[:, 1] = 1
    two[::3] = two[::3, ::-1]
    out.append(("mid_bf16/two_experts", cfg, two))
    bad = idx.copy()
    bad[5, 0] = cfg.E + 3
    bad[611, 1] = -1
    bad[:40, :] = cfg.E + 1  # a run of invalid ids: fewer valid rows than pairs
    out.append(("mid_bf16/out_of_range", cfg, bad))
    one = mi.LayerConfig("one_expert_256", T=1000, D=512, F=256, E=1, K=1)
    out.append(("one_expert", one, np.zeros((one.T, 1), np.int32)))
    rng = np.random.default_rng(5)
    for E, K, T in ((16, 4, 3000), (128, 8, 2500), (3, 2, 700)):
        cfg = mi.LayerConfig(f"rand{E}", T=T, D=512, F=256, E=E, K=K)
        r = np.argsort(rng.random((T, E)) ** np.linspace(0.3, 3, E), axis=1)[:, :K]
        out.append((f"random E={E} K={K}", cfg, r.astype(np.int32)))
    return out


ROUTINGS = _routings()


@pytest.mark.parametrize("case", range(len(ROUTINGS)), ids=[r[0] for r in ROUTINGS])
def test_schedule_properties(case):
    name, cfg, idx = ROUTINGS[case]
    r = orc.route(idx, cfg.E)
    t = qt.build(r["offsets"], 2 * cfg.F // 256, cfg.D // 256)
    qt.check(t, cfg.N)
    assert t["nvalid"] == int(((idx >= 0) & (idx < cfg.E)).sum())


def test_a_planted_wrong_lead_is_caught():
    """The check fails when the table places a W1 tile ahead of its rows' items."""
    name, cfg, idx = ROUTINGS[0]
    r = orc.route(idx, cfg.E)
    old = qt.LEAD
    try:
        qt.LEAD = -3
        t = qt.build(r["offsets"], 2 * cfg.F // 256, cfg.D // 256)
        with pytest.raises(AssertionError):
            qt.check(t, cfg.N)
    finally:
        qt.LEAD = old


def test_looped_variant_waits_across_queues():
    """The earlier looped persistent variant split the dispatch items into queues
    by item index and the W1 tiles by tile index, independently: on the first
    parity workload 14 of its 58 waits targeted another queue's items, so a
    workgroup's progress depended on workgroups of other queues."""
    cfg = mi.CONFIGS["mid_bf16"]
    idx, _ = mi.make_routing(cfg)
    r = orc.route(idx, cfg.E)
    v = qt.build_looped_variant(r["offsets"], cfg.N, 2 * cfg.F // 256, cfg.D // 256)
    waits = [(k, w) for k, ws in v["waits"].items() for w in ws]
    cross = [1 for k, w in waits if w[0] != k[0]]
    assert len(waits) == 58 and len(cross) == 14
