"""The seeded input generator: bf16 rounding, determinism and routing structure."""
import numpy as np
import torch

import moe_inputs as mi


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s for s in (1e-3, 1, 1e4)])
    # exact ties: bf16 value + half an ulp
    b = mi.from_bf16_bits(np.arange(0x3F80, 0x3F90, dtype=np.uint16))
    ties = (b.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    a = np.concatenate([a, ties, -ties])
    ref = torch.from_numpy(a.copy()).to(torch.bfloat16).float().numpy()
    got = mi.bf16_round(a.copy())
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(mi.from_bf16_bits(mi.bf16_bits(got)), got)


def test_inputs_deterministic_and_rounded():
    cfg = mi.CONFIGS["small_bf16"]
    a = mi.make_inputs(cfg)
    b = mi.make_inputs(cfg, threads=1)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    for k in ("x", "w1", "w2", "dy"):
        assert a[k].dtype == np.float32
        np.testing.assert_array_equal(mi.bf16_round(a[k].copy()), a[k])
    assert a["w1"].shape == (cfg.E, 2 * cfg.F, cfg.D) and a["w2"].shape == (cfg.E, cfg.D, cfg.F)
    assert 0.015 < a["w1"].std() < 0.025


def test_routing_structure():
    for name in ("tiny", "30b", "dead_bf16"):
        cfg = mi.CONFIGS[name]
        idx, w = mi.make_routing(cfg)
        assert idx.shape == (cfg.T, cfg.K) and idx.dtype == np.int32
        assert np.all((idx >= 0) & (idx < cfg.E))
        assert all(len(set(r)) == cfg.K for r in idx[:2000])
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
        assert np.all(w > 0)
    idx, _ = mi.make_routing(mi.CONFIGS["dead_bf16"])
    assert (np.bincount(idx.ravel(), minlength=12) == 0).sum() == 4


def test_zipf_routing_is_skewed_with_eight_dead_experts():
    cfg = mi.CONFIGS["30b_mxfp8"]
    idx, w = mi.make_routing(cfg)
    counts = np.bincount(idx.ravel(), minlength=cfg.E)
    assert (counts == 0).sum() == 8
    assert counts.sum() == cfg.N
    top16 = np.sort(counts)[::-1][:16].sum() / cfg.N
    assert top16 > 0.6
    assert counts.max() > 8 * cfg.N / cfg.E


def test_expert_subset_draws_the_same_weights():
    cfg = mi.CONFIGS["dead_bf16"]
    full = mi.make_inputs(cfg)
    sub = mi.make_inputs(cfg, experts=[7, 2])
    for k in ("x", "dy", "topk_idx", "topk_w"):
        np.testing.assert_array_equal(sub[k], full[k])
    for e in range(cfg.E):
        for k in ("w1", "w2"):
            if e in (2, 7):
                np.testing.assert_array_equal(sub[k][e], full[k][e])
            else:
                assert not sub[k][e].any()
