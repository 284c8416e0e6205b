"""Host-side checks of bench.py's contract that need no GPU: the refusal of more
than one GPU (the layer's expert-parallel exchange is not part of this library),
and the algorithmic byte counts behind the reported HBM rates."""
import os
import subprocess
import sys

import moe_inputs as mi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_for_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_row_mover_bytes_follow_the_definitions():
    b = _bench_module()
    cfg = mi.CONFIGS["30b"]
    T, N, D = cfg.T, cfg.N, cfg.D
    # bf16 at the 30B shape: the GEMMs carry the routing weights and the dispatch
    assert b.weights_in_gemms(cfg)
    wide = b.row_bytes(cfg)
    assert "dispatch" not in wide
    # unweighted combine: every pair's row read, the token row written, pos read
    assert wide["combine"] == 2 * N * D + 2 * T * D + N * 4
    # the backward's dispatch of dy: dy once, every pair's row written, pos read
    assert wide["dispatch_dy"] == 2 * T * D + 2 * N * D + N * 4
    assert wide["dprob_reduce"] == N * 4 * (2 + cfg.F // 64)
    # the same shape where the weights stay in the row movers (fp32 I/O with bf16 GEMMs)
    rb = b.row_bytes(mi.LayerConfig("30b_io", T=T, D=D, F=cfg.F, E=cfg.E, K=cfg.K,
                                    mode=mi.MODE_FP32_BF16GEMM))
    # dispatch: x once, every pair's row written, pos read, wperm written, topk_w read
    assert rb["dispatch"] == 2 * T * D + 2 * N * D + 3 * N * 4
    # combine / un-permute: every pair's row read, the token row written, indices (+ weights)
    assert rb["combine"] == 2 * N * D + 2 * T * D + N * 8
    assert rb["unpermute"] == 2 * N * D + 2 * T * D + N * 4
    # combine-backward: dy once, pair rows read (O) and written (w * dy), 3 index/weight arrays
    assert rb["dispatch_dy"] == 2 * T * D + 4 * N * D + 3 * N * 4
    # the FP8 forward modes' dispatch writes e4m3 codes and one 4-byte entry per 128 columns
    # instead of the bf16 rows (both under activation recompute)
    codes = N * D + N * (D // 128) * 4
    mx = mi.CONFIGS["30b_mxfp8"]
    assert b.row_bytes(mx)["dispatch"] - rb["dispatch"] == codes - 2 * N * D
    assert b.row_bytes(mx, recompute=True)["dispatch"] - rb["dispatch"] == codes
    # the blockwise combine-backward writes dYw's codes instead of its bf16 rows; the MXFP8
    # one neither (it computes only dtopk_w)
    assert b.row_bytes(mi.CONFIGS["30b_fp8"])["dispatch_dy"] - rb["dispatch_dy"] == codes - 2 * N * D
    assert b.row_bytes(mx)["dispatch_dy"] - rb["dispatch_dy"] == -2 * N * D
    fb = mi.CONFIGS["235b_fp8bwd"]
    fcodes = fb.N * fb.D + fb.N * (fb.D // 128) * 4
    io = b.row_bytes(mi.LayerConfig("235b_io", T=fb.T, D=fb.D, F=fb.F, E=fb.E, K=fb.K,
                                    mode=mi.MODE_FP32_BF16GEMM))
    assert b.row_bytes(fb)["dispatch"] == io["dispatch"]
    assert b.row_bytes(fb)["dispatch_dy"] - io["dispatch_dy"] == fcodes - 2 * fb.N * fb.D
