"""The rocprofv3 summary tool's kernel naming (host only, synthetic trace rows).

The committed profiles name each launch by the layer step it performs; where
the bf16 GEMMs carry the routing weights, the combine and the un-permute are the
same unweighted gather-reduce kernel and only their place in the step tells
them apart, and the row dispatch kernel moves dy.
"""
from __future__ import annotations

from mixture_experts_layer_31_amd import profile_summary as ps

GR = "void moe::(anonymous namespace)::gather_reduce_kernel<unsigned short, unsigned short, {w}, 8>(...)"
W2 = ("void moe::(anonymous namespace)::grouped_gemm_kernel<moe::gemm::Tile<256, 256, 2, 4, 2, true>, "
      "false, 0>(moe::gemm::GroupedArgs)")
W1 = ("void moe::(anonymous namespace)::grouped_gemm_kernel<moe::gemm::Tile<256, 256, 2, 4, 2, true>, "
      "false, 1>(moe::gemm::GroupedArgs)")
PAIR1 = ("void moe::(anonymous namespace)::pair_kernel<moe::gemm::Tile<256, 256, 2, 4, 4, false>, true, 0, "
         "moe::gemm::Tile<256, 256, 2, 4, 4, false>, false>(...)")
DISP = "void moe::(anonymous namespace)::dispatch_rows_kernel<4, 0>(...)"


def _rows(names):
    return [{"Kernel_Name": n, "Dispatch_Id": str(i + 1)} for i, n in enumerate(names)]


def _named(names, dy_dispatch):
    ps.DY_DISPATCH["flag"] = dy_dispatch
    try:
        return [n for n, _ in ps.name_rows(_rows(names))]
    finally:
        ps.DY_DISPATCH["flag"] = False


def test_unweighted_gathers_are_named_by_their_place_in_the_step():
    step = [W1, W2, GR.format(w="false"), DISP, PAIR1, GR.format(w="false")]
    assert _named(step, True) == ["gemm_w1_swiglu", "gemm_w2", "combine", "dispatch_dy",
                                  "pair_w1", "unpermute"]


def test_weighted_combine_and_forward_dispatch_keep_their_names():
    step = [DISP, W1, W2, GR.format(w="true"), PAIR1, GR.format(w="false")]
    assert _named(step, False) == ["dispatch", "gemm_w1_swiglu", "gemm_w2", "combine",
                                   "pair_w1", "unpermute"]


def test_rows_are_taken_in_dispatch_order():
    rows = _rows([W2, GR.format(w="false")])
    rows.reverse()  # a trace file lists them by completion, not by dispatch
    ps.DY_DISPATCH["flag"] = True
    try:
        assert [n for n, _ in ps.name_rows(rows)] == ["gemm_w2", "combine"]
    finally:
        ps.DY_DISPATCH["flag"] = False
