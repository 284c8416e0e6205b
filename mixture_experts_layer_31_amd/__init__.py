"""Python binding of the MI355X MoE layer's C ABI (include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP library
libmoe_mi355x.so built in-tree by ``mixture_experts_layer_31_amd.build``.  The
functions below carry the C names; tensors are torch tensors on the GPU (or
None for optional pointers) and `stream` defaults to torch's current stream.
Loading fails loudly when the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_FP32, MOE_FP32_BF16GEMM, MOE_BF16, MOE_FP8_BWD, MOE_MXFP8, MOE_FP8 = range(6)
MOE_OK, MOE_EINVAL, MOE_ESCRATCH, MOE_EALIGN, MOE_EUNSUPPORTED, MOE_EHIP, MOE_EINDEX, \
    MOE_ETIMEOUT = 0, -1, -2, -3, -4, -5, -6, -7
MOE_FLAG_OVERLAP = 0x1
MOE_FLAG_QUEUE_TIMEOUT_TEST = 0x2
MOE_FLAG_RECOMPUTE = 0x4
MOE_FLAG_OVERLAP_BWD = 0x8
MOE_FLAG_SERIAL_BWD = 0x10
MOE_NOALLOC_SCRATCH_BYTES = 256 << 20
(MOE_VIEW_XPERM, MOE_VIEW_H, MOE_VIEW_A, MOE_VIEW_O, MOE_VIEW_DYPERM, MOE_VIEW_DH,
 MOE_VIEW_DXPERM, MOE_VIEW_WPERM, MOE_VIEW_Q_ROWS, MOE_VIEW_Q_ROWS_SCALE, MOE_VIEW_Q_TOK_A,
 MOE_VIEW_Q_TOK_A_SCALE, MOE_VIEW_Q_TOK_B, MOE_VIEW_Q_TOK_B_SCALE, MOE_VIEW_QUEUE) = range(15)

# Exported symbols, in the order include/moe.h declares them.
EXPORTS = (
    "moe_scratch_bytes", "moe_wprep_bytes", "moe_prepare_weights", "moe_route",
    "moe_routing_view", "moe_scratch_view", "moe_fwd", "moe_bwd", "moe_fwd_noalloc", "moe_router_fwd",
    "moe_router_bwd", "moe_check", "moe_strerror", "moe_abi_version", "moe_profile_enable", "moe_profile_collect",
    "moe_profile_get", "moe_profile_reset",
)


class moe_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "D", "F", "E", "K", "mode", "flags")]


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} ({code})")


_lib = None
_vp, _sz, _i32, _i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64
_dp = ctypes.POINTER(moe_desc)


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m mixture_experts_layer_31_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "moe_scratch_bytes": (_sz, [_dp]),
            "moe_wprep_bytes": (_sz, [_dp]),
            "moe_prepare_weights": (_i32, [_dp, _vp, _vp, _vp, _sz, _vp]),
            "moe_route": (_i32, [_dp, _vp, _vp, _sz, _vp]),
            "moe_routing_view": (_i32, [_dp, _vp, _sz] + [ctypes.POINTER(_vp)] * 4),
            "moe_scratch_view": (_i32, [_dp, _vp, _sz, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_sz)]),
            "moe_fwd": (_i32, [_dp] + [_vp] * 8 + [_sz, _vp]),
            "moe_bwd": (_i32, [_dp] + [_vp] * 10 + [_sz, _vp]),
            "moe_fwd_noalloc": (_i32, [_dp] + [_vp] * 8),
            "moe_router_fwd": (_i32, [_dp, _vp, _vp, _vp, _vp]),
            "moe_router_bwd": (_i32, [_dp, _vp, _vp, _vp, _vp, _vp]),
            "moe_check": (_i32, [_dp, _vp, _sz, _vp]),
            "moe_strerror": (ctypes.c_char_p, [_i32]),
            "moe_abi_version": (_i32, []),
            "moe_profile_enable": (_i32, [_i32]),
            "moe_profile_collect": (_i32, []),
            "moe_profile_get": (_i32, [_i32, ctypes.POINTER(ctypes.c_char_p),
                                       ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
            "moe_profile_reset": (_i32, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _p(t):
    """Device address of a tensor (or None), as a ctypes pointer."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def make_desc(T, D, F, E, K, mode=MOE_BF16, flags=0) -> moe_desc:
    return moe_desc(T, D, F, E, K, mode, flags)


def strerror(code: int) -> str:
    return lib().moe_strerror(code).decode()


def abi_version() -> int:
    return lib().moe_abi_version()


def moe_scratch_bytes(desc: moe_desc) -> int:
    return lib().moe_scratch_bytes(ctypes.byref(desc))


def moe_wprep_bytes(desc: moe_desc) -> int:
    return lib().moe_wprep_bytes(ctypes.byref(desc))


def moe_prepare_weights(desc, w1, w2, wprep, stream=None) -> int:
    return lib().moe_prepare_weights(ctypes.byref(desc), _p(w1), _p(w2), _p(wprep),
                                     0 if wprep is None else _nbytes(wprep), _stream(stream))


def moe_route(desc, topk_idx, scratch, stream=None) -> int:
    return lib().moe_route(ctypes.byref(desc), _p(topk_idx), _p(scratch), _nbytes(scratch),
                           _stream(stream))


def moe_router_fwd(desc, logits, topk_idx, topk_w, stream=None) -> int:
    return lib().moe_router_fwd(ctypes.byref(desc), _p(logits), _p(topk_idx), _p(topk_w),
                                _stream(stream))


def moe_router_bwd(desc, topk_idx, topk_w, dtopk_w, dlogits, stream=None) -> int:
    return lib().moe_router_bwd(ctypes.byref(desc), _p(topk_idx), _p(topk_w), _p(dtopk_w),
                                _p(dlogits), _stream(stream))


def moe_routing_view(desc, scratch) -> tuple:
    """(status, counts, offsets, pos, src) device addresses inside scratch."""
    out = [_vp() for _ in range(4)]
    rc = lib().moe_routing_view(ctypes.byref(desc), _p(scratch), _nbytes(scratch),
                                *[ctypes.byref(o) for o in out])
    return (rc, *[o.value for o in out])


def moe_scratch_view(desc, scratch, which: int) -> tuple:
    """(status, device address, bytes) of an intermediate inside scratch."""
    ptr, n = _vp(), _sz()
    rc = lib().moe_scratch_view(ctypes.byref(desc), _p(scratch), _nbytes(scratch), which,
                                ctypes.byref(ptr), ctypes.byref(n))
    return rc, ptr.value, n.value


def moe_fwd(desc, x, topk_idx, topk_w, w1, w2, wprep, y, scratch, stream=None) -> int:
    return lib().moe_fwd(ctypes.byref(desc), _p(x), _p(topk_idx), _p(topk_w), _p(w1), _p(w2),
                         _p(wprep), _p(y), _p(scratch), _nbytes(scratch), _stream(stream))


def moe_fwd_noalloc(desc, x, topk_idx, topk_w, w1, w2, wprep, y, stream=None) -> int:
    return lib().moe_fwd_noalloc(ctypes.byref(desc), _p(x), _p(topk_idx), _p(topk_w), _p(w1),
                                 _p(w2), _p(wprep), _p(y), _stream(stream))


def moe_bwd(desc, dy, topk_w, w1, w2, wprep, dx, dw1, dw2, dtopk_w, scratch, stream=None) -> int:
    return lib().moe_bwd(ctypes.byref(desc), _p(dy), _p(topk_w), _p(w1), _p(w2), _p(wprep),
                         _p(dx), _p(dw1), _p(dw2), _p(dtopk_w), _p(scratch), _nbytes(scratch),
                         _stream(stream))


def moe_check(desc, scratch, stream=None) -> int:
    return lib().moe_check(ctypes.byref(desc), _p(scratch), _nbytes(scratch), _stream(stream))


def moe_profile_enable(on: bool) -> int:
    return lib().moe_profile_enable(1 if on else 0)


def moe_profile_collect() -> dict:
    """{kernel name: (total ms, launches)} accumulated since the last reset."""
    L = lib()
    n = L.moe_profile_collect()
    if n < 0:
        raise MoeError(n, "moe_profile_collect")
    out = {}
    for i in range(n):
        name, ms, cnt = ctypes.c_char_p(), ctypes.c_double(), _i64()
        L.moe_profile_get(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(cnt))
        out[name.value.decode()] = (ms.value, cnt.value)
    return out


def moe_profile_reset() -> int:
    return lib().moe_profile_reset()


def check(code: int, what: str = "moe") -> None:
    """Raise MoeError for a non-zero status."""
    if code != MOE_OK:
        raise MoeError(code, what)
