"""FP8 encodings used by the layer's blockwise-FP8 and MXFP8 modes.  TEST INFRASTRUCTURE ONLY.

The pages list BF16, MXFP8 and blockwise FP8 as the supported types and an
fp8_bwd mode (BF16 forward, FP8 backward) (Prime Mega MoE news item, "How does
the fused kernel work?"; precisions in "How do developers use it?").  They do
not define the encodings; this module writes them out from the public format
definitions, in float64 / exact arithmetic, slowly and plainly:

* e4m3 (OCP 8-bit float "E4M3FN"): 1 sign, 4 exponent bits (bias 7), 3 mantissa
  bits; exponent field 0 is subnormal (m/8 * 2^-6); code S.1111.111 is NaN;
  the largest finite magnitude is 448.  Encoding rounds to the nearest finite
  value, ties to the code with an even mantissa, and saturates to +-448.
* Blockwise FP8: a block of values shares one fp32 scale s = amax / 448 (fp32
  division; s = 1 when amax = 0); each value is encoded as e4m3(x / s) with an
  fp32 division, and decodes as e4m3 value * s.
* MX (e8m0 scale per 32 values): the scale is 2^X with X the smallest integer in
  [-127, 127] such that amax <= 448 * 2^X (X = 0 when amax = 0), so no value
  saturates; values encode as e4m3(x * 2^-X).  The e8m0 byte is X + 127.

Parity pins: every code against torch.float8_e4m3fn, ties and saturation by
closed form, the scale rules by closed form.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(code) -> np.ndarray:
    """float64 value of e4m3 codes (NaN for S.1111.111)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


# the 127 non-negative finite values, in code order 0x00..0x7E (increasing)
_POS_CODES = np.arange(0x7F)
_POS_VALUES = e4m3_decode(_POS_CODES)


def e4m3_encode(x) -> np.ndarray:
    """e4m3 codes of finite values: nearest finite value, ties to even mantissa,
    magnitudes above 448 saturate to 448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")       # first value >= a
    hi = np.clip(hi, 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(a == _POS_VALUES[hi], _POS_CODES[hi], code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def block_scale(amax) -> np.ndarray:
    """fp32 scale amax/448 (fp32 division), 1 where amax == 0."""
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def e8m0_exponent(amax) -> np.ndarray:
    """Smallest integer X in [-127, 127] with amax <= 448 * 2^X (0 when amax == 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    # X starts at -127 and steps up once for every candidate X' < 127 whose
    # 448 * 2^X' is still below amax: the first X with amax <= 448 * 2^X
    X = np.full(amax.shape, -127, dtype=np.int64)
    for cand in range(-127, 127):
        X += amax > E4M3_MAX * 2.0 ** cand
    return np.where(amax == 0, 0, X)


def quant_block(x, scale) -> np.ndarray:
    """e4m3 codes of x / scale (fp32 division), scale broadcast to x."""
    q = (np.asarray(x, np.float32) / np.asarray(scale, np.float32)).astype(np.float32)
    return e4m3_encode(q)


def quant_rows(a, group: int, mx: bool):
    """Quantise [R, C] along C in groups of `group` (C % group == 0).

    Returns (codes [R, C] uint8, scales [R, C/group]): fp32 block scales, or
    e8m0 exponents X (int) when mx.
    """
    a = np.asarray(a, np.float32)
    R, C = a.shape
    g = a.reshape(R, C // group, group)
    amax = np.abs(g).max(axis=2)
    if mx:
        X = e8m0_exponent(amax)
        q = (g.astype(np.float64) * np.exp2(-X.astype(np.float64))[:, :, None]).astype(np.float32)
        return e4m3_encode(q).reshape(R, C), X
    s = block_scale(amax)
    return quant_block(g, s[:, :, None]).reshape(R, C), s


def dequant_rows(codes, scales, group: int, mx: bool) -> np.ndarray:
    R, C = codes.shape
    v = e4m3_decode(codes).reshape(R, C // group, group)
    f = np.exp2(np.asarray(scales, np.float64)) if mx else np.asarray(scales, np.float64)
    return (v * f[:, :, None]).reshape(R, C)


def quant_tokens(a, offsets, group: int, mx: bool):
    """Quantise token-major rows [N, C] along the token axis, in groups of `group`
    consecutive tokens within each expert's segment [offsets[e], offsets[e+1]),
    starting at the segment's first token; a segment's last group is padded with
    zeros.  Returns (codes [C, Npad], scales [Npad/group, C] for fp32 or
    [C, Npad/group] exponents for mx, column offsets [E+1] of each segment in the
    padded token axis).  Segments are padded to a multiple of 128 tokens."""
    a = np.asarray(a, np.float32)
    C = a.shape[1]
    E = len(offsets) - 1
    pad = [int(-(-(offsets[e + 1] - offsets[e]) // 128) * 128) for e in range(E)]
    poff = np.concatenate([[0], np.cumsum(pad)]).astype(np.int64)
    Npad = int(poff[-1])
    t = np.zeros((C, Npad), np.float32)
    for e in range(E):
        n = offsets[e + 1] - offsets[e]
        t[:, poff[e]:poff[e] + n] = a[offsets[e]:offsets[e + 1]].T
    codes, sc = quant_rows(t, group, mx)
    return codes, (sc if mx else sc.T.copy()), poff


def quant_weight_blocks(w):
    """Blockwise-FP8 weight [R, C] in 128 x 128 blocks: (codes [R, C], fp32 scales [R/128, C/128])."""
    w = np.asarray(w, np.float32)
    R, C = w.shape
    b = w.reshape(R // 128, 128, C // 128, 128)
    amax = np.abs(b).max(axis=(1, 3))
    s = block_scale(amax)
    codes = quant_block(b, s[:, None, :, None]).reshape(R, C)
    return codes, s


def dequant_weight_blocks(codes, scales) -> np.ndarray:
    R, C = codes.shape
    v = e4m3_decode(codes).reshape(R // 128, 128, C // 128, 128)
    return (v * np.asarray(scales, np.float64)[:, None, :, None]).reshape(R, C)
