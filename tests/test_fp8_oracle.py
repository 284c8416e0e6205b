"""Pins of the oracle's FP8 encodings: OCP e4m3 against torch.float8_e4m3fn and
closed forms, the blockwise and e8m0 scale rules by closed form."""
import numpy as np
import pytest
import torch

from oracle import fp8_oracle as f8


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = f8.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_decode_closed_form_points():
    assert f8.e4m3_decode(0x7E) == 448.0 and f8.e4m3_decode(0xFE) == -448.0
    assert f8.e4m3_decode(0x01) == 2.0 ** -9 and f8.e4m3_decode(0x08) == 2.0 ** -6
    assert f8.e4m3_decode(0x38) == 1.0 and f8.e4m3_decode(0x3C) == 1.5


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    np.testing.assert_array_equal(f8.e4m3_encode(f8.e4m3_decode(codes)), codes)


def test_encode_matches_torch_in_range_including_ties():
    vals = f8.e4m3_decode(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(0)
    x = np.concatenate([mids, -mids, rng.uniform(-448, 448, 20000), rng.normal(0, 0.01, 20000),
                        rng.normal(0, 1e-3, 2000)]).astype(np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(f8.e4m3_encode(x), ref)


def test_ties_round_to_even_mantissa():
    # 1 + 1/16 lies halfway between 1.0 (0x38, mantissa 0) and 1.125 (0x39): even -> 0x38
    assert f8.e4m3_encode(np.float32(1.0625)) == 0x38
    # 1.1875 between 1.125 (0x39) and 1.25 (0x3A): even -> 0x3A
    assert f8.e4m3_encode(np.float32(1.1875)) == 0x3A


def test_saturation():
    np.testing.assert_array_equal(f8.e4m3_encode(np.array([449.0, 500.0, 1e6, -1e9])),
                                  [0x7E, 0x7E, 0x7E, 0xFE])


def test_e8m0_rule_closed_forms():
    a = np.array([448.0, 448.0001, 896.0, 896.001, 224.0, 1.0, 0.0, 1e-40, 1e30])
    np.testing.assert_array_equal(f8.e8m0_exponent(a), [0, 1, 1, 2, -1, -8, 0, -127, 91])


def test_block_scale_rule():
    np.testing.assert_array_equal(f8.block_scale(np.array([448.0, 0.0, 1.0], np.float32)),
                                  np.array([1.0, 1.0, np.float32(1.0) / np.float32(448.0)], np.float32))


@pytest.mark.parametrize("mx,group", [(False, 128), (True, 32)])
def test_quant_rows_error_bound(mx, group):
    rng = np.random.default_rng(1)
    a = (rng.standard_normal((16, 256)) * np.exp(rng.normal(0, 2, (16, 1)))).astype(np.float32)
    codes, sc = f8.quant_rows(a, group, mx)
    deq = f8.dequant_rows(codes, sc, group, mx)
    amax = np.abs(a.reshape(16, -1, group)).max(axis=2)
    q = np.abs(a.reshape(16, -1, group)) / (np.exp2(sc) if mx else sc)[:, :, None]
    assert q.max() <= 448.0 * (1 + 2 ** -20)
    normal = (q >= 2.0 ** -6).reshape(16, 256)
    rel = np.abs(deq - a)[normal] / np.abs(a)[normal]
    assert rel.max() <= 2.0 ** -4 * (1 + 1e-6)
    # the block maximum is represented to within the same bound
    assert np.all(np.abs(np.abs(deq).reshape(16, -1, group).max(axis=2) - amax) <= amax * 2 ** -4)


def test_quant_tokens_segments_and_padding():
    rng = np.random.default_rng(2)
    offsets = np.array([0, 5, 5, 140])  # experts of 5, 0 and 135 tokens
    a = rng.standard_normal((140, 32)).astype(np.float32)
    codes, sc, poff = f8.quant_tokens(a, offsets, 128, False)
    assert list(poff) == [0, 128, 128, 384]
    assert codes.shape == (32, 384) and sc.shape == (3, 32)
    assert np.all(codes[:, 5:128] == 0) and np.all(codes[:, 128 + 135:] == 0)
    # the first expert's tokens form their own block: scale from those 5 tokens only
    np.testing.assert_array_equal(sc[0], f8.block_scale(np.abs(a[:5]).max(axis=0)))
    deq = f8.e4m3_decode(codes[:, 128:256]) * sc[1][:, None]
    np.testing.assert_allclose(deq.T, a[5:133], rtol=2 ** -4, atol=1e-6)


def test_weight_blocks():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w[:128, :128] *= 100
    codes, s = f8.quant_weight_blocks(w)
    assert s.shape == (2, 3)
    np.testing.assert_array_equal(s, f8.block_scale(np.abs(w.reshape(2, 128, 3, 128)).max(axis=(1, 3))))
    np.testing.assert_allclose(f8.dequant_weight_blocks(codes, s), w, rtol=2 ** -4, atol=2 ** -9 * s.max())
