"""Pins of the FP8 oracle (no GPU): the E4M3 code table and rounding against
torch's float8_e4m3fn conversion and hand-worked values, the brute-force and
vectorised encoders against each other, the row exponent's minimality, and
the stored values' error bound and bf16 exactness."""
import numpy as np
import pytest
import torch

from oracle import fp8


def test_decode_table_hand_worked_values():
    d = fp8.DECODE
    assert d[0x00] == 0.0 and np.signbit(d[0x80]) and d[0x80] == 0.0
    assert d[0x01] == 2.0 ** -9 and d[0x07] == 7 * 2.0 ** -9          # subnormals
    assert d[0x08] == 2.0 ** -6                                        # smallest normal
    assert d[0x38] == 1.0 and d[0x3C] == 1.5 and d[0xB8] == -1.0
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.sum(~np.isnan(d)) == 254
    assert np.all(np.diff(d[:0x7F]) > 0)                                # codes 0..0x7e ascend


def test_decode_matches_torch_float8():
    t = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(np.isnan(t), np.isnan(fp8.DECODE))
    np.testing.assert_array_equal(np.nan_to_num(t), np.nan_to_num(fp8.DECODE))


def test_encode_matches_torch_float8_and_brute_force():
    rng = np.random.default_rng(1)
    y = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 0.01, 5000), rng.normal(0, 2.0 ** -8, 2000),
                        [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -12]])
    y = y.astype(np.float32).astype(np.float64)          # the kernels encode float32 values
    ref = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(fp8.e4m3_encode_array(y), ref)
    np.testing.assert_array_equal(np.array([fp8.e4m3_encode(v) for v in y[::9]], np.uint8), ref[::9])


def test_encode_round_trip_and_ties_to_even():
    finite = [c for c in range(256) if not np.isnan(fp8.DECODE[c])]
    assert all(fp8.e4m3_encode(fp8.DECODE[c]) == c for c in finite)
    assert fp8.e4m3_encode(1.0625) == 0x38      # between 1.0 (0x38) and 1.125 (0x39): even code
    assert fp8.e4m3_encode(1.1875) == 0x3A      # between 1.125 and 1.25 (0x3a)
    assert fp8.e4m3_encode(2.0 ** -10) == 0x00  # half the smallest subnormal: to zero (even)
    assert fp8.e4m3_encode(3 * 2.0 ** -10) == 0x02
    assert fp8.e4m3_encode(-(2.0 ** -6 + 2.0 ** -10)) == 0x88


@pytest.mark.parametrize("amax", [1e-30, 2.0 ** -20, 0.3, 1.0, 3.5, 448.0, 449.0, 896.0, 1e6, 7.9e-3, 3.3e38])
def test_row_exponent_is_the_smallest_that_fits(amax):
    e = fp8.row_exponent(amax)
    assert amax * 2.0 ** -e <= 448.0 < amax * 2.0 ** -(e - 1)
    assert fp8.row_exponent(0.0) == 0


def test_row_exponent_lower_bound():
    # rows far below the E4M3 range keep the smallest normal float32 scale
    assert fp8.row_exponent(1e-40) == -126 and fp8.row_exponent(2.0 ** -140) == -126
    assert fp8.row_exponent(448.0 * 2.0 ** -126) == -126
    assert fp8.row_exponent(449.0 * 2.0 ** -126) == -125


def test_quantized_rows_error_bound_and_bf16_exactness():
    rng = np.random.default_rng(2)
    X = np.round(rng.normal(size=(300, 64)) * 32) / 32 * rng.uniform(0.01, 40, (300, 1))
    X[7] = 0.0
    codes, sb = fp8.quantize_rows(X)
    Xh = fp8.dequantize_rows(codes, sb)
    e = sb.astype(np.int64) - 127
    assert e[7] == 0 and np.all(codes[7] & 0x7F == 0)
    # half a unit in the last place: 2^-4 relative for normals, 2^-10 * 2^e absolute below 2^-6 * 2^e
    bound = np.maximum(np.abs(X) * 2.0 ** -4, 2.0 ** (e[:, None] - 10))
    assert np.all(np.abs(Xh - X) <= bound)
    bf = torch.from_numpy(Xh.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(bf, Xh)                          # stored values are exact in bf16
    assert np.all(np.abs(X).max(axis=1) * 2.0 ** -e <= 448.0)
