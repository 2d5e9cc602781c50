"""Pins for oracle.fp8: torch's float8_e4m3fn (a library routine) and
constants of the OCP E4M3FN format."""

import numpy as np
import torch

from oracle import fp8


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_table_matches_torch():
    ours = fp8.decode_table()
    ref = _torch_decode_all()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros kept
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_format_constants():
    t = fp8.decode_table()
    assert t[0x7E] == 448.0                      # largest finite
    assert t[0x01] == 2.0 ** -9                  # smallest subnormal
    assert t[0x08] == 2.0 ** -6                  # smallest normal
    assert t[0x38] == 1.0                        # exponent bias 7
    assert t[0x07] == 7 * 2.0 ** -9              # largest subnormal
    assert np.all(np.diff(t[:0x7F]) > 0)         # monotone in the code


def _torch_round(y32):
    y = torch.from_numpy(np.clip(y32, -448, 448).astype(np.float32))
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _edge_values():
    t = fp8.decode_table()[:0x7F]
    mids = (t[:-1] + t[1:]) / 2
    vals = np.concatenate([t, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                           [0.0, 2.0 ** -10, 2.0 ** -11, 447.9, 448.0, 449.0, 464.0,
                            479.9, 480.0, 1e4, 3e38]])
    vals = vals.astype(np.float32)
    return np.concatenate([vals, -vals])


def test_round_matches_torch_on_edges():
    y = _edge_values()
    assert np.array_equal(fp8.round_to_e4m3(y), _torch_round(y))


def test_round_matches_torch_random():
    rng = np.random.default_rng(7)
    y = np.concatenate([
        rng.standard_normal(1_000_000).astype(np.float32) * 100,
        rng.standard_normal(1_000_000).astype(np.float32) * 0.01,
        (rng.uniform(-500, 500, 200_000)).astype(np.float32),
    ])
    assert np.array_equal(fp8.round_to_e4m3(y), _torch_round(y))


def test_saturation_nan_and_signed_zero():
    codes = fp8.round_to_e4m3(np.array([1e30, -1e30, np.nan, -0.0, 0.0, -1e-30],
                                        dtype=np.float32))
    assert list(codes) == [0x7E, 0xFE, 0x7F, 0x80, 0x00, 0x80]


def test_ties_go_to_even():
    # 1.0 (0x38) and 1.125 (0x39): midpoint 1.0625 -> 0x38 (even)
    # 1.125 (0x39) and 1.25 (0x3A): midpoint 1.1875 -> 0x3A (even)
    assert list(fp8.round_to_e4m3(np.array([1.0625, 1.1875], np.float32))) == [0x38, 0x3A]


def test_quantize_divides_in_fp32():
    x = np.array([1.0, 3.0, -7.5], dtype=np.float32)
    s = 0.013950892724096775
    y = x / np.float32(s)
    assert np.array_equal(fp8.quantize(x, s), fp8.round_to_e4m3(y))
    # decode(quantize(x)) stays within half an E4M3 step (relative 2^-4)
    xs = np.random.default_rng(1).standard_normal(10000).astype(np.float32)
    sc = float(np.float32(np.abs(xs).max()) / np.float32(448))
    back = fp8.decode(fp8.quantize(xs, sc), sc)
    big = np.abs(xs) > 2 ** -6 * sc
    assert np.all(np.abs(back[big] - xs[big]) <= np.abs(xs[big]) * 2 ** -4 + 1e-12)
