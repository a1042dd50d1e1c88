"""Pins for the oracle's binary16 conversions against numpy's float16
(an independent IEEE 754 implementation): every fp16 pattern one way, and a
stratified set of fp32 patterns that covers every rounding case the other way."""

import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _same_bits_or_both_nan_f32(a, b):
    an, bn = np.isnan(a), np.isnan(b)
    assert np.array_equal(an, bn)
    assert np.array_equal(a.view(np.uint32)[~an], b.view(np.uint32)[~bn])


def _same_bits_or_both_nan_f16(a, b):
    a = a.view(np.uint16)
    b = b.view(np.uint16)
    an = ((a & 0x7C00) == 0x7C00) & ((a & 0x3FF) != 0)
    bn = ((b & 0x7C00) == 0x7C00) & ((b & 0x3FF) != 0)
    assert np.array_equal(an, bn)
    assert np.array_equal(a[~an], b[~bn])


def test_half_to_float_all_patterns(oracle_lib):
    h = np.arange(1 << 16, dtype=np.uint16)
    got = oracle_lib.half_to_float(h)
    want = h.view(np.float16).astype(np.float32)
    _same_bits_or_both_nan_f32(got, want)


def _stratified_fp32_patterns():
    """All fp32 exponents that can land in or near the fp16 range, both signs,
    every 10-bit high mantissa, and low-mantissa patterns around every
    possible rounding position (the kept/discarded split moves with the
    exponent in the subnormal range)."""
    lows = {0, 1, 2, 3}
    for shift in range(1, 24):
        half = 1 << (shift - 1)
        for d in (-1, 0, 1):
            val = half + d
            if 0 <= val < (1 << 23):
                lows.add(val)
                lows.add((val | (1 << shift)) & ((1 << 23) - 1))   # odd kept bit
        lows.add((1 << shift) - 1)
    lows = np.array(sorted(lows), dtype=np.uint32)
    exps = np.arange(90, 150, dtype=np.uint32)          # 2^-37 .. 2^22
    highs = np.arange(0, 1 << 23, 1 << 13, dtype=np.uint32)  # top 10 mantissa bits
    mant = (highs[:, None] | (lows[None, :] & ((1 << 13) - 1))).reshape(-1)
    # the subnormal cases discard more than 13 bits: also vary bits 13..22
    mant2 = (lows[None, :] | highs[:, None]).reshape(-1) & ((1 << 23) - 1)
    mant = np.unique(np.concatenate([mant, mant2]))
    bits = (exps[:, None] << 23 | mant[None, :]).reshape(-1)
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    return bits.view(np.float32)


def test_float_to_half_stratified(oracle_lib):
    x = _stratified_fp32_patterns()
    assert x.size > 1_000_000
    got = oracle_lib.float_to_half(x)
    want = x.astype(np.float16)
    _same_bits_or_both_nan_f16(got, want)


def test_float_to_half_random_bits(oracle_lib):
    rng = np.random.default_rng(12345)
    x = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32).view(np.float32)
    got = oracle_lib.float_to_half(x)
    want = x.astype(np.float16)
    _same_bits_or_both_nan_f16(got, want)


@pytest.mark.slow
def test_float_to_half_exhaustive(oracle_lib):
    """Every one of the 2^32 fp32 bit patterns, in chunks over the host's
    threads (the oracle's C conversion and numpy's cast both release the
    GIL): equal to numpy's float16 bit for bit, NaN for NaN."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    chunk = 1 << 24

    def check(c):
        bits = np.arange(c * chunk, (c + 1) * chunk, dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        got = oracle_lib.float_to_half(x)
        with np.errstate(all="ignore"):
            want = x.astype(np.float16).view(np.uint16)
        nan_x = np.isnan(x)
        got_nan = ((got & 0x7C00) == 0x7C00) & ((got & 0x3FF) != 0)
        want_nan = ((want & 0x7C00) == 0x7C00) & ((want & 0x3FF) != 0)
        ok = (np.array_equal(got_nan, nan_x) and np.array_equal(want_nan, nan_x)
              and np.array_equal(got[~nan_x], want[~nan_x]))
        return c, ok

    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as pool:
        bad = [c for c, ok in pool.map(check, range((1 << 32) // chunk)) if not ok]
    assert not bad, f"chunks with a difference: {bad[:8]}"


def test_float_to_half_special_values(oracle_lib):
    x = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 65504.0, 65519.996, 65520.0,
                  -65520.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -14,
                  2.0 ** -14 * (1 - 2 ** -11), 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11,
                  np.finfo(np.float32).max, np.finfo(np.float32).tiny, 1e-45],
                 dtype=np.float32)
    got = oracle_lib.float_to_half(x)
    want = x.astype(np.float16)
    _same_bits_or_both_nan_f16(got, want)
    # ties to even at the fp16 overflow edge and the subnormal edge
    assert got[7] == 0x7C00 and got[8] == 0xFC00 and got[6] == 0x7BFF
    assert got[10] == 0x0000 and got[11] == 0x0001 and got[9] == 0x0001
    assert got[14] == 0x3C00 and got[15] == 0x3C02   # 1+2^-11 -> 1.0, 1+3*2^-11 -> up


def test_round_trip_identity(oracle_lib):
    h = np.arange(1 << 16, dtype=np.uint16)
    finite = (h & 0x7C00) != 0x7C00
    back = oracle_lib.float_to_half(oracle_lib.half_to_float(h))
    assert np.array_equal(back[finite], h[finite])
