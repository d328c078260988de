"""Pins for the oracle's FP8 codec (CPU only).

The codec is fixed by the OCP 8-bit float formats the pages name (E4M3 and
E5M2 stored as raw bytes: textbook 10.4.5, the guide's kv_cache_dtype table and
its note that FP8 caches are uint8 tensors read with FP8 meaning).  Each check
below compares the oracle with something other than itself: torch's float8
dtypes (an independent library implementation), brute-force enumeration, and
closed-form limits of the formats.
"""
import math

import numpy as np
import pytest
import torch

import oracle

TORCH_DT = {oracle.FMT_E4M3: torch.float8_e4m3fn, oracle.FMT_E5M2: torch.float8_e5m2}
FMTS = [oracle.FMT_E4M3, oracle.FMT_E5M2]


def torch_decode_all(fmt):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(TORCH_DT[fmt]).to(torch.float64).numpy()


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_all_codes_match_torch(fmt):
    ours = oracle.fp8_decode_table(fmt)
    ref = torch_decode_all(fmt)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # signed zero is kept
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3_census_and_limits():
    t = oracle.fp8_decode_table(oracle.FMT_E4M3)
    assert np.isnan(t).sum() == 2 and np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isinf(t).sum() == 0
    assert np.isfinite(t).sum() == 254
    assert t[0x7E] == 448.0 and oracle.fp8_max(oracle.FMT_E4M3) == 448.0
    assert np.nanmax(t) == 448.0 and np.nanmin(t) == -448.0
    pos = t[(t > 0) & np.isfinite(t)]
    assert pos.min() == 2.0 ** -9  # smallest subnormal
    assert t[0x08] == 2.0 ** -6  # smallest normal


def test_e5m2_census_and_limits():
    t = oracle.fp8_decode_table(oracle.FMT_E5M2)
    assert np.isnan(t).sum() == 6
    assert np.isinf(t).sum() == 2 and t[0x7C] == np.inf and t[0xFC] == -np.inf
    assert np.isfinite(t).sum() == 248
    assert t[0x7B] == 57344.0 and oracle.fp8_max(oracle.FMT_E5M2) == 57344.0
    pos = t[(t > 0) & np.isfinite(t)]
    assert pos.min() == 2.0 ** -16
    assert t[0x04] == 2.0 ** -14


@pytest.mark.parametrize("fmt", FMTS)
def test_round_trip_every_finite_code(fmt):
    t = oracle.fp8_decode_table(fmt)
    codes = np.arange(256)
    fin = np.isfinite(t)
    back = oracle.fp8_encode(fmt, t[fin].astype(np.float32))
    assert np.array_equal(back, codes[fin].astype(np.uint8))


@pytest.mark.parametrize("fmt", FMTS)
def test_special_inputs(fmt):
    mx = 0x7E if fmt == oracle.FMT_E4M3 else 0x7B
    x = np.array([np.inf, -np.inf, np.nan, -np.nan, 0.0, -0.0, 1e30, -1e30], np.float32)
    c = oracle.fp8_encode(fmt, x)
    assert c[0] == mx and c[1] == (mx | 0x80)  # +-Inf saturate
    t = oracle.fp8_decode_table(fmt)
    assert np.isnan(t[c[2]]) and np.isnan(t[c[3]])  # NaN stays NaN
    assert c[4] == 0x00 and c[5] == 0x80  # signed zero
    assert c[6] == mx and c[7] == (mx | 0x80)


@pytest.mark.parametrize("fmt", FMTS)
def test_ties_to_even_on_both_grids(fmt):
    """Midpoints between adjacent codes round to the code with an even mantissa,
    both on the subnormal and on the normal grid."""
    t = oracle.fp8_decode_table(fmt)
    pos = np.array(sorted(set(t[(t >= 0) & np.isfinite(t)].tolist())))
    for a, b in zip(pos[:-1], pos[1:]):
        mid = np.float32((a + b) / 2)  # exact: fp8 midpoints are fp32 values
        assert float(mid) == (a + b) / 2
        c = int(oracle.fp8_encode(fmt, np.array([mid]))[0])
        ca = int(oracle.fp8_encode(fmt, np.array([a], np.float32))[0])
        cb = int(oracle.fp8_encode(fmt, np.array([b], np.float32))[0])
        assert c == (ca if ca % 2 == 0 else cb)
        # just off the midpoint rounds to the nearer code
        lo = np.nextafter(mid, np.float32(0))
        hi = np.nextafter(mid, np.float32(np.inf))
        assert oracle.fp8_encode(fmt, np.array([lo]))[0] == ca
        assert oracle.fp8_encode(fmt, np.array([hi]))[0] == cb


@pytest.mark.parametrize("fmt", FMTS)
def test_encoder_all_fp32_patterns_against_torch(fmt):
    """Exhaustive: every one of the 2^32 fp32 bit patterns.  Where torch's cast
    (round-to-nearest-even, non-saturating) gives a finite code the oracle must
    give the same byte; where torch overflows (NaN for E4M3fn, Inf for E5M2) the
    input lies beyond the largest code and the oracle must saturate to it with
    the input's sign; NaN inputs must give a NaN code."""
    mx = 0x7E if fmt == oracle.FMT_E4M3 else 0x7B
    fmax_bits = int(np.float32(oracle.fp8_max(fmt)).view(np.uint32))
    finite_code = np.isfinite(oracle.fp8_decode_table(fmt))
    chunk = 1 << 26
    step = np.arange(chunk, dtype=np.uint32)
    for i in range(1 << 32 >> 26):
        u = step + np.uint32(i * chunk)
        x = u.view(np.float32)
        ours = oracle.fp8_encode(fmt, x)
        ref = torch.from_numpy(x).to(TORCH_DT[fmt]).view(torch.uint8).numpy()
        lo, hi = (i * chunk) & 0x7FFFFFFF, ((i + 1) * chunk - 1) & 0x7FFFFFFF
        sgn = np.uint8(0x80 if i * chunk >= 1 << 31 else 0)
        if hi <= fmax_bits:  # every input in range: identical bytes
            assert np.array_equal(ours, ref), f"chunk {i}"
        elif lo > fmax_bits and hi < 0x7F800000:  # every input finite and beyond max
            assert np.all(ours == (sgn | mx)), f"chunk {i}"
            # torch either rounded down onto max or overflowed to a non-finite code
            assert np.all((ref == ours) | ~finite_code[ref]), f"chunk {i}"
        else:  # mixed chunk: classify element by element
            ax = u & np.uint32(0x7FFFFFFF)
            isnan = ax > 0x7F800000
            over = (ax > fmax_bits) & ~isnan  # includes +-Inf
            expected = np.where(over, sgn | np.uint8(mx), ref)
            assert np.all((ours == expected) | isnan), f"chunk {i}"
            assert not finite_code[ours[isnan]].any(), f"chunk {i}: NaN must stay NaN"
            tf = finite_code[ref]
            assert np.all(tf | over | isnan), f"chunk {i}: torch overflowed in range"
            assert np.all(~(over & tf) | (ref == ours)), f"chunk {i}"
