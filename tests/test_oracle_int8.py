"""Pins of the oracle's symmetric INT8 codec (the KV-cache quantization
textbook, section 10.4.2: Kq = clip(round(K / sK), -127, 127), read back as
K_hat = sK * Kq), against closed forms and numpy's own rounding."""
import numpy as np
import pytest

import oracle
import workloads as W

I8 = oracle.FMT_INT8
ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def numpy_int8(q_f32):
    """clip(rint(q), -127, 127) with numpy (rint rounds half to even); NaN -> 0."""
    q = np.asarray(q_f32, np.float32)
    with np.errstate(invalid="ignore"):
        r = np.clip(np.rint(q), -127, 127)
    r = np.where(np.isnan(q), 0, r)
    return r.astype(np.int8).view(np.uint8)


def test_decode_table_is_twos_complement():
    t = oracle.fp8_decode_table(I8)
    assert np.array_equal(t, np.arange(256, dtype=np.uint8).view(np.int8).astype(np.float64))
    assert oracle.fp8_max(I8) == 127.0


def test_ties_limits_and_specials():
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5, 127.49, 127.5, -127.5,
                  128.0, 3e38, np.inf, -np.inf, np.nan, -0.0, 1e-30], np.float32)
    want = np.array([0, 2, 2, 0, -2, -2, 126, -126, 127, 127, -127, 127, 127, 127, -127, 0, 0, 0],
                    np.int8).view(np.uint8)
    assert np.array_equal(oracle.fp8_encode(I8, x), want)


@pytest.mark.parametrize("s", [1.0, 0.5, 1.0 / 127, 3.0, 0.0123, 123.456, 2.0 ** -20, 1e20])
def test_quantize_every_bf16_matches_numpy(s):
    """code = clip(rint(fl32(x / s))) for all 65536 bf16 inputs; numpy's fp32
    division is correctly rounded, so this is an independent check of the
    quotient and the rounding together."""
    s = np.float32(s)
    codes = oracle.quantize(I8, ALL_BF16, s)
    x = W.bf16_bits_to_f32(ALL_BF16)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = (x / s).astype(np.float32)
    assert np.array_equal(codes, numpy_int8(q))


def test_scale_is_amax_over_127():
    g = W.rng(31)
    x = W.normal_bf16(g, (100, 3, 32), 1, np.array([0.5, 4.0, 30.0], np.float32))
    amax, scale = oracle.calibrate(x, I8, oracle.GRAN_HEAD)
    ref = np.abs(W.bf16_bits_to_f32(x)).max(axis=(0, 2))
    assert np.array_equal(amax, ref.astype(np.float32))
    assert np.array_equal(scale, (ref.astype(np.float64) / 127.0).astype(np.float32))
    # the scale maps the largest magnitude onto the clip bound
    codes = oracle.quantize(I8, x[:, 2], scale[2]).view(np.int8)
    assert np.abs(codes).max() == 127


def test_round_trip_error_is_at_most_half_a_step():
    g = W.rng(32)
    x = W.normal_bf16(g, (4096,))
    _, s = oracle.calibrate(x.reshape(4096, 1, 1), I8, oracle.GRAN_TENSOR)
    xh = oracle.dequantize(I8, oracle.quantize(I8, x, s[0]), s[0])
    err = np.abs(xh - W.bf16_bits_to_f32(x).astype(np.float64))
    assert err.max() <= 0.5 * float(s[0]) * (1 + 1e-6)
