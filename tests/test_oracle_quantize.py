"""Pins for the oracle's quantize step, scale calibration and paged write (CPU only).

Quantize follows textbook 10.4.5 (write with cast_fp8(K / sK)) and, for the
integer grid it replaces, 10.4.2 (Kq = clip(round(K / sK))).  The guide's
section on scale sources fixes the default: with scale 1.0 the operation is a
plain cast.  Independent checks: torch's float8 casts, numpy's IEEE fp32
division and reductions, and the exhaustive bf16 input domain.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TORCH_DT = {oracle.FMT_E4M3: torch.float8_e4m3fn, oracle.FMT_E5M2: torch.float8_e5m2}
FMTS = [oracle.FMT_E4M3, oracle.FMT_E5M2]
ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def torch_cast_codes(fmt, x_f32):
    return torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(
        TORCH_DT[fmt]).view(torch.uint8).numpy()


def check_against_torch(fmt, codes, q_f32):
    """codes must equal torch's cast of q wherever torch stays finite, and be
    +-max where |q| is beyond the format (torch overflows there)."""
    dec = oracle.fp8_decode_table(fmt)
    ref = torch_cast_codes(fmt, q_f32)
    nan = np.isnan(q_f32)
    fin = np.isfinite(dec[ref]) & ~nan
    assert np.array_equal(codes[fin], ref[fin])
    over = ~np.isfinite(dec[ref]) & ~nan
    mx = 0x7E if fmt == oracle.FMT_E4M3 else 0x7B
    sign = (np.signbit(q_f32[over]).astype(np.uint8) << 7)
    assert np.array_equal(codes[over], sign | mx)
    assert np.all(np.isnan(dec[codes[nan]]))


@pytest.mark.parametrize("fmt", FMTS)
def test_scale_one_is_a_plain_cast(fmt):
    """Guide, scale sources: with every scale 1.0 the quantizer is a plain cast
    of the bf16 value; checked over all 65536 bf16 bit patterns."""
    x = W.bf16_bits_to_f32(ALL_BF16)
    codes = oracle.quantize(fmt, ALL_BF16, 1.0)
    check_against_torch(fmt, codes, x)
    # direct bf16 -> fp8 cast in torch agrees too (finite, in-range inputs)
    tb = torch.from_numpy(ALL_BF16.view(np.int16)).view(torch.bfloat16)
    direct = tb.to(TORCH_DT[fmt]).view(torch.uint8).numpy()
    dec = oracle.fp8_decode_table(fmt)
    ok = np.isfinite(dec[direct]) & np.isfinite(x)
    assert np.array_equal(codes[ok], direct[ok])


def test_quotient_is_correctly_rounded_fp32_division():
    """The fp64-then-fp32 quotient equals IEEE fp32 division (numpy)."""
    g = W.rng(7)
    a = W.bf16_bits_to_f32(g.integers(0, 1 << 16, 200000, dtype=np.uint32).astype(np.uint16))
    s = np.exp(g.uniform(-12, 12, 200000)).astype(np.float32)
    ok = np.isfinite(a)
    a, s = a[ok], s[ok]
    # numpy float32 divide: correctly rounded, overflowing to +-Inf where the
    # quotient passes the fp32 range (the oracle must do the same)
    with np.errstate(over="ignore"):
        ref = (a / s).astype(np.float32)
    ours = np.array([oracle.quotient(float(x), float(y)) for x, y in zip(a[:20000], s[:20000])],
                    np.float32)
    assert np.array_equal(ours.view(np.uint32), ref[:20000].view(np.uint32))


SCALES = [1.0, 0.5, 2.0 ** -7, 3.0, 0.0123, 7.77e-3, 123.456, 1.0 / 448, 10.0 / 448,
          4.6875e-2, 1e-30, 3.3e20]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("s", SCALES)
def test_quantize_every_bf16_against_torch(fmt, s):
    """For each scale, all 65280 finite bf16 inputs: code == cast(fl32(x / s))
    with the fp32 division done by numpy (IEEE) and the cast by torch."""
    s = np.float32(s)
    x = W.bf16_bits_to_f32(ALL_BF16)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        q = (x / s).astype(np.float32)
    codes = oracle.quantize(fmt, ALL_BF16, float(s))
    check_against_torch(fmt, codes, q)


def test_int8_grid_reference_relation():
    """Textbook 10.4.5 contrasts FP8 with INT8's round(K/s) grid: E4M3 codes of
    small integers are exact (every integer up to 16 is representable), so on
    those inputs the FP8 code decodes to round(x/s) exactly like the INT8 grid."""
    for fmt in FMTS:
        vals = np.arange(-16, 17, dtype=np.float32)
        bits = W.f32_to_bf16_bits(vals)
        codes = oracle.quantize(fmt, bits, 1.0)
        back = oracle.fp8_decode_table(fmt)[codes]
        lim = 16 if fmt == oracle.FMT_E4M3 else 8
        m = np.abs(vals) <= lim
        assert np.array_equal(back[m], vals[m])


# ----------------------------------------------------------------- calibration


@pytest.mark.parametrize("fmt", FMTS)
def test_calibrate_per_tensor_and_per_head(fmt):
    g = W.rng(11)
    mult = W.log_uniform(g, 6, 0.5, 20.0)
    x = W.normal_bf16(g, (333, 6, 64), 1, mult)
    xf = W.bf16_bits_to_f32(x)
    amax_t, sc_t = oracle.calibrate(x, fmt, oracle.GRAN_TENSOR)
    amax_h, sc_h = oracle.calibrate(x, fmt, oracle.GRAN_HEAD)
    fmax = np.float32(oracle.fp8_max(fmt))
    assert amax_t.shape == (1,) and amax_h.shape == (6,)  # guide: [1] and [num_kv_heads]
    assert amax_t[0] == np.abs(xf).max()
    assert np.array_equal(amax_h, np.abs(xf).max(axis=(0, 2)))
    assert sc_t[0] == np.float32(amax_t[0] / fmax)  # numpy fp32 divide, IEEE
    assert np.array_equal(sc_h, (amax_h / fmax).astype(np.float32))
    # the largest element of each head maps onto (or saturates to) the top code
    for h in range(6):
        row = x[:, h, :].reshape(-1)
        i = np.argmax(np.abs(W.bf16_bits_to_f32(row)))
        c = oracle.quantize(fmt, row[i:i + 1], float(sc_h[h]))[0] & 0x7F
        assert c == (0x7E if fmt == oracle.FMT_E4M3 else 0x7B)


def test_calibrate_degenerate_sets():
    z = np.zeros((5, 2, 8), np.uint16)  # all +0
    amax, sc = oracle.calibrate(z, oracle.FMT_E4M3, oracle.GRAN_HEAD)
    assert np.all(amax == 0) and np.all(sc == 1.0)  # amax = 0 -> scale 1.0
    z[0, 1, 3] = 0x7FC0  # a NaN in head 1 only
    amax, sc = oracle.calibrate(z, oracle.FMT_E4M3, oracle.GRAN_HEAD)
    assert amax[0] == 0 and np.isnan(amax[1]) and sc[1] == 1.0
    z[0, 1, 3] = 0x7F80  # +Inf
    amax, sc = oracle.calibrate(z, oracle.FMT_E4M3, oracle.GRAN_TENSOR)
    assert np.isinf(amax[0]) and sc[0] == 1.0
    e = np.zeros((0, 3, 8), np.uint16)  # no tokens at all
    amax, sc = oracle.calibrate(e, oracle.FMT_E5M2, oracle.GRAN_HEAD)
    assert np.all(amax == 0) and np.all(sc == 1.0)


def test_scale_shapes_golden():
    gold = json.load(open(os.path.join(GOLDEN, "scale_shapes.json")))
    g = W.rng(3)
    q = W.normal_bf16(g, (4, 32, 16))
    kv = W.normal_bf16(g, (4, 8, 16))
    assert gold["per_tensor"]["k_scale"] == "[1]"
    assert oracle.calibrate(kv, 0, oracle.GRAN_TENSOR)[1].shape == (1,)
    assert gold["per_head"]["q_scale"] == "[num_heads]"
    assert oracle.calibrate(q, 0, oracle.GRAN_HEAD)[1].shape == (32,)
    assert gold["per_head"]["k_scale"] == "[num_kv_heads]"
    assert oracle.calibrate(kv, 0, oracle.GRAN_HEAD)[1].shape == (8,)
    assert gold["default_scale_without_calibration"] == 1.0


# ----------------------------------------------------------------- paged write


@pytest.mark.parametrize("fmt,gran", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_cache_write_places_every_code(fmt, gran):
    g = W.rng(5)
    Hkv, dh, bs = 3, 32, 16
    paging = W.make_paging(g, [37, 16, 1, 50], bs)
    kv = W.make_kv(g, paging, Hkv, dh, head_range=(0.5, 20.0))
    ks = np.array([0.01, 0.02, 0.03], np.float32)[: (Hkv if gran else 1)]
    vs = np.array([0.04, 0.05, 0.06], np.float32)[: (Hkv if gran else 1)]
    sm = kv.slot_mapping.copy()
    sm[5] = -1  # a padding token: skipped
    kc5 = np.full(oracle.k_cache_shape(paging.num_blocks, Hkv, bs, dh), 0xA5, np.uint8)
    vc = np.full((paging.num_blocks, Hkv, dh, bs), 0xA5, np.uint8)  # channel-major V tiles
    oracle.cache_write(kv.k, kv.v, sm, kc5, vc, ks, vs, fmt, gran)
    # K tiles hold 16-channel chunks, token-major inside a chunk: byte
    # (((blk * Hkv + h) * dh/16 + d/16) * bs + off) * 16 + d % 16
    flat = kc5.reshape(-1)
    idx = ((((np.arange(paging.num_blocks)[:, None, None, None] * Hkv
              + np.arange(Hkv)[None, :, None, None]) * (dh // 16)
             + np.arange(dh)[None, None, None, :] // 16) * bs
            + np.arange(bs)[None, None, :, None]) * 16 + np.arange(dh)[None, None, None, :] % 16)
    kc = flat[idx]  # [num_blocks][Hkv][bs][dh], gathered by the layout formula
    assert np.array_equal(kc, oracle.k_token_view(kc5))
    touched = np.zeros(kc.shape[:3], bool)
    for t in range(len(sm)):
        if sm[t] < 0:
            continue
        blk, off = sm[t] // bs, sm[t] % bs
        for h in range(Hkv):
            s_k = ks[h if gran else 0]
            s_v = vs[h if gran else 0]
            xk = (W.bf16_bits_to_f32(kv.k[t, h]) / s_k).astype(np.float32)
            xv = (W.bf16_bits_to_f32(kv.v[t, h]) / s_v).astype(np.float32)
            check_against_torch(fmt, kc[blk, h, off], xk)
            check_against_torch(fmt, vc[blk, h, :, off], xv)
            touched[blk, h, off] = True
    assert np.all(kc[~touched] == 0xA5)
    assert np.all(vc.transpose(0, 1, 3, 2)[~touched] == 0xA5)
    # the skipped token's slot was left alone
    blk, off = kv.slot_mapping[5] // bs, kv.slot_mapping[5] % bs
    assert np.all(kc[blk, :, off] == 0xA5) and np.all(vc[blk, :, :, off] == 0xA5)
