"""Pins of the oracle's KIVI-style asymmetric 2-bit KV (the KV-cache
quantization textbook, section 10.4.4: K grouped per channel over G tokens,
V per token over groups of channels, a bf16 residual for the newest tokens).
The codec is pinned by values exactly on its grid, by numpy's fp16 rounding for
the stored (s, z), by the error bound of rounding to the grid, and by special
cases; the tile layout by a bijection check; decode by torch's fp64 SDPA."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

G, DH = oracle.KIVI_G, oracle.KIVI_DH


def f16(x):
    return np.float16(np.float32(x))


def f16_bits(x):
    return int(np.array([f16(x)], np.float16).view(np.uint16)[0])


def f16_val(bits):
    return float(np.array([bits], np.uint16).view(np.float16)[0])


def test_layout_is_a_bijection():
    k = {oracle.kivi_k_pos(t, c) for t in range(G) for c in range(DH)}
    v = {oracle.kivi_v_pos(t, c) for t in range(G) for c in range(DH)}
    assert len(k) == G * DH and len(v) == G * DH
    assert k == {(b, i) for b in range(0, 1024) for i in (0, 2, 4, 6)}
    assert v == {(b, i) for b in range(1536, 2560) for i in (0, 2, 4, 6)}


@pytest.mark.parametrize("seed", range(6))
def test_values_on_the_grid_are_exact(seed):
    """x = z + k s with dyadic z, s (exact in bf16 and fp16) and both ends of
    the grid present: s and z come back exactly, codes are k, x_hat = x."""
    g = W.rng(700 + seed)
    for _ in range(50):
        e = int(g.integers(-8, 6))
        s = float(g.choice([1, 3, 5, 7])) * 2.0 ** e
        z = float(g.integers(-20, 20)) * 2.0 ** e
        k = g.integers(0, 4, size=32)
        k[:2] = [0, 3]
        g.shuffle(k)
        x = (z + k * s).astype(np.float32)
        s16, z16, codes = oracle.kivi_group(x)
        assert f16_val(s16) == s and f16_val(z16) == z
        assert np.array_equal(codes, k)
        assert np.array_equal(codes * f16_val(s16) + f16_val(z16), x.astype(np.float64))


def test_scale_and_zero_are_numpy_fp16_roundings():
    g = W.rng(710)
    for _ in range(400):
        x = (g.standard_normal(32) * np.exp(g.uniform(-12, 12))).astype(np.float32)
        x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
        s16, z16, _ = oracle.kivi_group(x)
        rng32 = np.float32(x.max()) - np.float32(x.min())
        s32 = np.float32(rng32 / np.float32(3.0))
        assert s16 == f16_bits(min(s32, np.float32(65504.0)))
        assert z16 == f16_bits(np.clip(x.min(), -65504.0, 65504.0))


def _numpy_kivi_codec(x: np.ndarray):
    """The 2-bit codec of every row of x (float32 [n, 32]) in numpy's own fp32
    and fp16 arithmetic: s = fl16(min(fl32(fl32(max - min) / 3), 65504)),
    z = fl16(clamp(min, +-65504)), code = clip(rint(fl32(fl32(x - z) / s)), 0, 3)
    (0 where s is 0); rows holding an Inf or NaN store s = z = 0 and codes 0."""
    x = x.astype(np.float32)
    bad = ~np.all(np.isfinite(x), axis=1)
    xs = np.where(bad[:, None], np.float32(0), x)
    mn, mx = xs.min(axis=1), xs.max(axis=1)
    with np.errstate(over="ignore"):
        s32 = (mx - mn) / np.float32(3.0)          # fp32 subtract, then fp32 divide
    s16 = np.minimum(s32, np.float32(65504.0)).astype(np.float16)
    z16 = np.clip(mn, np.float32(-65504.0), np.float32(65504.0)).astype(np.float16)
    s16[bad], z16[bad] = 0, 0
    sf, zf = s16.astype(np.float32), z16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        q = (xs - zf[:, None]) / sf[:, None]      # fp32 subtract, then fp32 divide
    codes = np.clip(np.rint(np.nan_to_num(q, nan=0.0, posinf=3.0, neginf=0.0)), 0, 3)
    codes[(sf == 0) | bad] = 0
    return s16.view(np.uint16), z16.view(np.uint16), codes.astype(np.uint8)


def test_codec_matches_a_numpy_fp32_recompute():
    """100,000 seeded sets of 32 bf16 values: normal sets over 24 decades of
    magnitude, sets with outliers, sets whose values sit on the midpoints of
    their own code grid (ties), near-constant sets, sets whose range or minimum
    leaves the fp16 range, and sets holding an Inf or NaN.  The oracle's
    (s, z, codes) equal a recompute in numpy's fp32 / fp16 arithmetic, which
    shares nothing with the oracle's fp64-then-round code."""
    g = W.rng(730)
    n = 100_000
    mag = np.exp(g.uniform(np.log(1e-12), np.log(1e12), n)).astype(np.float32)
    x = (g.standard_normal((n, 32)) * mag[:, None]).astype(np.float32)
    kind = g.integers(0, 8, n)
    # outliers: one value 50x the rest
    o = kind == 1
    x[o, 0] *= 50
    # ties: z + (k + 1/2) s for dyadic z, s, with both ends of the grid present
    t = np.nonzero(kind == 2)[0]
    e = g.integers(-10, 8, t.size)
    sg = (g.choice([1, 3, 5], t.size) * 2.0 ** e).astype(np.float64)
    zg = (g.integers(-40, 40, t.size) * 2.0 ** e).astype(np.float64)
    kk = g.integers(0, 3, (t.size, 32)) + 0.5
    kk[:, 0], kk[:, 1] = -0.5, 3.5  # extend the range so s stays sg and z stays zg - s/2
    x[t] = (zg[:, None] + kk * sg[:, None]).astype(np.float32)
    # near-constant sets
    c = kind == 3
    x[c] = (x[c, :1] * (1 + 1e-3 * g.standard_normal((c.sum(), 32)))).astype(np.float32)
    # range or minimum beyond fp16
    w = kind == 4
    x[w] = (g.standard_normal((w.sum(), 32)) * 1e5).astype(np.float32)
    m = kind == 5
    x[m] = (-1e5 + g.standard_normal((m.sum(), 32))).astype(np.float32)
    # non-finite members
    f = np.nonzero(kind == 6)[0]
    x[f, g.integers(0, 32, f.size)] = g.choice([np.inf, -np.inf, np.nan], f.size)
    x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x)).reshape(n, 32)
    ws, wz, wc = _numpy_kivi_codec(x)
    s16 = np.empty(n, np.uint16)
    z16 = np.empty(n, np.uint16)
    codes = np.empty((n, 32), np.uint8)
    for i in range(n):
        s16[i], z16[i], codes[i] = oracle.kivi_group(x[i])
    assert np.array_equal(s16, ws)
    assert np.array_equal(z16, wz)
    assert np.array_equal(codes, wc)
    # the tie sets really do hit midpoints, so round-half-even decides codes
    assert np.any((wc[t] == 2) & (kk == 1.5))


@pytest.mark.parametrize("scale", [1e-3, 1.0, 30.0, 3000.0])
def test_rounding_error_bound_and_monotone_codes(scale):
    """Every code is in 0..3, codes do not decrease with x, and
    |x - x_hat| <= s/2 + |min - z| + 3 |(max - min)/3 - s| (+ fp32 rounding)."""
    g = W.rng(720)
    for _ in range(300):
        x = (g.standard_normal(32) * scale).astype(np.float32)
        x[g.integers(0, 32)] *= 8  # an outlier
        x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
        s16, z16, codes = oracle.kivi_group(x)
        s, z = f16_val(s16), f16_val(z16)
        assert codes.max() <= 3
        order = np.argsort(x, kind="stable")
        assert np.all(np.diff(codes[order].astype(int)) >= 0)
        xh = codes * s + z
        mn, mx = float(x.min()), float(x.max())
        bound = s / 2 + abs(mn - z) + 3 * abs((mx - mn) / 3 - s) + 1e-6 * (abs(mn) + abs(mx))
        assert np.max(np.abs(xh - x)) <= bound


def test_special_sets():
    c = np.full(32, 1.2345, np.float32)
    s16, z16, codes = oracle.kivi_group(c)  # constant: no range
    assert s16 == 0 and z16 == f16_bits(np.float32(1.2345)) and not codes.any()
    for bad in (np.nan, np.inf, -np.inf):
        x = np.linspace(-1, 1, 32).astype(np.float32)
        x[5] = bad
        assert oracle.kivi_group(x)[:2] == (0, 0) and not oracle.kivi_group(x)[2].any()
    x = np.linspace(-3e5, 3e5, 32).astype(np.float32)  # range/3 above fp16 max, min below -max
    s16, z16, codes = oracle.kivi_group(x)
    assert s16 == 0x7BFF and z16 == 0xFBFF and codes[0] == 0 and codes[-1] == 3
    x = np.float32(1e-4) + np.arange(32, dtype=np.float32) * np.float32(1e-9)
    s16, _, codes = oracle.kivi_group(x)  # (max - min) / 3 < 2^-25 rounds to fp16 zero
    assert s16 == 0 and not codes.any()
    x = np.float32(1e-4) + np.arange(32, dtype=np.float32) * np.float32(1e-8)
    s16, _, codes = oracle.kivi_group(x)  # ... and just above it, to fp16 subnormals
    assert 0 < s16 < 0x0400 and codes[0] == 0 and codes.max() >= 2
    s16, z16, codes = oracle.kivi_group(np.array([2.5, -0.5], np.float32))  # ties to even
    assert f16_val(s16) == 1.0 and f16_val(z16) == -0.5 and list(codes) == [3, 0]
    s16, z16, codes = oracle.kivi_group(np.array([0.0, 3.0, 0.5, 1.5, 2.5], np.float32))
    assert list(codes) == [0, 3, 0, 2, 2]  # 0.5 -> 0, 1.5 -> 2, 2.5 -> 2


def make_groups(seed, n_groups, Hkv):
    g = W.rng(seed)
    k = W.normal_bf16(g, (n_groups * G, Hkv, DH), 1, W.log_uniform(g, Hkv, 0.5, 4.0),
                      g.choice(DH, 4, replace=False), 10.0)
    v = W.normal_bf16(g, (n_groups * G, Hkv, DH), 1, W.log_uniform(g, Hkv, 0.5, 4.0))
    return g, k, v


def test_quantize_matches_the_codec_per_set_and_skips_invalid_blocks():
    g, k, v = make_groups(730, 5, 2)
    nb = 9
    blocks = np.array([3, -1, 0, 8, 99], np.int32)  # -1 and 99 are skipped
    cache = np.full(oracle.kivi_cache_shape(nb, 2), 0x5A, np.uint8)
    oracle.kivi_quantize(k, v, blocks, cache)
    untouched = [b for b in range(nb) if b not in (3, 0, 8)]
    assert np.all(cache[untouched] == 0x5A)
    kf, vf = W.bf16_bits_to_f32(k), W.bf16_bits_to_f32(v)
    for gi, blk in enumerate(blocks):
        if not 0 <= blk < nb:
            continue
        for h in range(2):
            tile = cache[blk, h]
            kh, vh = oracle.kivi_dequant_tile(tile)
            for c in range(0, DH, 7):
                s16, z16, codes = oracle.kivi_group(kf[gi * G:(gi + 1) * G, h, c])
                assert tile[1024 + 2 * c:1026 + 2 * c].view(np.uint16)[0] == s16
                assert tile[1280 + 2 * c:1282 + 2 * c].view(np.uint16)[0] == z16
                assert np.array_equal(kh[:, c], codes * f16_val(s16) + f16_val(z16))
            for t in range(0, G, 5):
                for gc in range(DH // 32):
                    s16, z16, codes = oracle.kivi_group(vf[gi * G + t, h, 32 * gc:32 * gc + 32])
                    m = tile[2560 + 16 * t + 4 * gc:2564 + 16 * t + 4 * gc].view(np.uint16)
                    assert m[0] == s16 and m[1] == z16
                    assert np.array_equal(vh[t, 32 * gc:32 * gc + 32],
                                          codes * f16_val(s16) + f16_val(z16))


def test_decode_matches_library_sdpa():
    """Quantized groups then the residual, in position order, through torch's
    fp64 scaled_dot_product_attention on the dequantized values."""
    g, k, v = make_groups(740, 7, 2)
    B, Hq, Hkv, R = 2, 8, 2, 64
    quant_groups = np.array([4, 3], np.int32)
    res_lens = np.array([17, 64], np.int32)
    bt = np.array([[6, 0, 2, 5], [1, 4, 3, -1]], np.int32)  # unused entries may hold anything
    cache = np.zeros(oracle.kivi_cache_shape(7, Hkv), np.uint8)
    oracle.kivi_quantize(k, v, np.arange(7, dtype=np.int32), cache)
    rk = W.normal_bf16(g, (B, Hkv, R, DH))
    rv = W.normal_bf16(g, (B, Hkv, R, DH))
    q = W.normal_bf16(g, (B, Hq, DH))
    rows = np.array([(b, h) for b in range(B) for h in range(Hq)], np.int32)
    out = oracle.kivi_decode_rows(rows, q, cache, bt, quant_groups, rk, rv, res_lens)
    for i, (b, hq) in enumerate(rows):
        h = hq // (Hq // Hkv)
        ks, vs = [], []
        for gi in range(quant_groups[b]):
            kh, vh = oracle.kivi_dequant_tile(cache[bt[b, gi], h])
            ks.append(kh)
            vs.append(vh)
        ks.append(W.bf16_bits_to_f32(rk[b, h, :res_lens[b]]).astype(np.float64))
        vs.append(W.bf16_bits_to_f32(rv[b, h, :res_lens[b]]).astype(np.float64))
        kk, vv = np.concatenate(ks), np.concatenate(vs)
        qd = W.bf16_bits_to_f32(q[b, hq]).astype(np.float64)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qd[None, None]), torch.from_numpy(kk[None]),
            torch.from_numpy(vv[None])).numpy()[0, 0]
        np.testing.assert_allclose(out[i], ref, rtol=1e-10, atol=1e-12)


def test_compression_is_below_eight_times():
    """The textbook warns that KIVI's real footprint is not 1/8 of fp16 once
    the metadata and the residual are counted: at S = 16384 with a 128-token
    residual this layout stores 5.16x less than fp16."""
    S, R = 16384, 128
    kivi = (S - R) // G * oracle.KIVI_TILE + 2 * R * DH * 2
    fp16 = 2 * S * DH * 2
    assert 5.0 < fp16 / kivi < 8.0
