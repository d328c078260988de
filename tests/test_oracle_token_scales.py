"""Pins of the oracle's per-token-head scales (the KV-cache quantization
textbook, section 10.4.3: one scale per token along dh; its metadata example
keeps one FP16 scale per (token, head) for K and for V)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

FMTS = [oracle.FMT_E4M3, oracle.FMT_E5M2, oracle.FMT_INT8]


def numpy_scale16(fmt, amax):
    """fp16 bits of clamp(fl32(amax / fmax), 2^-24, 65504) via numpy's float16
    cast (round to nearest even); 1.0 where amax is 0 or not finite."""
    a = np.asarray(amax, np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        s = a / np.float32(oracle.fp8_max(fmt))
    s = np.clip(s, np.float32(2.0 ** -24), np.float32(65504.0))
    bits = s.astype(np.float16).view(np.uint16)
    bad = ~(a > 0) | ~np.isfinite(a)
    return np.where(bad, np.uint16(0x3C00), bits)


def test_f16_decode_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = np.array([oracle.f16_to_double(int(b)) for b in bits[::7]])
    ref = bits[::7].view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


@pytest.mark.parametrize("fmt", FMTS)
def test_scale16_matches_numpy(fmt):
    g = W.rng(41)
    amax = np.concatenate([
        np.exp(g.uniform(np.log(1e-12), np.log(1e12), 4000)).astype(np.float32),
        W.bf16_bits_to_f32(np.arange(0x0001, 0x7F80, 37, dtype=np.uint16)),  # positive bf16
        np.array([0.0, np.inf, np.nan, 448.0, 57344.0, 127.0, 1e-30, 3e38], np.float32)])
    got = np.array([oracle.scale16_from_amax(fmt, float(a)) for a in amax], np.uint16)
    assert np.array_equal(got, numpy_scale16(fmt, amax))


@pytest.mark.parametrize("fmt", FMTS)
def test_token_write_matches_a_numpy_recomputation(fmt):
    g = W.rng(42)
    Hkv, dh, bs = 2, 32, 16
    paging = W.make_paging(g, [37, 5, 16], bs)
    kv = W.make_kv(g, paging, Hkv, dh, k_outliers=(2, 30.0), head_range=(0.01, 100.0))
    kv.k[3] = 0  # an all-zero row: scale 1.0, every code zero
    sm = kv.slot_mapping.copy()
    sm[7] = -1  # padding: skipped
    nb = paging.num_blocks
    kc = np.full(oracle.k_cache_shape(nb, Hkv, bs, dh), 0xA5, np.uint8)
    vc = np.full(oracle.v_cache_shape(nb, Hkv, bs, dh), 0xA5, np.uint8)
    ksc = np.full(oracle.scale_cache_shape(nb, Hkv, bs), 0xBEEF, np.uint16)
    vsc = ksc.copy()
    oracle.cache_write_token(kv.k, kv.v, sm, kc, vc, ksc, vsc, fmt)
    kt = oracle.k_token_view(kc)
    for t in range(len(sm)):
        blk, off = divmod(int(kv.slot_mapping[t]), bs)
        for h in range(Hkv):
            if sm[t] < 0:
                assert ksc[blk, h, off] == 0xBEEF and np.all(kt[blk, h, off] == 0xA5)
                continue
            for x, sc, codes in ((kv.k[t, h], ksc, kt[blk, h, off]), (kv.v[t, h], vsc, vc[blk, h, :, off])):
                amax = np.abs(W.bf16_bits_to_f32(x)).max()
                want = numpy_scale16(fmt, amax)
                assert sc[blk, h, off] == want
                s = np.float32(np.uint16(want).view(np.float16))
                assert np.array_equal(codes, oracle.quantize(fmt, x, s))
    assert np.all(kt[divmod(int(kv.slot_mapping[3]), bs)[0], :, kv.slot_mapping[3] % bs]
                  .view(np.int8 if fmt == oracle.FMT_INT8 else np.uint8) == 0)


@pytest.mark.parametrize("fmt", FMTS)
def test_token_decode_matches_library_sdpa(fmt):
    g = W.rng(43)
    B, Hq, Hkv, dh, bs = 2, 8, 2, 32, 16
    cl = [45, 17]
    paging = W.make_paging(g, cl, bs)
    kv = W.make_kv(g, paging, Hkv, dh, k_outliers=(2, 30.0), head_range=(0.05, 50.0))
    q = W.normal_bf16(g, (B, Hq, dh))
    nb = paging.num_blocks
    kc = np.zeros(oracle.k_cache_shape(nb, Hkv, bs, dh), np.uint8)
    vc = np.zeros(oracle.v_cache_shape(nb, Hkv, bs, dh), np.uint8)
    ksc = np.zeros(oracle.scale_cache_shape(nb, Hkv, bs), np.uint16)
    vsc = ksc.copy()
    oracle.cache_write_token(kv.k, kv.v, kv.slot_mapping, kc, vc, ksc, vsc, fmt)
    rows = np.array([(b, h) for b in range(B) for h in range(Hq)], np.int32)
    out = oracle.decode_token_rows(rows, q, kc, vc, ksc, vsc, paging.block_tables,
                                   paging.context_lens, fmt)
    kt = oracle.k_token_view(kc)
    G = Hq // Hkv
    for i, (b, hq) in enumerate(rows):
        n = cl[b]
        pos = np.arange(n)
        blk = paging.block_tables[b, pos // bs]
        off = pos % bs
        h = hq // G
        sk = ksc[blk, h, off].view(np.float16).astype(np.float64)
        sv = vsc[blk, h, off].view(np.float16).astype(np.float64)
        k = oracle.dequantize(fmt, kt[blk, h, off], 1.0) * sk[:, None]
        v = oracle.dequantize(fmt, vc[blk, h, :, off], 1.0) * sv[:, None]
        qd = W.bf16_bits_to_f32(q[b, hq]).astype(np.float64)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qd[None, None]), torch.from_numpy(k[None]),
            torch.from_numpy(v[None])).numpy()[0, 0]
        np.testing.assert_allclose(out[i], ref, rtol=1e-10, atol=1e-12)
