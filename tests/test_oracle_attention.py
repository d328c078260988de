"""Pins for the oracle's attention over the paged FP8 cache (CPU only).

Definition: textbook 10.4.2, P = softmax(Q K_hat^T / sqrt(dh) + mask), O = P V_hat
with K_hat = sK * Kq and V_hat = sV * Vq (10.4.5: cast_float(Kfp8) * sK).  The
checks use torch's fp64 scaled_dot_product_attention (a library routine) on
dequantized K/V gathered through the block table, and closed-form special cases.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

FMTS = [oracle.FMT_E4M3, oracle.FMT_E5M2, oracle.FMT_INT8]


def build_cache(paging, kv, Hkv, dh, fmt, gran, g):
    n = Hkv if gran == oracle.GRAN_HEAD else 1
    ks = (g.uniform(0.005, 0.05, n)).astype(np.float32)
    vs = (g.uniform(0.005, 0.05, n)).astype(np.float32)
    kc = np.zeros(oracle.k_cache_shape(paging.num_blocks, Hkv, paging.bs, dh), np.uint8)
    vc = np.zeros((paging.num_blocks, Hkv, dh, paging.bs), np.uint8)
    oracle.cache_write(kv.k, kv.v, kv.slot_mapping, kc, vc, ks, vs, fmt, gran)
    return kc, vc, ks, vs


def gather(cache, paging, b, n, fmt, scales, gran, kind):
    """Dequantized [Hkv, n, dh] history of sequence b, read through the block
    table; K tiles are [dh/16][bs][16] (viewed token-major), V tiles [dh][bs]
    (channel-major)."""
    pos = np.arange(n)
    blk = paging.block_tables[b, pos // paging.bs]
    if kind == "k":
        codes = oracle.k_token_view(cache)[blk, :, pos % paging.bs, :]  # [n, Hkv, dh]
    else:
        codes = cache[blk, :, :, pos % paging.bs]  # [n, Hkv, dh]
    Hkv = cache.shape[1]
    s = np.asarray(scales, np.float64).reshape(-1)
    s = s if gran == oracle.GRAN_HEAD else np.repeat(s, Hkv)
    return oracle.dequantize(fmt, codes, 1.0).transpose(1, 0, 2) * s[:, None, None]


def sdpa(q, k, v, G, mask=None, scale=None):
    """q [Hq, nq, dh], k/v [Hkv, nk, dh] fp64 -> [Hq, nq, dh] via torch."""
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(k).repeat_interleave(G, dim=0)
    tv = torch.from_numpy(v).repeat_interleave(G, dim=0)
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m,
                                                            scale=scale).numpy()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("gran", [oracle.GRAN_TENSOR, oracle.GRAN_HEAD])
def test_decode_matches_library_sdpa(fmt, gran):
    g = W.rng(21)
    B, Hq, Hkv, dh = 3, 8, 2, 32
    paging = W.make_paging(g, [1, 17, 40], 16)
    kv = W.make_kv(g, paging, Hkv, dh, k_outliers=(2, 8.0), head_range=(0.5, 20.0))
    q = W.normal_bf16(g, (B, Hq, dh))
    kc, vc, ks, vs = build_cache(paging, kv, Hkv, dh, fmt, gran, g)
    out = oracle.decode_attn(q, kc, vc, paging.block_tables, paging.context_lens, ks, vs, fmt,
                             gran)
    qf = W.bf16_bits_to_f32(q).astype(np.float64)
    for b in range(B):
        n = int(paging.context_lens[b])
        k = gather(kc, paging, b, n, fmt, ks, gran, "k")
        v = gather(vc, paging, b, n, fmt, vs, gran, "v")
        ref = sdpa(qf[b][:, None, :], k, v, Hq // Hkv)[:, 0, :]
        np.testing.assert_allclose(out[b], ref, rtol=1e-12, atol=1e-12)


def test_decode_special_cases():
    g = W.rng(22)
    Hq, Hkv, dh, bs = 4, 2, 16, 16
    fmt, gran = oracle.FMT_E4M3, oracle.GRAN_TENSOR
    # ctx = 1: the output is that one dequantized value row
    paging = W.make_paging(g, [1], bs)
    kv = W.make_kv(g, paging, Hkv, dh)
    kc, vc, ks, vs = build_cache(paging, kv, Hkv, dh, fmt, gran, g)
    q = W.normal_bf16(g, (1, Hq, dh))
    out = oracle.decode_attn(q, kc, vc, paging.block_tables, paging.context_lens, ks, vs, fmt,
                             gran)
    v0 = gather(vc, paging, 0, 1, fmt, vs, gran, "v")[:, 0, :]
    assert np.array_equal(out[0], np.repeat(v0, Hq // Hkv, axis=0))
    # q = 0: uniform weights, the output is the mean of the dequantized values
    paging = W.make_paging(g, [45], bs)
    kv = W.make_kv(g, paging, Hkv, dh)
    kc, vc, ks, vs = build_cache(paging, kv, Hkv, dh, fmt, gran, g)
    q0 = np.zeros((1, Hq, dh), np.uint16)
    out = oracle.decode_attn(q0, kc, vc, paging.block_tables, paging.context_lens, ks, vs, fmt,
                             gran)
    vmean = gather(vc, paging, 0, 45, fmt, vs, gran, "v").mean(axis=1)
    np.testing.assert_allclose(out[0], np.repeat(vmean, 2, axis=0), rtol=1e-13, atol=1e-15)
    # every key equal: same uniform weights for any q
    kv.k[:] = kv.k[0]
    kc, vc, ks, vs = build_cache(paging, kv, Hkv, dh, fmt, gran, g)
    out = oracle.decode_attn(q, kc, vc, paging.block_tables, paging.context_lens, ks, vs, fmt,
                             gran)
    vmean = gather(vc, paging, 0, 45, fmt, vs, gran, "v").mean(axis=1)
    np.testing.assert_allclose(out[0], np.repeat(vmean, 2, axis=0), rtol=1e-13, atol=1e-15)
    # one dominant logit: the output is (almost exactly) that key's value row
    kv = W.make_kv(g, paging, Hkv, dh)
    qd = np.zeros((1, Hq, dh), np.float32)
    qd[..., 0] = 64.0
    kv.k[:, :, 0] = W.f32_to_bf16_bits(np.zeros(1, np.float32))[0]
    kv.k[30, :, 0] = W.f32_to_bf16_bits(np.array([8.0], np.float32))[0]
    kc, vc, _, _ = build_cache(paging, kv, Hkv, dh, fmt, gran, g)
    one = np.ones(1, np.float32)
    out = oracle.decode_attn(W.f32_to_bf16_bits(qd), kc, vc, paging.block_tables,
                             paging.context_lens, one, one, fmt, gran, softmax_scale=1.0)
    v30 = gather(vc, paging, 0, 45, fmt, one, gran, "v")[:, 30, :]
    np.testing.assert_allclose(out[0], np.repeat(v30, 2, axis=0), rtol=0, atol=1e-100)


def test_decode_invariant_under_key_order_and_block_placement():
    """Attention without a mask is a function of the set of (k, v) pairs: moving
    tokens to other positions and other physical blocks leaves the output alone."""
    g = W.rng(23)
    Hq, Hkv, dh = 6, 3, 48
    fmt, gran = oracle.FMT_E5M2, oracle.GRAN_HEAD
    paging = W.make_paging(g, [70], 16)
    kv = W.make_kv(g, paging, Hkv, dh, head_range=(0.5, 20.0))
    q = W.normal_bf16(g, (1, Hq, dh), 1, W.log_uniform(g, Hq, 0.5, 20))
    kc, vc, ks, vs = build_cache(paging, kv, Hkv, dh, fmt, gran, g)
    out1 = oracle.decode_attn(q, kc, vc, paging.block_tables, paging.context_lens, ks, vs, fmt,
                              gran)
    perm = g.permutation(70)
    paging2 = W.make_paging(W.rng(99), [70], 16)
    kv2 = W.KVBatch(kv.k[perm].copy(), kv.v[perm].copy(), paging2.slots(0, np.arange(70)),
                    kv.seq_offsets)
    kc2 = np.zeros(oracle.k_cache_shape(paging2.num_blocks, Hkv, 16, dh), np.uint8)
    vc2 = np.zeros((paging2.num_blocks, Hkv, dh, 16), np.uint8)
    oracle.cache_write(kv2.k, kv2.v, kv2.slot_mapping, kc2, vc2, ks, vs, fmt, gran)
    out2 = oracle.decode_attn(q, kc2, vc2, paging2.block_tables, paging2.context_lens, ks, vs,
                              fmt, gran)
    np.testing.assert_allclose(out1, out2, rtol=1e-13, atol=1e-15)


def test_decode_zero_context_gives_zero_row():
    g = W.rng(24)
    paging = W.make_paging(g, [0, 5], 16)
    kv = W.make_kv(g, paging, 1, 16)
    kc, vc, ks, vs = build_cache(paging, kv, 1, 16, 0, 0, g)
    out = oracle.decode_attn(W.normal_bf16(g, (2, 2, 16)), kc, vc, paging.block_tables,
                             paging.context_lens, ks, vs, 0, 0)
    assert np.all(out[0] == 0) and np.all(np.isfinite(out[1])) and np.any(out[1] != 0)


def test_decode_rows_equal_full_decode():
    g = W.rng(25)
    paging = W.make_paging(g, [19, 33], 16)
    kv = W.make_kv(g, paging, 2, 16)
    kc, vc, ks, vs = build_cache(paging, kv, 2, 16, 0, 1, g)
    q = W.normal_bf16(g, (2, 4, 16))
    full = oracle.decode_attn(q, kc, vc, paging.block_tables, paging.context_lens, ks, vs, 0, 1)
    rows = np.array([[1, 3], [0, 0], [1, 1]], np.int32)
    sub = oracle.decode_rows(rows, q, kc, vc, paging.block_tables, paging.context_lens, ks, vs,
                             0, 1)
    for i, (b, h) in enumerate(rows):
        assert np.array_equal(sub[i], full[b, h])


def quantized_q(q_bits, q_scale, gran):
    """q_hat = s_q * cast_float(cast_e4m3(fl32(q / s_q))), via numpy division and torch casts."""
    qf = W.bf16_bits_to_f32(q_bits)
    s = np.asarray(q_scale, np.float32)
    s = s[None, :, None] if gran == oracle.GRAN_HEAD else s.reshape(1, 1, 1)
    c = torch.from_numpy((qf / s).astype(np.float32)).to(torch.float8_e4m3fn)
    return c.to(torch.float64).numpy() * s.astype(np.float64)


@pytest.mark.parametrize("fmt", FMTS)
def test_prefill_matches_library_sdpa_with_causal_offset(fmt):
    g = W.rng(31)
    Hq, Hkv, dh = 4, 2, 32
    wl = W.prefill_workload("t", 31, [20, 0, 16], [13, 9, 1], Hq, Hkv, dh, 16)
    kc, vc, ks, vs = build_cache(wl.paging, wl.kv, Hkv, dh, fmt, oracle.GRAN_HEAD, g)
    qs = (np.abs(W.bf16_bits_to_f32(wl.q)).max(axis=(0, 2)) / np.float32(448)).astype(np.float32)
    out = oracle.prefill_attn(wl.q, wl.cu_seqlens, qs, oracle.GRAN_HEAD, kc, vc,
                              wl.paging.block_tables, wl.paging.context_lens, ks, vs, fmt,
                              oracle.GRAN_HEAD)
    qh = quantized_q(wl.q, qs, oracle.GRAN_HEAD)
    for b in range(3):
        lo, hi = wl.cu_seqlens[b], wl.cu_seqlens[b + 1]
        n = int(wl.paging.context_lens[b])
        k = gather(kc, wl.paging, b, n, fmt, ks, oracle.GRAN_HEAD, "k")
        v = gather(vc, wl.paging, b, n, fmt, vs, oracle.GRAN_HEAD, "v")
        qlen = hi - lo
        pos = n - qlen + np.arange(qlen)
        mask = np.arange(n)[None, :] <= pos[:, None]
        ref = sdpa(qh[lo:hi].transpose(1, 0, 2).copy(), k, v, Hq // Hkv, mask)
        np.testing.assert_allclose(out[lo:hi], ref.transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


def test_prefill_last_row_equals_decode_of_quantized_query():
    """With a power-of-two q scale the quantized query is exactly a bf16 value,
    so the last chunk row of a prefill equals a decode step over the same cache."""
    g = W.rng(32)
    Hq, Hkv, dh = 4, 1, 16
    wl = W.prefill_workload("t", 32, [21], [11], Hq, Hkv, dh, 16)
    kc, vc, ks, vs = build_cache(wl.paging, wl.kv, Hkv, dh, 0, 0, g)
    qs = np.array([2.0 ** -6], np.float32)
    pre = oracle.prefill_attn(wl.q, wl.cu_seqlens, qs, 0, kc, vc, wl.paging.block_tables,
                              wl.paging.context_lens, ks, vs, 0, 0)
    qh = quantized_q(wl.q, qs, 0)[-1:]  # [1, Hq, dh]
    qh_bits = W.f32_to_bf16_bits(qh.astype(np.float32))
    assert np.array_equal(W.bf16_bits_to_f32(qh_bits), qh.astype(np.float32))
    dec = oracle.decode_attn(qh_bits, kc, vc, wl.paging.block_tables, wl.paging.context_lens, ks,
                             vs, 0, 0)
    assert np.array_equal(pre[-1], dec[0])


def test_prefill_rows_equal_full_prefill():
    g = W.rng(33)
    wl = W.prefill_workload("t", 33, [5, 30], [7, 18], 4, 2, 16, 16)
    kc, vc, ks, vs = build_cache(wl.paging, wl.kv, 2, 16, 1, 1, g)
    qs = np.array([0.02], np.float32)
    full = oracle.prefill_attn(wl.q, wl.cu_seqlens, qs, 0, kc, vc, wl.paging.block_tables,
                               wl.paging.context_lens, ks, vs, 1, 1)
    rows = np.array([[0, 0], [24, 3], [7, 1], [6, 2]], np.int64)
    sub = oracle.prefill_rows(rows, wl.q, wl.cu_seqlens, qs, 0, kc, vc, wl.paging.block_tables,
                              wl.paging.context_lens, ks, vs, 1, 1)
    for i, (r, h) in enumerate(rows):
        assert np.array_equal(sub[i], full[r, h])


def test_dense_attention_helper_against_sdpa():
    g = W.rng(34)
    q, k, v = g.standard_normal((5, 8)), g.standard_normal((9, 8)), g.standard_normal((9, 8))
    for causal in (False, True):
        ours = oracle.dense_attn(q, k, v, causal, 0.3)
        mask = None
        if causal:
            mask = np.arange(9)[None, :] <= (9 - 5 + np.arange(5))[:, None]
        ref = sdpa(q[None], k[None], v[None], 1, None if mask is None else mask, 0.3)[0]
        np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-13)
