"""GPU parity of the quantized calls on a mixed pool of padded pages (the vLLM
FP8 KV-cache guide's skip-layers section: skipped layers keep the native dtype,
every layer's page is padded to one common size so the mixed cache aligns page
by page).

A pool holds, per block, one page of each of three layers: FP8 (E4M3), a
skipped bf16 layer, FP8 (E5M2); pages are the bf16 layer's size.  Bar: the FP8
layers' codes bit-exact against the oracle's dense caches, the skipped layer's
bytes and every padding byte untouched; decode / prefill outputs on the
padded layout identical to the same calls on dense caches and within 2e-3 of
the oracle's attention over its own dense caches.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import ATTN_TOL, FMT_ID, rel_err, row_rel_err, same_codes, to_dev, to_np

pytestmark = pytest.mark.gpu

LAYER_BITS = [8, 16, 8]
FILL = 0xA5


def views(pool, layer, nb, Hkv, dh, page):
    """K / V cache views of an FP8 layer inside pool [nb, L, page] (uint8)."""
    import torch
    L = pool.shape[1]
    nat = Hkv * 16 * dh
    base = layer * page
    k = torch.as_strided(pool, (nb, Hkv, dh // 16, 16, 16), (L * page, 16 * dh, 256, 16, 1), base)
    v = torch.as_strided(pool, (nb, Hkv, dh, 16), (L * page, 16 * dh, 16, 1), base + nat)
    return k, v


def make_pool(wl):
    import torch
    import quantized_kv_cache_fp8_amd as K
    nb = wl.paging.num_blocks
    page = K.kvq_common_page_bytes(LAYER_BITS, wl.Hkv, wl.dh, 16)
    assert page == K.kvq_page_bytes(wl.Hkv, wl.dh, 16, 16)
    pool = torch.full((nb, len(LAYER_BITS), page), FILL, dtype=torch.uint8, device="cuda:0")
    # the skipped layer's pages: bf16 K/V as the model would keep them (any bytes)
    g = W.rng(901)
    skipped = torch.from_numpy(g.integers(0, 256, (nb, page), dtype=np.uint8)).to("cuda:0")
    pool[:, 1, :] = skipped
    return pool, page, skipped


def write_layer(wl, pool, layer, page, fmt):
    import torch
    import quantized_kv_cache_fp8_amd as K
    kc, vc = views(pool, layer, wl.paging.num_blocks, wl.Hkv, wl.dh, page)
    k, v = to_dev(wl.kv.k), to_dev(wl.kv.v)
    ks = torch.empty(wl.Hkv, device="cuda:0")
    vs = torch.empty(wl.Hkv, device="cuda:0")
    am = torch.empty(wl.Hkv, device="cuda:0")
    K.kvq_calibrate_scales(k, fmt, "head", am, ks)
    K.kvq_calibrate_scales(v, fmt, "head", am, vs)
    K.kvq_cache_write_paged(k, v, to_dev(wl.kv.slot_mapping), kc, vc, ks, vs, fmt, "head")
    torch.cuda.synchronize()
    return kc, vc, ks, vs


@pytest.mark.parametrize("T_kind", ["decode-step", "long"])
def test_write_into_padded_pages(T_kind):
    cl = [17, 600, 1] if T_kind == "long" else [1, 2, 3]
    wl = W.decode_workload("paged", 910, len(cl), 16, 4, 128, cl, 16, "e4m3", "head",
                           k_outliers=(4, 10.0))
    pool, page, skipped = make_pool(wl)
    nat = wl.Hkv * 16 * wl.dh
    for layer, fmt in ((0, "e4m3"), (2, "e5m2")):
        kc, vc, ks, vs = write_layer(wl, pool, layer, page, fmt)
        rk = np.full(oracle.k_cache_shape(wl.paging.num_blocks, wl.Hkv, 16, wl.dh), FILL, np.uint8)
        rv = np.full(oracle.v_cache_shape(wl.paging.num_blocks, wl.Hkv, 16, wl.dh), FILL, np.uint8)
        oracle.cache_write(wl.kv.k, wl.kv.v, wl.kv.slot_mapping, rk, rv, to_np(ks), to_np(vs),
                           FMT_ID[fmt], oracle.GRAN_HEAD)
        assert same_codes(FMT_ID[fmt], to_np(kc), rk) and same_codes(FMT_ID[fmt], to_np(vc), rv)
    p = to_np(pool)
    assert np.array_equal(p[:, 1, :], to_np(skipped))      # the skipped layer is untouched
    assert np.all(p[:, 0, 2 * nat:] == FILL) and np.all(p[:, 2, 2 * nat:] == FILL)  # padding


def test_decode_and_prefill_on_padded_pages_match_dense_caches_and_the_oracle():
    import torch
    import quantized_kv_cache_fp8_amd as K
    # prefill workload: 3 sequences, cached prefix + chunk; its caches serve decode too
    pw = W.prefill_workload("paged-prefill", 920, [100, 300, 0], [40, 129, 77], Hq=16, Hkv=4)
    pool, page, _ = make_pool(pw)
    kc, vc, ks, vs = write_layer(pw, pool, 2, page, "e4m3")
    dk, dv = kc.contiguous(), vc.contiguous()  # the same bytes, unpadded
    # the oracle's own scales and dense caches of the same layer
    fmt, gh = oracle.FMT_E4M3, oracle.GRAN_HEAD
    rks = oracle.calibrate(pw.kv.k, fmt, gh)[1]
    rvs = oracle.calibrate(pw.kv.v, fmt, gh)[1]
    assert np.array_equal(to_np(ks), rks) and np.array_equal(to_np(vs), rvs)
    nb = pw.paging.num_blocks
    rk = np.full(oracle.k_cache_shape(nb, pw.Hkv, 16, pw.dh), FILL, np.uint8)
    rv = np.full(oracle.v_cache_shape(nb, pw.Hkv, 16, pw.dh), FILL, np.uint8)
    oracle.cache_write(pw.kv.k, pw.kv.v, pw.kv.slot_mapping, rk, rv, rks, rvs, fmt, gh)
    bt, cl = to_dev(pw.paging.block_tables), to_dev(pw.paging.context_lens)
    g = W.rng(921)
    q_np = W.normal_bf16(g, (len(pw.prefix_lens), pw.Hq, pw.dh))
    q = to_dev(q_np)
    mc = int(pw.paging.context_lens.max())
    outs = []
    for kk, vv, fn in ((kc, vc, K.kvq_decode_attn_paged), (dk, dv, K.kvq_decode_attn)):
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda:0")
        fn(out, q, kk, vv, bt, cl, mc, ks, vs, "e4m3", "head")
        torch.cuda.synchronize()
        outs.append(to_np(out))
    assert np.array_equal(outs[0], outs[1])
    ref = oracle.decode_attn(q_np, rk, rv, pw.paging.block_tables, pw.paging.context_lens, rks,
                             rvs, fmt, gh)
    e, er = rel_err(outs[0], ref), row_rel_err(outs[0], ref)
    print(f"padded decode: global rel err {e:.3e}  worst row {er:.3e}", flush=True)
    assert e <= ATTN_TOL and er <= ATTN_TOL
    qp = to_dev(pw.q)
    qs = torch.empty(pw.Hq, device="cuda:0")
    am = torch.empty(pw.Hq, device="cuda:0")
    K.kvq_calibrate_scales(qp, "e4m3", "head", am, qs)
    cu = to_dev(pw.cu_seqlens)
    mq = int(np.diff(pw.cu_seqlens).max())
    outs = []
    for kk, vv, fn in ((kc, vc, K.kvq_prefill_attn_paged), (dk, dv, K.kvq_prefill_attn)):
        out = torch.full(qp.shape, float("nan"), dtype=torch.float32, device="cuda:0")
        fn(out, qp, cu, mq, qs, "head", kk, vv, bt, cl, ks, vs, "e4m3", "head")
        torch.cuda.synchronize()
        outs.append(to_np(out))
    assert np.array_equal(outs[0], outs[1])
    rqs = oracle.calibrate(pw.q, fmt, gh)[1]
    assert np.array_equal(to_np(qs), rqs)
    ref = oracle.prefill_attn(pw.q, pw.cu_seqlens, rqs, gh, rk, rv, pw.paging.block_tables,
                              pw.paging.context_lens, rks, rvs, fmt, gh)
    e = rel_err(outs[0], ref)
    print(f"padded prefill: global rel err {e:.3e}  worst row {row_rel_err(outs[0], ref):.3e}",
          flush=True)
    assert e <= ATTN_TOL
