"""GPU parity on cache pools larger than 4 GiB and on inputs of more than 2^32
elements: no offset a kernel forms may wrap at 32 bits.

A device with 288 GB of memory holds KV pools of tens of GB, so in ordinary
serving a block's byte offset in its pool passes 2^31 and 2^32.  Each pool case
takes a seeded workload and moves its blocks to ids spread over a pool of about
4.9 GB per cache, with ids on both sides of the 2^31 and 2^32 byte offsets.
The pool is pre-filled with NaN codes.  It then checks:
- the bytes of every used block, gathered back, bit-exact against the oracle's
  compact pool; blocks that no token maps to, among them the 32-bit wraps of
  the used ids, still hold the fill;
- attention against the oracle on the compact pool, within 2e-3 globally and
  per row.

The calibration and write case reads inputs of more than 2^32 bf16 elements.
One seeded 4096-token block is tiled on the device, and distinct tokens are
planted past the 2^31 and 2^32 element offsets and at the end.  The oracle then
runs on the distinct tokens only.  This is exact for two reasons: a maximum
depends only on the set of values, and a token's codes depend only on its own
values and the scale.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import ATTN_TOL, FMT_ID, GRAN_ID, rel_err, row_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

HKV, DH, BS = 8, 128, 16
BLOCK_BYTES = HKV * BS * DH  # one cache's bytes per block: 16 KiB
NB_BIG = 300_000  # 4.9 GB per cache
EDGE_IDS = [(1 << 31) // BLOCK_BYTES - 1, (1 << 31) // BLOCK_BYTES,
            (1 << 32) // BLOCK_BYTES - 1, (1 << 32) // BLOCK_BYTES, NB_BIG - 1]
NAN_FILL = 0x7F  # a NaN code in E4M3 and in E5M2 (and 127 in INT8)


@pytest.fixture(autouse=True)
def _release_pools():
    import torch
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def spread_ids(seed, n, nb_big, edges):
    """n distinct block ids of a pool of nb_big blocks, in seeded order: the
    edge ids, then ids drawn from the rest of the pool."""
    g = W.rng(seed)
    rest = np.setdiff1d(np.arange(nb_big, dtype=np.int64), edges)
    ids = np.concatenate([np.asarray(edges, np.int64),
                          g.choice(rest, n - len(edges), replace=False)])
    return g.permutation(ids)


def remap(block_tables, slot_mapping, ids, bs):
    """Block tables and slots with compact block i moved to ids[i]."""
    bt = ids[block_tables].astype(np.int32)
    s = np.asarray(slot_mapping, np.int64)
    slots = np.where(s >= 0, ids[np.maximum(s, 0) >> 4] * bs + (s & (bs - 1)), s)
    return bt, slots.astype(np.int64)


def unused_probe_ids(ids, nb_big, wrap_blocks, seed, n=16):
    """Ids no token maps to: the 32-bit wraps of the used ids, and a seeded sample."""
    used = set(int(i) for i in ids)
    wraps = {int(i) % wrap_blocks for i in ids if i >= wrap_blocks} - used
    g = W.rng(seed)
    sample = {int(i) for i in g.choice(nb_big, 4 * n, replace=False)} - used
    return np.array(sorted(wraps | set(sorted(sample)[:n])), np.int64)


def gather(t, ids):
    import torch
    return to_np(t[torch.from_numpy(np.asarray(ids, np.int64)).to(t.device)])


def check_attn(out, ref):
    e, er = rel_err(out, ref), row_rel_err(out, ref)
    print(f"global rel err {e:.3e}  worst row {er:.3e}", flush=True)
    assert np.all(np.isfinite(out)), "some output rows were never written"
    assert e <= ATTN_TOL and er <= ATTN_TOL


def big_pools(shape_fn, fill=NAN_FILL):
    import torch
    return (torch.full(shape_fn(NB_BIG, HKV, BS, DH), fill, dtype=torch.uint8, device="cuda:0"),
            torch.full(oracle.v_cache_shape(NB_BIG, HKV, BS, DH), fill, dtype=torch.uint8,
                       device="cuda:0"))


@pytest.mark.parametrize("Hq,fmt,gran", [(32, "e4m3", "tensor"), (64, "e5m2", "head"),
                                         (32, "int8", "head")])
def test_write_decode_and_append_over_a_pool_beyond_4gib(Hq, fmt, gran):
    """Write and decode (groups of 4 and of 8 heads), then the fused append of
    each sequence's newest token, on block ids past 2^31 and 2^32 bytes."""
    import torch
    import quantized_kv_cache_fp8_amd as K
    cl = [4097, 600, 1, 2500]
    wl = W.decode_workload("big-pool", 1400 + Hq, len(cl), Hq, HKV, DH, cl, BS, fmt, gran,
                           k_outliers=(2, 8.0), head_range=(0.5, 20.0))
    f, gr = FMT_ID[fmt], GRAN_ID[gran]
    nb = wl.paging.num_blocks
    ids = spread_ids(1450 + Hq, nb, NB_BIG, EDGE_IDS)
    bt, slots = remap(wl.paging.block_tables, wl.kv.slot_mapping, ids, BS)
    print(f"Hq={Hq} {fmt} {gran}: {nb} blocks, highest id {int(ids.max())}", flush=True)
    # oracle on the compact pool
    ks_ref = oracle.calibrate(wl.kv.k, f, gr)[1]
    vs_ref = oracle.calibrate(wl.kv.v, f, gr)[1]
    kc_ref = np.full(oracle.k_cache_shape(nb, HKV, BS, DH), NAN_FILL, np.uint8)
    vc_ref = np.full(oracle.v_cache_shape(nb, HKV, BS, DH), NAN_FILL, np.uint8)
    oracle.cache_write(wl.kv.k, wl.kv.v, wl.kv.slot_mapping, kc_ref, vc_ref, ks_ref, vs_ref, f,
                       gr)
    ref = oracle.decode_attn(wl.q, kc_ref, vc_ref, wl.paging.block_tables,
                             wl.paging.context_lens, ks_ref, vs_ref, f, gr)
    # GPU on the big pool
    dev = "cuda:0"
    nh = HKV if gr == oracle.GRAN_HEAD else 1
    ks, vs, am = (torch.empty(nh, device=dev) for _ in range(3))
    k, v, q = to_dev(wl.kv.k), to_dev(wl.kv.v), to_dev(wl.q)
    K.kvq_calibrate_scales(k, f, gr, am, ks)
    K.kvq_calibrate_scales(v, f, gr, am, vs)
    kc, vc = big_pools(oracle.k_cache_shape)
    K.kvq_cache_write(k, v, to_dev(slots), kc, vc, ks, vs, f, gr)
    out = torch.full((wl.B, Hq, DH), float("nan"), dtype=torch.float32, device=dev)
    d_bt, d_cl = to_dev(bt), to_dev(wl.paging.context_lens)
    K.kvq_decode_attn(out, q, kc, vc, d_bt, d_cl, max(cl), ks, vs, f, gr)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(ks), ks_ref) and np.array_equal(to_np(vs), vs_ref)
    assert np.array_equal(gather(kc, ids), kc_ref) and np.array_equal(gather(vc, ids), vc_ref)
    probe = unused_probe_ids(ids, NB_BIG, (1 << 32) // BLOCK_BYTES, 1460 + Hq)
    assert np.all(gather(kc, probe) == NAN_FILL) and np.all(gather(vc, probe) == NAN_FILL)
    check_attn(to_np(out), ref)

    # the fused append: every token but each sequence's newest is in the
    # cache; the call writes the newest and attends over all of them
    offs = wl.kv.seq_offsets
    last = offs[1:] - 1
    old = slots.copy()
    old[last] = -1
    kc.fill_(NAN_FILL)
    vc.fill_(NAN_FILL)
    K.kvq_cache_write(k, v, to_dev(old), kc, vc, ks, vs, f, gr)
    li = torch.from_numpy(last).to(dev)
    out2 = torch.full_like(out, float("nan"))
    K.kvq_decode_attn_append(out2, q, k[li].contiguous(), v[li].contiguous(), kc, vc, d_bt, d_cl,
                             max(cl), ks, vs, f, gr)
    torch.cuda.synchronize()
    assert np.array_equal(gather(kc, ids), kc_ref) and np.array_equal(gather(vc, ids), vc_ref)
    assert np.array_equal(to_np(out2), to_np(out)), "append differs from write-then-decode"


def test_token_scales_over_a_pool_beyond_4gib():
    """Per-token-head fp16 scales: write and decode on high block ids, the
    scale caches ([blocks][Hkv][16] fp16) indexed by the same ids."""
    import torch
    import quantized_kv_cache_fp8_amd as K
    g = W.rng(1470)
    cl = [3000, 17, 1025]
    paging = W.make_paging(g, cl, BS)
    kv = W.make_kv(g, paging, HKV, DH, k_outliers=(4, 10.0), v_outliers=(4, 10.0))
    k = W.scale_rows(g, kv.k, 0.2, 5.0)
    v = W.scale_rows(g, kv.v, 1e-3, 1e3)
    q = W.normal_bf16(g, (len(cl), 32, DH))
    nb = paging.num_blocks
    ids = spread_ids(1471, nb, NB_BIG, EDGE_IDS)
    bt, slots = remap(paging.block_tables, kv.slot_mapping, ids, BS)
    f = FMT_ID["e4m3"]
    kc_ref = np.full(oracle.k_cache_shape(nb, HKV, BS, DH), NAN_FILL, np.uint8)
    vc_ref = np.full(oracle.v_cache_shape(nb, HKV, BS, DH), NAN_FILL, np.uint8)
    ksc_ref = np.full(oracle.scale_cache_shape(nb, HKV, BS), 0x7E00, np.uint16)
    vsc_ref = ksc_ref.copy()
    oracle.cache_write_token(k, v, kv.slot_mapping, kc_ref, vc_ref, ksc_ref, vsc_ref, f)
    rows = np.array([(b, h) for b in range(len(cl)) for h in range(32)], np.int32)
    ref = oracle.decode_token_rows(rows, q, kc_ref, vc_ref, ksc_ref, vsc_ref, paging.block_tables,
                                   paging.context_lens, f).reshape(len(cl), 32, DH)
    dev = "cuda:0"
    kc, vc = big_pools(oracle.k_cache_shape)
    # fp16 NaN bits (0x7E00 fits int16) in every scale no token writes
    ksc = torch.full(oracle.scale_cache_shape(NB_BIG, HKV, BS), 0x7E00, dtype=torch.int16,
                     device=dev)
    vsc = ksc.clone()
    K.kvq_cache_write_token_scales(to_dev(k), to_dev(v), to_dev(slots), kc, vc, ksc, vsc, f)
    out = torch.full((len(cl), 32, DH), float("nan"), dtype=torch.float32, device=dev)
    K.kvq_decode_attn_token_scales(out, to_dev(q), kc, vc, ksc, vsc, to_dev(bt),
                                   to_dev(paging.context_lens), max(cl), f)
    torch.cuda.synchronize()
    assert np.array_equal(gather(kc, ids), kc_ref) and np.array_equal(gather(vc, ids), vc_ref)
    assert np.array_equal(gather(ksc, ids).view(np.uint16), ksc_ref)
    assert np.array_equal(gather(vsc, ids).view(np.uint16), vsc_ref)
    check_attn(to_np(out), ref)


def test_prefill_over_a_pool_beyond_4gib():
    """The FP8-domain chunked prefill reading prefix and chunk from high block ids."""
    import torch
    import quantized_kv_cache_fp8_amd as K
    wl = W.prefill_workload("big-pool-prefill", 1480, [700, 0, 1500], [300, 64, 129], Hq=32,
                            Hkv=HKV, dh=DH, fmt="e4m3")
    f, gr = FMT_ID["e4m3"], oracle.GRAN_HEAD
    nb = wl.paging.num_blocks
    ids = spread_ids(1481, nb, NB_BIG, EDGE_IDS)
    bt, slots = remap(wl.paging.block_tables, wl.kv.slot_mapping, ids, BS)
    qs_ref = oracle.calibrate(wl.q, oracle.FMT_E4M3, gr)[1]
    ks_ref = oracle.calibrate(wl.kv.k, f, gr)[1]
    vs_ref = oracle.calibrate(wl.kv.v, f, gr)[1]
    kc_ref = np.full(oracle.k_cache_shape(nb, HKV, BS, DH), NAN_FILL, np.uint8)
    vc_ref = np.full(oracle.v_cache_shape(nb, HKV, BS, DH), NAN_FILL, np.uint8)
    oracle.cache_write(wl.kv.k, wl.kv.v, wl.kv.slot_mapping, kc_ref, vc_ref, ks_ref, vs_ref, f,
                       gr)
    ref = oracle.prefill_attn(wl.q, wl.cu_seqlens, qs_ref, gr, kc_ref, vc_ref,
                              wl.paging.block_tables, wl.paging.context_lens, ks_ref, vs_ref, f,
                              gr)
    dev = "cuda:0"
    q = to_dev(wl.q)
    qs, ks, vs = torch.empty(32, device=dev), torch.empty(HKV, device=dev), \
        torch.empty(HKV, device=dev)
    am = torch.empty(32, device=dev)
    k, v = to_dev(wl.kv.k), to_dev(wl.kv.v)
    K.kvq_calibrate_scales(q, oracle.FMT_E4M3, gr, am, qs)
    K.kvq_calibrate_scales(k, f, gr, am[:HKV], ks)
    K.kvq_calibrate_scales(v, f, gr, am[:HKV], vs)
    kc, vc = big_pools(oracle.k_cache_shape)
    K.kvq_cache_write(k, v, to_dev(slots), kc, vc, ks, vs, f, gr)
    out = torch.full((wl.q.shape[0], 32, DH), float("nan"), dtype=torch.float32, device=dev)
    K.kvq_prefill_attn(out, q, to_dev(wl.cu_seqlens), int(np.diff(wl.cu_seqlens).max()), qs, gr,
                       kc, vc, to_dev(bt), to_dev(wl.paging.context_lens), ks, vs, f, gr)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(qs), qs_ref) and np.array_equal(to_np(ks), ks_ref)
    assert np.array_equal(gather(kc, ids), kc_ref) and np.array_equal(gather(vc, ids), vc_ref)
    o = to_np(out)
    assert np.all(np.isfinite(o)), "some output rows were never written"
    e = rel_err(o, ref)
    print(f"global rel err {e:.3e}  worst row {row_rel_err(o, ref):.3e}", flush=True)
    assert e <= ATTN_TOL


def test_kivi_over_a_pool_beyond_4gib():
    """The 2-bit cache: 24 KiB per block at 8 heads, 200,000 blocks (4.9 GB);
    quantize and decode on ids past 2^31 and 2^32 bytes."""
    import torch
    import quantized_kv_cache_fp8_amd as K
    tile_block = HKV * K.KIVI_TILE  # bytes per block
    nb_big = 200_000
    edges = [(1 << 31) // tile_block, (1 << 31) // tile_block + 1,
             (1 << 32) // tile_block, (1 << 32) // tile_block + 1, nb_big - 1]
    wl = W.kivi_workload("big-pool-kivi", 1490, 32, HKV, [40, 0, 17, 33], [5, 128, 0, 77])
    nb = wl.paging.num_blocks
    ids = spread_ids(1491, nb, nb_big, edges)
    gb = ids[wl.group_blocks].astype(np.int32)
    bt = ids[wl.paging.block_tables].astype(np.int32)
    fill = 0x5A
    cache_ref = np.full(oracle.kivi_cache_shape(nb, HKV), fill, np.uint8)
    oracle.kivi_quantize(wl.k, wl.v, wl.group_blocks, cache_ref)
    rows = np.array([(b, h) for b in range(wl.B) for h in range(wl.Hq)], np.int32)
    ref = oracle.kivi_decode_rows(rows, wl.q, cache_ref, wl.paging.block_tables, wl.quant_groups,
                                  wl.res_k, wl.res_v, wl.res_lens).reshape(wl.B, wl.Hq, 128)
    dev = "cuda:0"
    cache = torch.full(oracle.kivi_cache_shape(nb_big, HKV), fill, dtype=torch.uint8, device=dev)
    K.kvq_kivi_quantize(to_dev(wl.k), to_dev(wl.v), to_dev(gb), cache)
    out = torch.full((wl.B, wl.Hq, 128), float("nan"), dtype=torch.float32, device=dev)
    K.kvq_kivi_decode_attn(out, to_dev(wl.q), cache, to_dev(bt), to_dev(wl.quant_groups),
                           int(wl.quant_groups.max()), to_dev(wl.res_k), to_dev(wl.res_v),
                           to_dev(wl.res_lens))
    torch.cuda.synchronize()
    assert np.array_equal(gather(cache, ids), cache_ref)
    probe = unused_probe_ids(ids, nb_big, (1 << 32) // tile_block, 1492)
    assert np.all(gather(cache, probe) == fill)
    check_attn(to_np(out), ref)


def test_calibrate_and_write_beyond_2p32_elements():
    """K and V of 4.3 million tokens at 8 x 128 (4.4e9 elements each, 8.8 GB of
    bf16): calibration per head in one call for K and V, and per tensor; then
    the write into block-permuted slots.  Checked on the distinct tokens."""
    import torch
    import quantized_kv_cache_fp8_amd as K
    T, nbase = 4_300_000, 4096
    assert T * HKV * DH > 1 << 32
    g = W.rng(1500)
    base_k = W.normal_bf16(g, (nbase, HKV, DH), 1, W.log_uniform(g, HKV, 0.5, 4.0))
    base_v = W.normal_bf16(g, (nbase, HKV, DH), 1, W.log_uniform(g, HKV, 0.5, 4.0))
    row = HKV * DH
    plant_at = np.array([(1 << 31) // row + 5, (1 << 32) // row + 7, T - 1], np.int64)
    plant_k = W.scale_rows(g, W.normal_bf16(g, (3, HKV, DH)), 2.0, 50.0)
    plant_v = W.scale_rows(g, W.normal_bf16(g, (3, HKV, DH)), 2.0, 50.0)
    perm = g.permutation(T // BS).astype(np.int64)
    assert T % BS == 0
    dev = "cuda:0"
    reps = (T + nbase - 1) // nbase
    k = to_dev(base_k).repeat(reps, 1, 1)[:T]
    v = to_dev(base_v).repeat(reps, 1, 1)[:T]
    pa = torch.from_numpy(plant_at).to(dev)
    k[pa] = to_dev(plant_k)
    v[pa] = to_dev(plant_v)
    print(f"{T} tokens, planted rows at {plant_at.tolist()}", flush=True)

    f = FMT_ID["e4m3"]
    distinct_k = np.concatenate([base_k, plant_k])
    distinct_v = np.concatenate([base_v, plant_v])
    # per head, K and V in one call
    kam, vam, ks, vs = (torch.empty(HKV, device=dev) for _ in range(4))
    K.kvq_calibrate_scales_kv(k, v, f, oracle.GRAN_HEAD, kam, vam, ks, vs)
    # per tensor
    am1, s1 = torch.empty(1, device=dev), torch.empty(1, device=dev)
    K.kvq_calibrate_scales(v, f, oracle.GRAN_TENSOR, am1, s1)
    torch.cuda.synchronize()
    ka_ref, ks_ref = oracle.calibrate(distinct_k, f, oracle.GRAN_HEAD)
    va_ref, vs_ref = oracle.calibrate(distinct_v, f, oracle.GRAN_HEAD)
    a1_ref, s1_ref = oracle.calibrate(distinct_v, f, oracle.GRAN_TENSOR)
    assert np.array_equal(to_np(kam), ka_ref) and np.array_equal(to_np(ks), ks_ref)
    assert np.array_equal(to_np(vam), va_ref) and np.array_equal(to_np(vs), vs_ref)
    assert np.array_equal(to_np(am1), a1_ref) and np.array_equal(to_np(s1), s1_ref)
    # the planted rows decide some of the maxima
    assert np.any(ka_ref > oracle.calibrate(base_k, f, oracle.GRAN_HEAD)[0])

    # the write: token t goes to slot perm[t / 16] * 16 + t % 16
    t_all = np.arange(T, dtype=np.int64)
    slots = perm[t_all >> 4] * BS + (t_all & (BS - 1))
    del t_all
    kc = torch.empty(oracle.k_cache_shape(T // BS, HKV, BS, DH), dtype=torch.uint8, device=dev)
    vc = torch.empty(oracle.v_cache_shape(T // BS, HKV, BS, DH), dtype=torch.uint8, device=dev)
    K.kvq_cache_write(k, v, to_dev(slots), kc, vc, ks, vs, f, oracle.GRAN_HEAD)
    torch.cuda.synchronize()
    del k, v
    sample = np.unique(np.concatenate([
        [0, 1, nbase - 1, nbase, (1 << 31) // row - 1, (1 << 31) // row, (1 << 32) // row - 1,
         (1 << 32) // row, T - 2], plant_at, W.rng(1501).integers(0, T, 16)])).astype(np.int64)
    is_plant = {int(t): i for i, t in enumerate(plant_at)}
    sk = np.stack([plant_k[is_plant[t]] if t in is_plant else base_k[t % nbase] for t in sample])
    sv = np.stack([plant_v[is_plant[t]] if t in is_plant else base_v[t % nbase] for t in sample])
    n = len(sample)
    off = slots[sample] & (BS - 1)
    kc_ref = np.zeros(oracle.k_cache_shape(n, HKV, BS, DH), np.uint8)
    vc_ref = np.zeros(oracle.v_cache_shape(n, HKV, BS, DH), np.uint8)
    oracle.cache_write(sk, sv, np.arange(n, dtype=np.int64) * BS + off, kc_ref, vc_ref, ks_ref,
                       vs_ref, f, oracle.GRAN_HEAD)
    gk, gv = gather(kc, slots[sample] >> 4), gather(vc, slots[sample] >> 4)
    for i in range(n):
        o = int(off[i])
        assert np.array_equal(gk[i, :, :, o, :], kc_ref[i, :, :, o, :]), f"K of token {sample[i]}"
        assert np.array_equal(gv[i, :, :, o], vc_ref[i, :, :, o]), f"V of token {sample[i]}"
