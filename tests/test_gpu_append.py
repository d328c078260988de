"""GPU parity of decode with the step's new token appended in the same kernel
(kvq_decode_attn_append) against the two-call path it replaces
(kvq_cache_write of the new tokens, then kvq_decode_attn), and against the
oracle.

Bar: cache bytes and output identical to the two-call path (same codec
arithmetic, same attention arithmetic); output within 2e-3 of the oracle.
Slots not yet written hold NaN codes, the new token's slot included.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import ATTN_TOL, FMT_ID, GRAN_ID, k_shape, rel_err, row_rel_err, to_dev, to_np, v_shape

pytestmark = pytest.mark.gpu


def prepare(wl, fill=0xFF):
    """Device caches holding every token but each sequence's last, scales, and
    the last tokens' K/V / slots."""
    import torch
    import quantized_kv_cache_fp8_amd as K
    fmt, gran = FMT_ID[wl.fmt], GRAN_ID[wl.gran]
    nh = wl.Hkv if gran == oracle.GRAN_HEAD else 1
    k, v = to_dev(wl.kv.k), to_dev(wl.kv.v)
    ks = torch.empty(nh, device="cuda:0")
    vs = torch.empty(nh, device="cuda:0")
    am = torch.empty(nh, device="cuda:0")
    K.kvq_calibrate_scales(k, fmt, gran, am, ks)
    K.kvq_calibrate_scales(v, fmt, gran, am, vs)
    offs = wl.kv.seq_offsets
    last = np.array([offs[b + 1] - 1 for b in range(wl.B) if offs[b + 1] > offs[b]], np.int64)
    slots = wl.kv.slot_mapping.copy()
    slots[last] = -1  # everything but the newest token of each sequence
    kc = torch.full(k_shape(wl), fill, dtype=torch.uint8, device="cuda:0")
    vc = torch.full(v_shape(wl), fill, dtype=torch.uint8, device="cuda:0")
    K.kvq_cache_write(k, v, to_dev(slots), kc, vc, ks, vs, fmt, gran)
    # the new tokens, one per sequence (zeros for sequences without one)
    kn = np.zeros((wl.B, wl.Hkv, wl.dh), np.uint16)
    vn = np.zeros((wl.B, wl.Hkv, wl.dh), np.uint16)
    new_slots = np.full(wl.B, -1, np.int64)
    for b in range(wl.B):
        if offs[b + 1] > offs[b]:
            kn[b], vn[b] = wl.kv.k[offs[b + 1] - 1], wl.kv.v[offs[b + 1] - 1]
            new_slots[b] = wl.kv.slot_mapping[offs[b + 1] - 1]
    torch.cuda.synchronize()
    return kc, vc, ks, vs, to_dev(kn), to_dev(vn), to_dev(new_slots), fmt, gran


def both_paths(wl, out_dtype="f32"):
    import torch
    import quantized_kv_cache_fp8_amd as K
    kc, vc, ks, vs, kn, vn, ns, fmt, gran = prepare(wl)
    kc2, vc2 = kc.clone(), vc.clone()
    q, bt, cl = to_dev(wl.q), to_dev(wl.paging.block_tables), to_dev(wl.paging.context_lens)
    mc = int(wl.paging.context_lens.max())
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    o1 = torch.full((wl.B, wl.Hq, wl.dh), float("nan"), dtype=odt, device="cuda:0")
    o2 = torch.full_like(o1, float("nan"))
    K.kvq_cache_write(kn, vn, ns, kc, vc, ks, vs, fmt, gran)
    K.kvq_decode_attn(o1, q, kc, vc, bt, cl, mc, ks, vs, fmt, gran)
    K.kvq_decode_attn_append(o2, q, kn, vn, kc2, vc2, bt, cl, mc, ks, vs, fmt, gran)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(kc2), to_np(kc)) and np.array_equal(to_np(vc2), to_np(vc))
    return to_np(o1), to_np(o2), to_np(kc), to_np(vc), to_np(ks), to_np(vs)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "int8"])
@pytest.mark.parametrize("gran", ["tensor", "head"])
@pytest.mark.parametrize("Hq,Hkv,dh", [(32, 8, 128), (16, 8, 64), (8, 8, 128), (64, 8, 128),
                                       (24, 4, 64), (32, 2, 128)])
def test_append_equals_write_then_decode(fmt, gran, Hq, Hkv, dh):
    """Ragged contexts put the new token first, last and inside blocks, in the
    first split and in partial last splits."""
    cl = [1, 16, 17, 32, 511, 512, 513, 1500]
    wl = W.decode_workload("append", 930 + Hq + dh, len(cl), Hq, Hkv, dh, cl, 16, fmt, gran,
                           k_outliers=(4, 10.0), head_range=(0.5, 20.0))
    o1, o2, kc, vc, ks, vs = both_paths(wl)
    assert np.array_equal(o1, o2)
    ref = oracle.decode_attn(wl.q, kc, vc, wl.paging.block_tables, wl.paging.context_lens, ks, vs,
                             FMT_ID[fmt], GRAN_ID[gran])
    e, er = rel_err(o2, ref), row_rel_err(o2, ref)
    print(f"global rel err {e:.3e}  worst row {er:.3e}", flush=True)
    assert e <= ATTN_TOL and er <= ATTN_TOL


def test_append_bf16_output_and_empty_sequence():
    cl = [0, 5, 4097]
    wl = W.decode_workload("append-bf16", 940, len(cl), 32, 8, 128, cl, 16, "e4m3", "tensor")
    o1, o2, *_ = both_paths(wl, "bf16")
    assert np.array_equal(o1, o2)
    assert not o2[0].any()  # context 0: nothing appended, a zero row


def test_append_full_size_llama_layer():
    """The Llama-3-8B-shaped layer the benchmark times (B=32, contexts up to 8192)."""
    wl = W.llama_layer_decode()
    o1, o2, *_ = both_paths(wl)
    assert np.array_equal(o1, o2)


def test_append_context_beyond_the_host_bound_writes_nothing():
    """A sequence whose context length exceeds max_context_len attends its
    first max_context_len positions, like kvq_decode_attn, and its new token is
    neither written nor attended: no cache byte changes, in particular not the
    slot at position max_context_len - 1."""
    import torch
    import quantized_kv_cache_fp8_amd as K
    cl = [40, 100, 70]
    wl = W.decode_workload("append-bound", 945, len(cl), 32, 8, 128, cl, 16, "e4m3", "tensor")
    kc, vc, ks, vs, kn, vn, ns, fmt, gran = prepare(wl)
    mc = 99  # below sequence 1's length 100
    kc2, vc2 = kc.clone(), vc.clone()
    kb, vb = to_np(kc), to_np(vc)  # before any call
    q, bt, cl_d = to_dev(wl.q), to_dev(wl.paging.block_tables), to_dev(wl.paging.context_lens)
    o1 = torch.full((wl.B, wl.Hq, wl.dh), float("nan"), device="cuda:0")
    o2 = torch.full_like(o1, float("nan"))
    ns_ref = ns.clone()
    ns_ref[1] = -1  # the two-call path without sequence 1's write
    K.kvq_cache_write(kn, vn, ns_ref, kc, vc, ks, vs, fmt, gran)
    K.kvq_decode_attn(o1, q, kc, vc, bt, cl_d, mc, ks, vs, fmt, gran)
    K.kvq_decode_attn_append(o2, q, kn, vn, kc2, vc2, bt, cl_d, mc, ks, vs, fmt, gran)
    torch.cuda.synchronize()
    ka, va = to_np(kc2), to_np(vc2)
    assert np.array_equal(ka, to_np(kc)) and np.array_equal(va, to_np(vc))
    assert np.array_equal(to_np(o1), to_np(o2))
    # sequence 1: position 98 (= max_context_len - 1) keeps its token's codes,
    # position 99 (its new token's true slot) keeps the fill
    blk = wl.paging.block_tables[1]
    for pos in (98, 99):
        b, off = blk[pos // 16], pos % 16
        assert np.array_equal(ka[b, :, :, off, :], kb[b, :, :, off, :])
        assert np.array_equal(va[b, :, :, off], vb[b, :, :, off])
    b, off = blk[99 // 16], 99 % 16
    assert np.all(ka[b, :, :, off, :] == 0xFF) and np.all(va[b, :, :, off] == 0xFF)
