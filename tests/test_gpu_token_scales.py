"""GPU parity of the per-token-head scale path (one fp16 scale per (token, KV
head) for K and for V, the KV-cache quantization textbook's section 10.4.3
granularity) against the oracle.

Bar: codes and fp16 scales bit-exact after the write; decode output within
max |o - r| / max |r| <= 2e-3 over the whole output and over every row.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import ATTN_TOL, FMT_ID, SENTINEL, rel_err, row_rel_err, same_codes, to_dev, to_np

pytestmark = pytest.mark.gpu

FMTS = ["e4m3", "e5m2", "int8"]


def caches(nb, Hkv, bs, dh, fill=SENTINEL, sfill=0xBEEF):
    return (np.full(oracle.k_cache_shape(nb, Hkv, bs, dh), fill, np.uint8),
            np.full(oracle.v_cache_shape(nb, Hkv, bs, dh), fill, np.uint8),
            np.full(oracle.scale_cache_shape(nb, Hkv, bs), sfill, np.uint16),
            np.full(oracle.scale_cache_shape(nb, Hkv, bs), sfill, np.uint16))


def gpu_write(k, v, slots, nb, Hkv, bs, dh, fmt, fill=SENTINEL, sfill=0xBEEF):
    import torch
    import quantized_kv_cache_fp8_amd as K
    kc, vc, ksc, vsc = (to_dev(a) for a in caches(nb, Hkv, bs, dh, fill, sfill))
    ksc, vsc = ksc.view(torch.int16), vsc.view(torch.int16)
    K.kvq_cache_write_token_scales(to_dev(k), to_dev(v), to_dev(slots), kc, vc, ksc, vsc,
                                   FMT_ID[fmt])
    torch.cuda.synchronize()
    return kc, vc, ksc, vsc


def u16(t):
    return to_np(t).view(np.uint16)


# token counts that take the one-pass kernel (<= 512) and the LDS-staged one
CONTEXTS = {"short": [301, 17, 1, 64], "long": [301, 17, 1, 64, 700, 33]}


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dh", [64, 128])
@pytest.mark.parametrize("path", ["short", "long"])
def test_write_matches_oracle(fmt, dh, path):
    """Rows whose magnitudes span 1e-9 .. 1e10 (scales clamped at both ends of
    fp16), all-zero rows, rows holding NaN / Inf, padding and out-of-pool
    slots; token counts that are not multiples of the launch's tiles."""
    g = W.rng(500 + dh)
    Hkv, bs = 3, 16
    paging = W.make_paging(g, CONTEXTS[path], bs)
    kv = W.make_kv(g, paging, Hkv, dh, k_outliers=(3, 20.0))
    k = W.scale_rows(g, kv.k, 1e-9, 1e10)
    v = W.scale_rows(g, kv.v, 1e-9, 1e10)
    k[5] = 0
    v[6, 1] = 0
    k[7, 2, 3] = 0x7FC0  # NaN
    v[8, 0, 9] = 0xFF80  # -Inf
    k[9, 1, :] = 0x0001  # smallest subnormals: scale clamps to 2^-24
    slots = kv.slot_mapping.copy()
    slots[10] = -1
    slots[11] = paging.num_blocks * bs + 3  # outside the pool: skipped
    nb = paging.num_blocks
    kc, vc, ksc, vsc = caches(nb, Hkv, bs, dh)
    oracle.cache_write_token(k, v, slots, kc, vc, ksc, vsc, FMT_ID[fmt])
    gk, gv, gks, gvs = gpu_write(k, v, slots, nb, Hkv, bs, dh, fmt)
    assert np.array_equal(u16(gks), ksc) and np.array_equal(u16(gvs), vsc)
    # NaN inputs may take either NaN code (sign); every other byte is exact
    assert same_codes(FMT_ID[fmt], to_np(gk), kc) and same_codes(FMT_ID[fmt], to_np(gv), vc)
    # the clamps were reached
    used = ksc[ksc != 0xBEEF]
    assert (used == 0x0001).any() and (used == 0x7BFF).any() and (used == 0x3C00).any()


def decode_case(seed, fmt, Hq, Hkv, dh, cl, lo=1e-3, hi=1e3, fill=SENTINEL, sfill=0xBEEF,
                also_bf16=False):
    import torch
    import quantized_kv_cache_fp8_amd as K
    g = W.rng(seed)
    bs = 16
    paging = W.make_paging(g, cl, bs)
    kv = W.make_kv(g, paging, Hkv, dh, k_outliers=(4, 10.0), v_outliers=(4, 10.0))
    k = W.scale_rows(g, kv.k, 0.2, 5.0)  # K rows: moderate spread keeps the softmax soft
    v = W.scale_rows(g, kv.v, lo, hi)
    q = W.normal_bf16(g, (len(cl), Hq, dh))
    nb = paging.num_blocks
    kc, vc, ksc, vsc = caches(nb, Hkv, bs, dh, fill, sfill)
    oracle.cache_write_token(k, v, kv.slot_mapping, kc, vc, ksc, vsc, FMT_ID[fmt])
    gk, gv, gks, gvs = gpu_write(k, v, kv.slot_mapping, nb, Hkv, bs, dh, fmt, fill, sfill)
    assert np.array_equal(to_np(gk), kc) and np.array_equal(u16(gks), ksc)
    max_ctx = int(max(cl))
    outs = []
    for odt in ([torch.float32, torch.bfloat16] if also_bf16 else [torch.float32]):
        out = torch.full((len(cl), Hq, dh), float("nan"), dtype=odt, device="cuda:0")
        K.kvq_decode_attn_token_scales(out, to_dev(q), gk, gv, gks, gvs,
                                       to_dev(paging.block_tables),
                                       to_dev(paging.context_lens), max_ctx, FMT_ID[fmt])
        torch.cuda.synchronize()
        outs.append(to_np(out))
    rows = np.array([(b, h) for b in range(len(cl)) for h in range(Hq)], np.int32)
    ref = oracle.decode_token_rows(rows, q, kc, vc, ksc, vsc, paging.block_tables,
                                   paging.context_lens, FMT_ID[fmt]).reshape(len(cl), Hq, dh)
    if also_bf16:
        # the bf16 output is the fp32 one rounded to nearest even, element by element
        assert np.array_equal(outs[1], W.f32_to_bf16_bits(outs[0]))
    return outs[0], ref


def check(out, ref):
    e, er = rel_err(out, ref), row_rel_err(out, ref)
    print(f"global rel err {e:.3e}  worst row {er:.3e}", flush=True)
    assert e <= ATTN_TOL and er <= ATTN_TOL


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("Hq,Hkv,dh", [(32, 8, 128), (16, 8, 64), (8, 8, 128), (4, 2, 64)])
def test_decode_matches_oracle(fmt, Hq, Hkv, dh):
    """Ragged contexts (partial blocks and splits, one-token context) with V
    rows spanning six decades of magnitude."""
    cl = [1, 15, 17, 255, 600, 1100]
    out, ref = decode_case(600 + Hq + dh, fmt, Hq, Hkv, dh, cl)
    check(out, ref)


def test_decode_bf16_output_and_long_context():
    out, ref = decode_case(610, "e4m3", 32, 8, 128, [4097, 33], also_bf16=True)
    check(out, ref)


@pytest.mark.parametrize("fmt", ["e4m3", "int8"])
def test_decode_extreme_scales(fmt):
    """V rows from 1e-9 (scales at the fp16 floor) to 1e7 (at the fp16 ceiling)."""
    out, ref = decode_case(620, fmt, 16, 4, 128, [300, 77], lo=1e-9, hi=1e7)
    check(out, ref)


def test_stale_nan_codes_and_scales_past_the_context():
    """Slots past a context hold NaN codes and NaN scales: zero weight."""
    out, ref = decode_case(630, "e4m3", 32, 8, 128, [1, 17, 250, 519], fill=0xFF, sfill=0x7E00)
    check(out, ref)
