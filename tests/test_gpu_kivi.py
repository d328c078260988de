"""GPU parity of the KIVI-style 2-bit path (the KV-cache quantization
textbook, section 10.4.4) against the oracle.

Bar: the quantized tiles are bit-exact; decode output within
max |o - r| / max |r| <= 2e-3 over the whole output and over every row; the
bf16 output equals the fp32 output rounded to nearest even.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import ATTN_TOL, rel_err, row_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu

FILL = 0x5A


def gpu_cache(wl, fill=FILL):
    import torch
    import quantized_kv_cache_fp8_amd as K
    cache = torch.full(oracle.kivi_cache_shape(wl.paging.num_blocks, wl.Hkv), fill,
                       dtype=torch.uint8, device="cuda:0")
    if len(wl.group_blocks):
        K.kvq_kivi_quantize(to_dev(wl.k), to_dev(wl.v), to_dev(wl.group_blocks), cache)
    torch.cuda.synchronize()
    return cache


def oracle_cache(wl, fill=FILL):
    cache = np.full(oracle.kivi_cache_shape(wl.paging.num_blocks, wl.Hkv), fill, np.uint8)
    if len(wl.group_blocks):
        oracle.kivi_quantize(wl.k, wl.v, wl.group_blocks, cache)
    return cache


def test_quantize_matches_oracle():
    """Groups with outlier channels, constant sets, sets holding NaN / Inf,
    ranges beyond fp16, tiny ranges; skipped and out-of-pool blocks."""
    import torch
    import quantized_kv_cache_fp8_amd as K
    wl = W.kivi_workload("quant", 800, 8, 3, [5, 2, 9], [0, 0, 0])
    k, v = wl.k.copy(), wl.v.copy()
    k[0:32, 0, 7] = W.f32_to_bf16_bits(np.full(32, 1.5, np.float32))       # constant channel
    k[32:64, 1, 3] = W.f32_to_bf16_bits(np.linspace(-3e5, 3e5, 32).astype(np.float32))
    k[64:96, 2, 9] = W.f32_to_bf16_bits(np.float32(1e-4) + np.arange(32, dtype=np.float32) *
                                        np.float32(1e-9))                   # range -> s = 0
    k[100, 0, 50] = 0x7FC0                                                 # NaN in a K set
    v[130, 1, 64:96] = W.f32_to_bf16_bits(np.linspace(-2e6, 1e6, 32).astype(np.float32))
    v[140, 2, 5] = 0xFF80                                                  # -Inf in a V set
    v[150, 0, :] = 0                                                       # zero token
    gb = wl.group_blocks.copy()
    gb[3] = -1
    gb[7] = wl.paging.num_blocks + 4
    wl.k, wl.v, wl.group_blocks = k, v, gb
    ref = oracle_cache(wl)
    got = to_np(gpu_cache(wl))
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} bytes differ, first {bad[:5].tolist()}"
    # tokens must be whole groups; a larger n with the same data rewrites identically
    cache = gpu_cache(wl)
    K.kvq_kivi_quantize(to_dev(wl.k), to_dev(wl.v), to_dev(gb), cache)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(cache), ref)


def run_decode(wl, out_dtype="f32", max_groups=None, fill=FILL):
    import torch
    import quantized_kv_cache_fp8_amd as K
    cache = gpu_cache(wl, fill)
    mg = int(wl.quant_groups.max()) if max_groups is None else max_groups
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = torch.full((wl.B, wl.Hq, 128), float("nan"), dtype=odt, device="cuda:0")
    K.kvq_kivi_decode_attn(out, to_dev(wl.q), cache, to_dev(wl.paging.block_tables),
                           to_dev(wl.quant_groups), mg, to_dev(wl.res_k), to_dev(wl.res_v),
                           to_dev(wl.res_lens))
    torch.cuda.synchronize()
    return to_np(out)


def oracle_decode(wl, rows=None, fill=FILL):
    if rows is None:
        rows = np.array([(b, h) for b in range(wl.B) for h in range(wl.Hq)], np.int32)
    cache = oracle_cache(wl, fill)
    return oracle.kivi_decode_rows(rows, wl.q, cache, wl.paging.block_tables, wl.quant_groups,
                                   wl.res_k, wl.res_v, wl.res_lens)


def check(out, ref):
    e, er = rel_err(out, ref), row_rel_err(out, ref)
    print(f"global rel err {e:.3e}  worst row {er:.3e}", flush=True)
    assert e <= ATTN_TOL and er <= ATTN_TOL


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 4), (6, 6)])
def test_decode_matches_oracle(Hq, Hkv):
    """Ragged quantized lengths (none, one group, partial and several splits)
    and residual lengths (none, one token, partial, full)."""
    wl = W.kivi_workload("ragged", 810 + Hq, Hq, Hkv, [0, 1, 5, 40, 77, 0], [1, 0, 17, 128, 64, 37])
    out = run_decode(wl)
    check(out, oracle_decode(wl).reshape(out.shape))


def test_decode_bf16_output_and_loose_bound():
    """bf16 output = RNE of the fp32 output; a max_groups above every sequence's
    group count changes the split plan (and with more than 16 splits the order
    in which the combine merges them) but not the result beyond that rounding."""
    wl = W.kivi_workload("bf16", 820, 16, 4, [3, 50, 12], [128, 5, 0], max_blocks=70)
    f = run_decode(wl)
    assert np.array_equal(run_decode(wl, "bf16"), W.f32_to_bf16_bits(f))
    np.testing.assert_allclose(run_decode(wl, max_groups=70), f, rtol=0,
                               atol=1e-5 * np.abs(f).max())
    check(f, oracle_decode(wl).reshape(f.shape))


@pytest.mark.parametrize("R", [1, 100, 256])
def test_residual_capacities(R):
    wl = W.kivi_workload("res", 830 + R, 8, 2, [2, 9], [R, R // 2], R=R)
    out = run_decode(wl)
    check(out, oracle_decode(wl).reshape(out.shape))


def test_empty_sequence_gives_zero_row():
    wl = W.kivi_workload("empty", 840, 8, 2, [0, 4], [0, 3])
    out = run_decode(wl)
    assert not out[0].any()
    check(out[1:], oracle_decode(wl)[8:].reshape(out[1:].shape))


def test_full_size_every_row():
    """B=8, Hq=32, Hkv=8, 16384 tokens per sequence (508 groups + 128
    residual): every (sequence, head) row is written (the output starts as
    NaN) and all 256 rows match the oracle."""
    wl = W.kivi_2bit_decode()
    out = run_decode(wl).reshape(-1, 128)
    assert np.all(np.isfinite(out))
    check(out, oracle_decode(wl).reshape(out.shape))
