"""GPU parity of split-K paged decode attention against the oracle.

Bar: max |o - r| / max |r| <= 2e-3 over the whole output and over every
(sequence, head) row, with fp32 output; the bf16 output must be exactly the
fp32 output rounded to nearest even.  Every case first checks the cache bytes
bit-exactly.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import ATTN_TOL, DecodeRun, rel_err, row_rel_err, to_np

pytestmark = pytest.mark.gpu


def run_case(wl, check_cache=True, fill=None):
    run = DecodeRun(wl) if fill is None else DecodeRun(wl, fill=fill)
    run.gpu_scales()
    run.gpu_write()
    kc, vc = run.oracle_caches()
    if check_cache:
        assert np.array_equal(to_np(run.kc), kc) and np.array_equal(to_np(run.vc), vc)
    out = run.gpu_decode()
    ref = oracle.decode_attn(wl.q, kc, vc, wl.paging.block_tables, wl.paging.context_lens,
                             run.ks_ref, run.vs_ref, run.fmt, run.gran)
    return run, out, ref


def check(out, ref):
    e, er = rel_err(out, ref), row_rel_err(out, ref)
    print(f"global rel err {e:.3e}  worst row {er:.3e}", flush=True)
    assert e <= ATTN_TOL and er <= ATTN_TOL


def test_tiny_decode():
    """B=1, Hq=4, Hkv=2, dh=64, context 256 in 16 shuffled blocks, scale 1.0, E4M3."""
    wl = W.tiny_decode()
    _, out, ref = run_case(wl)
    check(out, ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "int8"])
@pytest.mark.parametrize("gran", ["tensor", "head"])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_ragged_batch(fmt, gran, out_dtype):
    """Ragged contexts (1 .. 1500 tokens: partial blocks, partial splits, a
    single-token context) for a Llama-shaped GQA group of 4."""
    cl = [1, 15, 16, 17, 255, 513, 1031, 1500]
    wl = W.decode_workload("ragged", 101, len(cl), 32, 8, 128, cl, 16, fmt, gran,
                           k_outliers=(4, 10.0), v_outliers=(4, 10.0), head_range=(0.5, 20.0))
    run, out, ref = run_case(wl)
    check(out, ref)
    if out_dtype == "bf16":
        # the bf16 output is the fp32 result rounded to nearest even, element by element
        import torch
        run.out = torch.full(run.out.shape, float("nan"), dtype=torch.bfloat16,
                             device=run.out.device)
        assert np.array_equal(run.gpu_decode(), W.f32_to_bf16_bits(out))


@pytest.mark.parametrize("fmt", ["e4m3", "int8"])
@pytest.mark.parametrize("Hq,Hkv,dh", [(8, 8, 128), (16, 8, 64), (12, 4, 128), (64, 8, 128),
                                       (6, 2, 64), (5, 5, 64)])
def test_group_sizes_and_head_dims(Hq, Hkv, dh, fmt):
    cl = [700, 33, 129]
    wl = W.decode_workload("groups", 102 + Hq, len(cl), Hq, Hkv, dh, cl, 16, fmt, "head",
                           head_range=(0.5, 20.0))
    _, out, ref = run_case(wl)
    check(out, ref)


@pytest.mark.parametrize("fmt,fill", [("e4m3", 0xFF), ("e4m3", 0x7F), ("e5m2", 0xFF),
                                      ("e5m2", 0x7C)])
def test_stale_nan_bytes_past_the_context(fmt, fill):
    """Slots of a block past its sequence's context hold NaN (or Inf) codes, as
    a reused pool may: they carry zero weight and must not reach the output."""
    cl = [1, 17, 31, 250, 517, 1029]
    wl = W.decode_workload("stale", 106, len(cl), 32, 8, 128, cl, 16, fmt, "head",
                           head_range=(0.5, 20.0))
    _, out, ref = run_case(wl, fill=fill)
    assert np.all(np.isfinite(out))
    check(out, ref)


def test_zero_length_context_gives_zero_row():
    wl = W.decode_workload("zero", 103, 3, 8, 2, 128, [40, 0, 5], 16, "e4m3", "tensor")
    _, out, ref = run_case(wl)
    assert np.all(out[1] == 0) and np.all(ref[1] == 0)
    check(out, ref)


def test_result_does_not_depend_on_the_split_plan():
    """A larger host bound changes the number of splits; the output stays within rounding."""
    wl = W.decode_workload("plan", 104, 2, 32, 8, 128, [3000, 2000], 16, "e4m3", "tensor")
    run = DecodeRun(wl)
    run.gpu_scales()
    run.gpu_write()
    a = run.gpu_decode()
    b = run.gpu_decode(max_ctx=int(wl.paging.block_tables.shape[1]) * 16)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-5 * np.abs(a).max())


def test_workspace_reuse_across_calls():
    """One workspace, never cleared, serves calls of different shapes and split
    plans; every output equals the output of a call with a fresh workspace."""
    import torch
    import quantized_kv_cache_fp8_amd as K
    runs = [DecodeRun(W.decode_workload("ws-a", 107, 3, 32, 8, 128, [3000, 40, 1700], 16,
                                        "e4m3", "tensor")),
            DecodeRun(W.decode_workload("ws-b", 108, 5, 16, 4, 64, [700, 1, 513, 0, 2222], 16,
                                        "e5m2", "head", head_range=(0.5, 20.0)))]
    for r in runs:
        r.gpu_scales()
        r.gpu_write()
    fresh = [r.gpu_decode() for r in runs]
    big = max(K.kvq_decode_workspace_size(r.wl.B, r.wl.Hq, r.wl.dh,
                                          int(r.wl.paging.block_tables.shape[1]) * 16, 16)
              for r in runs)
    ws = torch.full((big,), 0xFF, dtype=torch.uint8, device="cuda:0")  # NaN-filled
    for rep in range(3):
        for r, want in zip(runs, fresh):
            mc = r.max_ctx if rep != 1 else int(r.wl.paging.block_tables.shape[1]) * 16
            K.kvq_decode_attn(r.out, r.q, r.kc, r.vc, r.bt, r.cl, mc, r.ks, r.vs, r.fmt, r.gran,
                              workspace=ws)
            torch.cuda.synchronize()
            got = to_np(r.out)
            if rep != 1:
                assert np.array_equal(got, want)
            else:
                np.testing.assert_allclose(got, want, rtol=0, atol=1e-5 * np.abs(want).max())


@pytest.mark.parametrize("which", ["llama", "long-e4m3", "long-e5m2", "long-int8"])
def test_full_size_every_row(which):
    """Full-size workloads (the Llama-3-8B-shaped layer; the long-context
    batch with per-head scales): every output row is written (the output
    starts as NaN) and every (sequence, head) row matches the oracle."""
    wl = {"llama": W.llama_layer_decode, "long-e4m3": lambda: W.long_context_decode("e4m3"),
          "long-e5m2": lambda: W.long_context_decode("e5m2"),
          "long-int8": lambda: W.long_context_decode("int8")}[which]()
    print(f"[{which}] B={wl.B} tokens={wl.kv.k.shape[0]}", flush=True)
    run = DecodeRun(wl)
    run.gpu_scales()
    run.gpu_write()
    out = run.gpu_decode()
    assert np.all(np.isfinite(out))
    kc, vc = run.oracle_caches()
    ref = oracle.decode_attn(wl.q, kc, vc, wl.paging.block_tables, wl.paging.context_lens,
                             run.ks_ref, run.vs_ref, run.fmt, run.gran)
    check(out, ref)


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (64, 8)])
def test_explicit_softmax_scale(Hq, Hkv):
    """A caller-given softmax scale in place of 1/sqrt(dh), for both kernels."""
    import torch
    cl = [300, 17, 1029]
    wl = W.decode_workload("decode-sm", 107, len(cl), Hq, Hkv, 128, cl, 16, "e4m3", "head",
                           head_range=(0.5, 4.0))
    run = DecodeRun(wl)
    run.gpu_scales()
    run.gpu_write()
    run.K.kvq_decode_attn(run.out, run.q, run.kc, run.vc, run.bt, run.cl, run.max_ctx, run.ks,
                          run.vs, run.fmt, run.gran, softmax_scale=0.2)
    torch.cuda.synchronize()
    kc, vc = run.oracle_caches()
    ref = oracle.decode_attn(wl.q, kc, vc, wl.paging.block_tables, wl.paging.context_lens,
                             run.ks_ref, run.vs_ref, run.fmt, run.gran, 0.2)
    check(to_np(run.out), ref)

@pytest.mark.parametrize("B,Hq,Hkv,cl", [
    (3, 8, 2, [700, 1, 300]),      # up to 16 splits, 4 | Hq: 4 channels per thread, 4 rows
    (1, 3, 1, [1000]),             # up to 16 splits, 4 does not divide Hq: one row per workgroup
    (2, 3, 1, [2176, 100]),        # 17 splits, B * Hq * nsplit even: lanes, 4 channels per thread
    (1, 3, 1, [2176]),             # 17 splits, B * Hq * nsplit odd: lanes, one channel per thread
])
def test_every_split_merge_form(B, Hq, Hkv, cl):
    """Each form of the split merge, chosen by the split count and the parity of
    B x Hq x nsplit (16-byte aligned partials), against the oracle; the bf16
    output is the fp32 one rounded to nearest even."""
    wl = W.decode_workload("merge-forms", 1800 + B * 10 + Hq, B, Hq, Hkv, 128, cl, 16, "e4m3",
                           "head", k_outliers=(2, 8.0), head_range=(0.5, 20.0))
    run = DecodeRun(wl)
    run.gpu_scales()
    run.gpu_write()
    kc, vc = run.oracle_caches()
    out = run.gpu_decode()
    ref = oracle.decode_attn(wl.q, kc, vc, wl.paging.block_tables, wl.paging.context_lens,
                             run.ks_ref, run.vs_ref, run.fmt, run.gran)
    check(out, ref)
    run16 = DecodeRun(wl, out_dtype="bf16")
    run16.gpu_scales()
    run16.gpu_write()
    assert np.array_equal(run16.gpu_decode(), W.f32_to_bf16_bits(out))
