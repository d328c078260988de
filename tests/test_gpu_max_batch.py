"""GPU parity at the largest batch the attention calls accept: B = 65535
sequences, the grid's z extent (decode, the fused append and prefill), and the
same count for the 2-bit KIVI decode.  Contexts are short and ragged, with
empty sequences among them, so the oracle covers every row.  Bar as elsewhere:
cache bytes bit-exact, attention within 2e-3 of the oracle, globally and per
row; an empty sequence gives a zero row.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import ATTN_TOL, DecodeRun, rel_err, row_rel_err, to_np

pytestmark = pytest.mark.gpu

B_MAX = 65535


def check(out, ref):
    assert np.all(np.isfinite(out)), "some output rows were never written"
    e, er = rel_err(out, ref), row_rel_err(out, ref)
    print(f"global rel err {e:.3e}  worst row {er:.3e}", flush=True)
    assert e <= ATTN_TOL and er <= ATTN_TOL


def short_contexts(seed, hi):
    cl = W.rng(seed).integers(0, hi + 1, size=B_MAX).astype(np.int32)
    cl[:4] = [0, 1, 16, 17]
    cl[-1] = hi
    return cl


def test_decode_and_append_at_the_batch_limit():
    from test_gpu_append import both_paths
    cl = short_contexts(1700, 40)
    wl = W.decode_workload("max-batch", 1701, B_MAX, 8, 2, 64, cl, 16, "e4m3", "head",
                           k_outliers=(2, 8.0), head_range=(0.5, 20.0))
    run = DecodeRun(wl)
    run.gpu_scales()
    run.gpu_write()
    kc, vc = run.oracle_caches()
    assert np.array_equal(to_np(run.kc), kc) and np.array_equal(to_np(run.vc), vc)
    out = run.gpu_decode()
    ref = oracle.decode_attn(wl.q, kc, vc, wl.paging.block_tables, wl.paging.context_lens,
                             run.ks_ref, run.vs_ref, run.fmt, run.gran)
    check(out, ref)
    o1, o2, *_ = both_paths(wl)
    assert np.array_equal(o1, o2)
    check(o2, ref)


def test_kivi_decode_at_the_batch_limit():
    from test_gpu_kivi import gpu_cache, oracle_cache, oracle_decode, run_decode
    g = W.rng(1710)
    qg = g.integers(0, 3, size=B_MAX).astype(np.int32)
    rl = g.integers(0, 5, size=B_MAX).astype(np.int32)
    qg[:3], rl[:3] = [0, 1, 2], [0, 0, 4]
    wl = W.kivi_workload("max-batch-kivi", 1711, 4, 1, qg, rl, R=4)
    assert np.array_equal(to_np(gpu_cache(wl)), oracle_cache(wl))
    out = run_decode(wl)
    ref = oracle_decode(wl).reshape(out.shape)
    empty = (qg + rl) == 0
    assert not out[empty].any(), "an empty sequence must give zero rows"
    check(out[~empty], ref[~empty])


def test_prefill_at_the_batch_limit():
    from test_gpu_prefill import PrefillRun
    g = W.rng(1720)
    prefix = g.integers(0, 30, size=B_MAX)
    chunk = g.integers(0, 4, size=B_MAX)
    chunk[:3] = [1, 0, 3]
    chunk[-1] = 3
    wl = W.prefill_workload("max-batch-prefill", 1721, prefix, chunk, Hq=8, Hkv=2, dh=64,
                            fmt="e4m3")
    run = PrefillRun(wl)
    kc, vc = run.oracle_caches()
    assert np.array_equal(to_np(run.kc), kc) and np.array_equal(to_np(run.vc), vc)
    out = run.gpu()
    ref = run.oracle_full()
    assert np.all(np.isfinite(out)), "some output rows were never written"
    e = rel_err(out, ref)
    print(f"global rel err {e:.3e}  worst row {row_rel_err(out, ref):.3e}", flush=True)
    assert e <= ATTN_TOL
