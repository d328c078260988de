"""Seeded sweeps over random shape combinations: decode and prefill against the
oracle, on the same bars as the fixed cases (cache bytes bit-exact; attention
within 2e-3 of the oracle, globally and per (token, head) row for decode).

Each case draws its batch size, head layout, head dimension, format, scale
granularities and context lengths (empty, single-token, block and split
boundaries included) from its own seed, so the combinations differ from the
fixed parametrizations of the other files while staying reproducible.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import ATTN_TOL, DecodeRun, rel_err, row_rel_err, to_np

pytestmark = pytest.mark.gpu

SWEEP_SEED = 7100


def _contexts(g, B, hi):
    """B context lengths: mostly uniform in [1, hi], with block and split edges
    (16, 17, 512, 513) and an occasional empty context mixed in."""
    edges = np.array([0, 1, 15, 16, 17, 511, 512, 513], np.int64)
    cl = g.integers(1, hi + 1, size=B)
    pick = g.random(B) < 0.3
    cl[pick] = edges[g.integers(0, len(edges), size=int(pick.sum()))]
    if cl.max() == 0:
        cl[0] = int(g.integers(1, hi + 1))
    return cl.astype(np.int32)


@pytest.mark.parametrize("case", range(12))
def test_decode_sweep(case):
    g = np.random.default_rng(SWEEP_SEED + case)
    Hkv = int(g.choice([1, 2, 4, 8]))
    G = int(g.choice([1, 2, 3, 4, 6, 8]))
    dh = int(g.choice([64, 128]))
    fmt = str(g.choice(["e4m3", "e5m2", "int8"]))
    gran = str(g.choice(["tensor", "head"]))
    B = int(g.integers(1, 7))
    cl = _contexts(g, B, 2500)
    print(f"case {case}: B={B} Hq={G * Hkv} Hkv={Hkv} dh={dh} {fmt} {gran} ctx={cl.tolist()}",
          flush=True)
    wl = W.decode_workload(f"sweep{case}", SWEEP_SEED + 100 + case, B, G * Hkv, Hkv, dh, cl, 16,
                           fmt, gran, k_outliers=(2, 8.0), v_outliers=(2, 8.0),
                           head_range=(0.5, 20.0))
    run = DecodeRun(wl)
    run.gpu_scales()
    run.gpu_write()
    kc, vc = run.oracle_caches()
    assert np.array_equal(to_np(run.kc), kc) and np.array_equal(to_np(run.vc), vc)
    out = run.gpu_decode()
    ref = oracle.decode_attn(wl.q, kc, vc, wl.paging.block_tables, wl.paging.context_lens,
                             run.ks_ref, run.vs_ref, run.fmt, run.gran)
    assert np.all(np.isfinite(out)), "some output rows were never written"
    e, er = rel_err(out, ref), row_rel_err(out, ref)
    print(f"global rel err {e:.3e}  worst row {er:.3e}", flush=True)
    assert e <= ATTN_TOL and er <= ATTN_TOL


@pytest.mark.parametrize("case", range(6))
def test_prefill_sweep(case):
    from test_gpu_prefill import PrefillRun
    g = np.random.default_rng(SWEEP_SEED + 50 + case)
    Hkv = int(g.choice([2, 4, 8]))
    G = int(g.choice([1, 2, 3, 4, 8]))
    dh = int(g.choice([64, 128]))
    fmt = str(g.choice(["e4m3", "e5m2"]))
    q_gran = str(g.choice(["tensor", "head"]))
    kv_gran = str(g.choice(["tensor", "head"]))
    B = int(g.integers(1, 5))
    prefix = g.integers(0, 600, size=B)
    chunk = g.integers(1, 300, size=B)
    chunk[g.random(B) < 0.2] = 0
    if chunk.max() == 0:
        chunk[0] = 37
    print(f"case {case}: B={B} Hq={G * Hkv} Hkv={Hkv} dh={dh} {fmt} q:{q_gran} kv:{kv_gran} "
          f"prefix={prefix.tolist()} chunk={chunk.tolist()}", flush=True)
    wl = W.prefill_workload(f"psweep{case}", SWEEP_SEED + 150 + case, prefix, chunk,
                            Hq=G * Hkv, Hkv=Hkv, dh=dh, fmt=fmt)
    run = PrefillRun(wl, q_gran=q_gran, kv_gran=kv_gran)
    kc, vc = run.oracle_caches()
    assert np.array_equal(to_np(run.kc), kc) and np.array_equal(to_np(run.vc), vc)
    out = run.gpu()
    ref = run.oracle_full()
    assert np.all(np.isfinite(out)), "some output rows were never written"
    e, er = rel_err(out, ref), row_rel_err(out, ref)
    print(f"global rel err {e:.3e}  worst row {er:.3e}", flush=True)
    assert e <= ATTN_TOL


@pytest.mark.parametrize("case", range(6))
def test_kivi_sweep(case):
    """KIVI 2-bit path: tiles bit-exact, decode within 2e-3 globally and per row,
    over random group counts (none, one, split boundaries), residual lengths
    and capacities, and head layouts."""
    from test_gpu_kivi import gpu_cache, oracle_cache, oracle_decode, run_decode
    g = np.random.default_rng(SWEEP_SEED + 90 + case)
    Hkv = int(g.choice([1, 2, 4, 8]))
    G = int(g.choice([1, 2, 3, 4]))
    B = int(g.integers(1, 6))
    R = int(g.choice([1, 32, 128, 256]))
    qg = g.integers(0, 80, size=B)
    qg[g.random(B) < 0.25] = 0
    qg[g.random(B) < 0.2] = 32  # a split boundary
    rl = g.integers(0, R + 1, size=B)
    if (qg + rl).max() == 0:
        qg[0] = 3
    print(f"case {case}: B={B} Hq={G * Hkv} Hkv={Hkv} R={R} groups={qg.tolist()} "
          f"residual={rl.tolist()}", flush=True)
    wl = W.kivi_workload(f"ksweep{case}", SWEEP_SEED + 190 + case, G * Hkv, Hkv, qg, rl, R=R)
    assert np.array_equal(to_np(gpu_cache(wl)), oracle_cache(wl))
    out = run_decode(wl)
    ref = oracle_decode(wl).reshape(out.shape)
    empty = (qg + rl) == 0
    assert not out[empty].any(), "an empty sequence must give zero rows"
    o, r = out[~empty], ref[~empty]
    e, er = rel_err(o, r), row_rel_err(o, r)
    print(f"global rel err {e:.3e}  worst row {er:.3e}", flush=True)
    assert e <= ATTN_TOL and er <= ATTN_TOL
