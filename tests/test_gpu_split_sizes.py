"""GPU parity of decode at the largest split size, 40 cache blocks (640 tokens)
per workgroup, which the plan takes for batches with enough work to fill the
chip.  Each split-kernel instance runs it against the oracle: the generic kernel
for groups of 8 and 16 query heads; the kernel for groups of at most 4 heads,
plain and with the fused append; and its per-token-scale form.

The contexts are ragged.  They include a single token, the 640-token split
boundary on either side, two whole splits, and lengths that end a split after
one block.  Bar as elsewhere: cache bytes bit-exact, attention within 2e-3 of
the oracle, globally and per row.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import ATTN_TOL, DecodeRun, rel_err, row_rel_err, to_np

pytestmark = pytest.mark.gpu

B = 32
EDGES = [1, 639, 640, 641, 656, 1280, 1296]


def contexts(seed, hi):
    cl = W.rng(seed).integers(1, hi + 1, size=B).astype(np.int32)
    cl[:len(EDGES)] = EDGES
    cl[len(EDGES)] = hi
    return cl


def takes_forty_block_splits(Hq, cl):
    """The plan's condition for 40-block splits: ceil(blocks / 40) splits per
    sequence give the grid at least 2048 workgroups of 4 query heads."""
    nb = -(-int(cl.max()) // 16)
    fill = -(-2048 // (B * Hq // 4))
    return -(-nb // 40) >= fill


def check(out, ref):
    assert np.all(np.isfinite(out)), "some output rows were never written"
    e, er = rel_err(out, ref), row_rel_err(out, ref)
    print(f"global rel err {e:.3e}  worst row {er:.3e}", flush=True)
    assert e <= ATTN_TOL and er <= ATTN_TOL


@pytest.mark.parametrize("Hq,Hkv,dh,fmt,gran,hi", [
    (64, 8, 128, "e4m3", "head", 2700),    # generic kernel, 8 heads per group
    (64, 4, 64, "e5m2", "tensor", 2700),   # generic kernel, 16 heads per group
    (32, 8, 128, "int8", "head", 5000),    # groups of 4 heads
    (32, 8, 128, "e4m3", "tensor", 5000),
])
def test_decode_and_append_at_forty_block_splits(Hq, Hkv, dh, fmt, gran, hi):
    from test_gpu_append import both_paths
    cl = contexts(1600 + Hq + dh, hi)
    assert takes_forty_block_splits(Hq, cl)
    wl = W.decode_workload("split40", 1610 + Hq + dh, B, Hq, Hkv, dh, cl, 16, fmt, gran,
                           k_outliers=(2, 8.0), v_outliers=(2, 8.0), head_range=(0.5, 20.0))
    run = DecodeRun(wl)
    run.gpu_scales()
    run.gpu_write()
    kc, vc = run.oracle_caches()
    assert np.array_equal(to_np(run.kc), kc) and np.array_equal(to_np(run.vc), vc)
    out = run.gpu_decode()
    ref = oracle.decode_attn(wl.q, kc, vc, wl.paging.block_tables, wl.paging.context_lens,
                             run.ks_ref, run.vs_ref, run.fmt, run.gran)
    check(out, ref)
    # the fused append of each sequence's newest token (caches compared with
    # the write-then-decode pair inside both_paths)
    o1, o2, *_ = both_paths(wl)
    assert np.array_equal(o1, o2)
    check(o2, ref)


def test_token_scales_at_forty_block_splits():
    from test_gpu_token_scales import check as check_ts
    from test_gpu_token_scales import decode_case
    cl = contexts(1650, 5000)
    assert takes_forty_block_splits(32, cl)
    out, ref = decode_case(1651, "e4m3", 32, 8, 128, list(cl))
    check_ts(out, ref)
