"""GPU parity of the FP8-domain causal chunked prefill against the oracle.

The oracle quantizes Q to E4M3 exactly as the kernel does and keeps P exact;
the kernel carries P as two E4M3 terms on FP8 matrix cores.  Bar:
max |o - r| / max |r| <= 2e-3 over the output (per-row error is printed).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import (ATTN_TOL, FMT_ID, SENTINEL, k_shape, rel_err, row_rel_err, to_dev, to_np,
                     v_shape)

pytestmark = pytest.mark.gpu


class PrefillRun:
    def __init__(self, wl, q_gran="head", kv_gran="head", out_dtype="f32", fill=SENTINEL):
        import torch
        import quantized_kv_cache_fp8_amd as K
        self.wl, self.K = wl, K
        self.fmt = FMT_ID[wl.fmt]
        self.qg = oracle.GRAN_HEAD if q_gran == "head" else oracle.GRAN_TENSOR
        self.kg = oracle.GRAN_HEAD if kv_gran == "head" else oracle.GRAN_TENSOR
        # scales: Q always E4M3; K/V in the cache format, calibrated over prefix + chunk
        self.qs_ref = oracle.calibrate(wl.q, oracle.FMT_E4M3, self.qg)[1]
        self.ks_ref = oracle.calibrate(wl.kv.k, self.fmt, self.kg)[1]
        self.vs_ref = oracle.calibrate(wl.kv.v, self.fmt, self.kg)[1]
        dev = torch.device("cuda:0")
        self.q = to_dev(wl.q)
        self.fill = fill
        self.kc = torch.full(k_shape(wl), fill, dtype=torch.uint8, device=dev)
        self.vc = torch.full(v_shape(wl), fill, dtype=torch.uint8, device=dev)
        nq = wl.Hq if self.qg == oracle.GRAN_HEAD else 1
        nk = wl.Hkv if self.kg == oracle.GRAN_HEAD else 1
        self.qs = torch.empty(nq, device=dev)
        self.ks = torch.empty(nk, device=dev)
        self.vs = torch.empty(nk, device=dev)
        amax = torch.empty(max(nq, nk), device=dev)
        k, v = to_dev(wl.kv.k), to_dev(wl.kv.v)
        K.kvq_calibrate_scales(self.q, oracle.FMT_E4M3, self.qg, amax[:nq], self.qs)
        K.kvq_calibrate_scales(k, self.fmt, self.kg, amax[:nk], self.ks)
        K.kvq_calibrate_scales(v, self.fmt, self.kg, amax[:nk], self.vs)
        K.kvq_cache_write(k, v, to_dev(wl.kv.slot_mapping), self.kc, self.vc, self.ks, self.vs,
                          self.fmt, self.kg)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(self.qs), self.qs_ref)
        assert np.array_equal(to_np(self.ks), self.ks_ref)
        self.bt = to_dev(wl.paging.block_tables)
        self.cl = to_dev(wl.paging.context_lens)
        self.cu = to_dev(wl.cu_seqlens)
        odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
        # NaN until written: a tile the kernel never writes cannot pass as finite
        self.out = torch.full((wl.q.shape[0], wl.Hq, wl.dh), float("nan"), dtype=odt,
                              device=dev)
        self.max_q = int(np.diff(wl.cu_seqlens).max())

    def gpu(self, softmax_scale=0.0):
        import torch
        self.K.kvq_prefill_attn(self.out, self.q, self.cu, self.max_q, self.qs, self.qg, self.kc,
                                self.vc, self.bt, self.cl, self.ks, self.vs, self.fmt, self.kg,
                                softmax_scale=softmax_scale)
        torch.cuda.synchronize()
        return to_np(self.out)

    def oracle_caches(self):
        wl = self.wl
        kc = np.full(k_shape(wl), self.fill, np.uint8)
        vc = np.full(v_shape(wl), self.fill, np.uint8)
        oracle.cache_write(wl.kv.k, wl.kv.v, wl.kv.slot_mapping, kc, vc, self.ks_ref, self.vs_ref,
                           self.fmt, self.kg)
        return kc, vc

    def oracle_full(self, softmax_scale=0.0):
        kc, vc = self.oracle_caches()
        wl = self.wl
        return oracle.prefill_attn(wl.q, wl.cu_seqlens, self.qs_ref, self.qg, kc, vc,
                                   wl.paging.block_tables, wl.paging.context_lens, self.ks_ref,
                                   self.vs_ref, self.fmt, self.kg, softmax_scale)


def check(out, ref):
    e, er = rel_err(out, ref), row_rel_err(out, ref)
    print(f"global rel err {e:.3e}  worst row {er:.3e}", flush=True)
    assert e <= ATTN_TOL


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("dh", [128, 64])
def test_small_ragged_chunks(fmt, dh):
    """Chunks shorter than a query tile, an empty prefix, a one-token chunk."""
    wl = W.prefill_workload("small", 201, [20, 0, 16, 100], [13, 9, 1, 40], 8, 2, dh, 16, fmt)
    run = PrefillRun(wl)
    check(run.gpu(), run.oracle_full())


def test_empty_chunk_and_chunk_longer_than_context():
    """A sequence with no new rows between two others, and one whose context
    is shorter than its chunk: its first rows sit at negative positions, see
    no key and come out as zeros (the oracle's empty softmax)."""
    wl = W.prefill_workload("empty", 207, [30, 10, 0], [17, 0, 40], 8, 2, 128, 16, "e4m3")
    wl.paging.context_lens[2] = 25
    run = PrefillRun(wl)
    out = run.gpu()
    ref = run.oracle_full()
    cu = wl.cu_seqlens
    assert np.all(ref[cu[2]:cu[2] + 15] == 0)
    assert np.all(out[cu[2]:cu[2] + 15] == 0)
    check(out, ref)


@pytest.mark.parametrize("fmt,fill", [("e4m3", 0xFF), ("e5m2", 0xFF), ("e5m2", 0x7C)])
def test_stale_nan_bytes_past_the_context(fmt, fill):
    """Slots past each sequence's context hold NaN (or Inf) codes, as a reused
    pool may; the last blocks are partial, so those slots sit inside staged tiles."""
    wl = W.prefill_workload("stale", 206, [20, 0, 5, 100], [13, 9, 1, 40], 8, 2, 128, 16, fmt)
    run = PrefillRun(wl, fill=fill)
    out = run.gpu()
    assert np.all(np.isfinite(out))
    check(out, run.oracle_full())


@pytest.mark.parametrize("q_gran,kv_gran", [("tensor", "tensor"), ("head", "tensor"),
                                            ("tensor", "head")])
def test_scale_granularities(q_gran, kv_gran):
    wl = W.prefill_workload("gran", 202, [300, 77], [200, 130], 32, 8, 128, 16, "e4m3")
    run = PrefillRun(wl, q_gran, kv_gran)
    check(run.gpu(), run.oracle_full())


def test_bf16_output():
    """The bf16 output is the fp32 result rounded to nearest even, element by element."""
    wl = W.prefill_workload("bf16", 203, [64, 31], [96, 50], 16, 4, 128, 16, "e4m3")
    f32 = PrefillRun(wl).gpu()
    check(f32, PrefillRun(wl).oracle_full())
    b16 = PrefillRun(wl, out_dtype="bf16").gpu()
    assert np.array_equal(b16, W.f32_to_bf16_bits(f32))


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_group_sizes(G):
    wl = W.prefill_workload("g", 204 + G, [50, 130], [70, 33], 8 * G if G < 8 else 16, 8 if G < 8 else 2,
                            128, 16, "e4m3")
    run = PrefillRun(wl)
    check(run.gpu(), run.oracle_full())


def test_reduced_chunked_prefill():
    """Two sequences of 512 cached + 512 new tokens at the full head shape."""
    wl = W.fp8_chunked_prefill(B=2, prefix=512, chunk=512)
    run = PrefillRun(wl)
    check(run.gpu(), run.oracle_full())


def workgroup_sample(wl, seed, GT=4, QT=32):
    """One (row, head) pair per workgroup of the prefill grid -- every (sequence,
    32-row query tile, group of GT heads) -- at a seeded row of the tile and a
    seeded head of the group, plus every sequence's first and last row.  The
    kernel's XCD renumbering maps each of these workgroups somewhere, so the
    sample meets every stretch of it."""
    g = W.rng(seed)
    cu = wl.cu_seqlens
    rows = []
    for b in range(len(cu) - 1):
        qlen = int(cu[b + 1] - cu[b])
        if qlen == 0:
            continue
        rows += [(int(cu[b]), 0), (int(cu[b + 1]) - 1, wl.Hq - 1)]
        for qt in range((qlen + QT - 1) // QT):
            r = int(cu[b]) + qt * QT + int(g.integers(min(QT, qlen - qt * QT)))
            for grp in range(wl.Hq // GT):
                rows.append((r, grp * GT + int(g.integers(GT))))
    return np.array(rows, np.int64)


def full_size_check(wl, seed):
    run = PrefillRun(wl)
    out = run.gpu()
    assert np.all(np.isfinite(out)), "some output rows were never written"
    kc, vc = run.oracle_caches()
    rows = workgroup_sample(wl, seed)
    print(f"{len(rows)} sampled (row, head) pairs", flush=True)
    ref = oracle.prefill_rows(rows, wl.q, wl.cu_seqlens, run.qs_ref, run.qg, kc, vc,
                              wl.paging.block_tables, wl.paging.context_lens, run.ks_ref,
                              run.vs_ref, run.fmt, run.kg)
    check(out[rows[:, 0], rows[:, 1]], ref)


def test_full_size_sampled_rows():
    """8 x (4096 cached + 4096 new) tokens, Hq=32, Hkv=8, dh=128: every output
    row is written (the output starts as NaN), and one (row, head) pair per
    workgroup of the grid -- 8192 pairs -- matches the oracle."""
    full_size_check(W.fp8_chunked_prefill(), 66)


def test_ragged_full_size_sampled_rows():
    """The ragged batch of the bench (chunk = prefix, 256 to 4096 tokens, full
    head shape): every row written, one sampled pair per workgroup."""
    full_size_check(W.ragged_chunked_prefill(), 67)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_long_prefix_sampled_rows(fmt):
    """Chunks on top of long cached prefixes, at the full head shape: 32768 and
    20000 cached tokens (hundreds of key tiles per query tile, the running
    maximum raised over a long row) and an empty prefix.  Every row is written,
    and one sampled pair per workgroup matches the oracle."""
    wl = W.prefill_workload(f"long-prefix-{fmt}", 320, [32768, 20000, 0], [512, 1000, 300],
                            Hq=32, Hkv=8, dh=128, fmt=fmt)
    full_size_check(wl, 321)


def test_explicit_softmax_scale():
    """A caller-given softmax scale in place of 1/sqrt(dh)."""
    wl = W.prefill_workload("prefill-sm", 314, [50, 0], [70, 33], Hq=16, Hkv=4)
    run = PrefillRun(wl)
    check(run.gpu(0.05), run.oracle_full(0.05))
