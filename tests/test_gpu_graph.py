"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
the library allocates nothing and issues no memsets, so every replay must give
the eager result bit for bit.  Replays alternate with eager work on the same
stream, and each replay is checked; the eager result itself (and the cache the
step leaves) is checked against the oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import ATTN_TOL, rel_err, row_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


def test_append_decode_replays_match_eager():
    import torch
    import quantized_kv_cache_fp8_amd as K
    cl = [33, 700, 1, 2049]
    wl = W.decode_workload("graph", 950, len(cl), 32, 8, 128, cl, 16, "e4m3", "tensor",
                           k_outliers=(4, 10.0))
    k, v = to_dev(wl.kv.k), to_dev(wl.kv.v)
    ks = torch.empty(1, device="cuda:0")
    vs = torch.empty(1, device="cuda:0")
    am = torch.empty(1, device="cuda:0")
    K.kvq_calibrate_scales(k, "e4m3", "tensor", am, ks)
    K.kvq_calibrate_scales(v, "e4m3", "tensor", am, vs)
    offs = wl.kv.seq_offsets
    last = torch.from_numpy((offs[1:] - 1).astype(np.int64)).to("cuda:0")
    kn, vn = k[last].contiguous(), v[last].contiguous()
    kc = torch.full((wl.paging.num_blocks, 8, 8, 16, 16), 0xFF, dtype=torch.uint8,
                    device="cuda:0")
    vc = torch.full((wl.paging.num_blocks, 8, 128, 16), 0xFF, dtype=torch.uint8, device="cuda:0")
    K.kvq_cache_write(k, v, to_dev(wl.kv.slot_mapping), kc, vc, ks, vs, "e4m3", "tensor")
    q, bt, ctx = to_dev(wl.q), to_dev(wl.paging.block_tables), to_dev(wl.paging.context_lens)
    mc = int(max(cl))
    ws = torch.empty(K.kvq_decode_workspace_size(wl.B, wl.Hq, 128, mc, 16), dtype=torch.uint8,
                     device="cuda:0")
    out = torch.full((wl.B, wl.Hq, 128), float("nan"), device="cuda:0")

    def step():
        K.kvq_decode_attn_append(out, q, kn, vn, kc, vc, bt, ctx, mc, ks, vs, "e4m3", "tensor",
                                 workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = to_np(out).copy()
    # the eager step itself against the oracle over every token (the append
    # wrote each sequence's newest one)
    f, gr = oracle.FMT_E4M3, oracle.GRAN_TENSOR
    ks_ref, vs_ref = oracle.calibrate(wl.kv.k, f, gr)[1], oracle.calibrate(wl.kv.v, f, gr)[1]
    assert np.array_equal(to_np(ks), ks_ref) and np.array_equal(to_np(vs), vs_ref)
    kc_ref = np.full(tuple(kc.shape), 0xFF, np.uint8)
    vc_ref = np.full(tuple(vc.shape), 0xFF, np.uint8)
    oracle.cache_write(wl.kv.k, wl.kv.v, wl.kv.slot_mapping, kc_ref, vc_ref, ks_ref, vs_ref, f, gr)
    assert np.array_equal(to_np(kc), kc_ref) and np.array_equal(to_np(vc), vc_ref)
    ref = oracle.decode_attn(wl.q, kc_ref, vc_ref, wl.paging.block_tables,
                             wl.paging.context_lens, ks_ref, vs_ref, f, gr)
    assert rel_err(eager, ref) <= ATTN_TOL and row_rel_err(eager, ref) <= ATTN_TOL
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        out.fill_(float("nan"))
        ws.fill_(0xFF)  # eager work between replays; the partials must be rewritten
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_np(out), eager), f"replay {i}"
        q.mul_(1.0)  # more eager work on the stream
    torch.cuda.synchronize()
