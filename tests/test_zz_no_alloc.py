"""The allocation-free decode entry point (kvq_decode_attn_append_noalloc),
for callers that cannot allocate: through the C ABI it must give exactly what
kvq_decode_attn_append gives with a caller-allocated workspace (same kernels:
bit-identical output and cache bytes), on two calls in a row, the second
with a smaller input than the first; sizes beyond the static scratch are
refused before any device work."""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import ATTN_TOL, rel_err, row_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu


def case(wl):
    """Device inputs of one decode step: caches holding every token but each
    sequence's newest, the newest tokens, scales, and the oracle's view."""
    import torch
    import quantized_kv_cache_fp8_amd as K
    from test_gpu_append import prepare
    kc, vc, ks, vs, kn, vn, ns, fmt, gran = prepare(wl)
    return dict(kc=kc, vc=vc, ks=ks, vs=vs, kn=kn, vn=vn, fmt=fmt, gran=gran, q=to_dev(wl.q),
                bt=to_dev(wl.paging.block_tables), cl=to_dev(wl.paging.context_lens),
                mc=int(wl.paging.context_lens.max()))


def run_both(wl):
    import torch
    import quantized_kv_cache_fp8_amd as K
    c = case(wl)
    kc2, vc2 = c["kc"].clone(), c["vc"].clone()
    o_ref = torch.full((wl.B, wl.Hq, wl.dh), float("nan"), device="cuda:0")
    o_new = torch.full_like(o_ref, float("nan"))
    K.kvq_decode_attn_append(o_ref, c["q"], c["kn"], c["vn"], c["kc"], c["vc"], c["bt"], c["cl"],
                             c["mc"], c["ks"], c["vs"], c["fmt"], c["gran"])
    K.kvq_decode_attn_append_noalloc(o_new, c["q"], c["kn"], c["vn"], kc2, vc2, c["bt"], c["cl"],
                                     c["mc"], c["ks"], c["vs"], c["fmt"], c["gran"])
    torch.cuda.synchronize()
    assert np.array_equal(to_np(kc2), to_np(c["kc"])) and np.array_equal(to_np(vc2), to_np(c["vc"]))
    a, b = to_np(o_ref), to_np(o_new)
    assert np.all(np.isfinite(b))
    assert np.array_equal(a, b)
    # and the oracle, to the parity bar, on the caches both calls produced
    ref = oracle.decode_attn(wl.q, to_np(kc2), to_np(vc2), wl.paging.block_tables,
                             wl.paging.context_lens, to_np(c["ks"]), to_np(c["vs"]), c["fmt"],
                             c["gran"])
    assert rel_err(b, ref) <= ATTN_TOL and row_rel_err(b, ref) <= ATTN_TOL


def test_noalloc_equals_the_workspace_call_twice_in_a_row():
    """The headline Llama-3-8B-shaped layer first (B=32, contexts up to
    8192: about 8 MB of partials), then a smaller ragged batch with per-head
    E5M2 scales, whose partials overwrite part of what the first call left."""
    run_both(W.llama_layer_decode())
    cl = [1, 17, 513, 1500, 40]
    run_both(W.decode_workload("noalloc-small", 951, len(cl), 32, 8, 128, cl, 16, "e5m2", "head",
                               head_range=(0.5, 20.0)))


def test_sizes_beyond_the_static_scratch_are_refused():
    import quantized_kv_cache_fp8_amd as K
    B, Hq, dh = 32, 32, 128
    assert K.kvq_decode_workspace_size(B, Hq, dh, 19840, 16) <= K.STATIC_SCRATCH_BYTES
    assert K.kvq_decode_workspace_size(B, Hq, dh, 19841, 16) > K.STATIC_SCRATCH_BYTES
    # the workspace size never shrinks as the context grows, so every longer
    # context is refused too
    assert K.kvq_decode_workspace_size(B, Hq, dh, 20480, 16) > K.STATIC_SCRATCH_BYTES
    L = K.lib()
    FAKE = 0x10000
    args = [FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, 1280, FAKE, B, Hq, 8, dh, 16, 20480,
            FAKE, FAKE, 0, 0, 0.0, None]
    assert L.kvq_decode_attn_append_noalloc(*args) == -7  # KVQ_ERR_SCRATCH, no device work
