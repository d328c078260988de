"""Two host threads calling the library at once, each on its own stream (the
serving pattern of one thread per model replica or request queue): the
library's host state (device attributes looked up once per device) is shared,
each call has its own workspace, and the results must equal those of the same
calls made one after the other, bit for bit.  ctypes releases the GIL around
each library call, so the calls really overlap on the host and on the device."""
import threading

import numpy as np
import pytest

import workloads as W
from helpers import DecodeRun, to_np

pytestmark = pytest.mark.gpu


def test_two_threads_two_streams_match_serial():
    import torch
    import quantized_kv_cache_fp8_amd as K
    wls = [W.decode_workload("conc-a", 1900, 8, 32, 8, 128, [3000, 17, 900, 4097, 1, 640, 2222, 50],
                             16, "e4m3", "tensor", k_outliers=(2, 8.0)),
           W.decode_workload("conc-b", 1901, 5, 16, 4, 64, [100, 2500, 1, 777, 1300], 16, "e5m2",
                             "head", head_range=(0.5, 20.0))]
    runs = [DecodeRun(wl) for wl in wls]
    for r in runs:
        r.gpu_scales()
        r.gpu_write()
    serial = [r.gpu_decode() for r in runs]
    streams = [torch.cuda.Stream() for _ in runs]  # default priority
    wss = [torch.empty(K.kvq_decode_workspace_size(r.wl.B, r.wl.Hq, r.wl.dh, r.max_ctx, 16),
                       dtype=torch.uint8, device="cuda:0") for r in runs]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        r, st, ws = runs[i], streams[i], wss[i]
        try:
            for it in range(20):
                with torch.cuda.stream(st):  # the NaN fill and the call on one stream
                    out = torch.full_like(r.out, float("nan"))
                    K.kvq_decode_attn(out, r.q, r.kc, r.vc, r.bt, r.cl, r.max_ctx, r.ks, r.vs,
                                      r.fmt, r.gran, workspace=ws, stream=st.cuda_stream)
                st.synchronize()
                if not np.array_equal(to_np(out), serial[i]):
                    errors.append(f"thread {i}, iteration {it}: output differs from the serial call")
                    return
        except Exception as e:  # reported by the main thread
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(runs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
