"""Shared helpers for the GPU parity tests: moving seeded inputs to the device,
running the GPU path through the C-ABI binding and the oracle side by side,
and the error metrics the parity bar is stated in."""
from __future__ import annotations

import numpy as np

import oracle

FMT_ID = {"e4m3": oracle.FMT_E4M3, "e5m2": oracle.FMT_E5M2, "int8": oracle.FMT_INT8}
GRAN_ID = {"tensor": oracle.GRAN_TENSOR, "head": oracle.GRAN_HEAD}
SENTINEL = 0xA5

# Attention parity bar: max |o - r| / max |r| over the output tensor (and per
# (token, head) row for decode) must stay within this bound.
ATTN_TOL = 2e-3


def torch_dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype=None):
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    t = t.to(torch_dev())
    return t if dtype is None else t.to(dtype)


def to_np(t) -> np.ndarray:
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max |out - ref| / max |ref| (global)."""
    denom = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(out.astype(np.float64) - ref))) / (denom if denom > 0 else 1.0)


def row_rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max over rows (last axis = channels) of max |o - r| / max |r| of that row."""
    o = out.reshape(-1, out.shape[-1]).astype(np.float64)
    r = ref.reshape(-1, ref.shape[-1])
    den = np.max(np.abs(r), axis=1)
    num = np.max(np.abs(o - r), axis=1)
    ok = den > 0
    worst = float(np.max(num[ok] / den[ok])) if ok.any() else 0.0
    assert np.all(num[~ok] == 0), "a zero reference row must give a zero output row"
    return worst


def k_shape(wl):
    """K cache: [num_blocks][Hkv][dh/16][bs][16] (16-channel chunks, token-major
    inside a chunk)."""
    return oracle.k_cache_shape(wl.paging.num_blocks, wl.Hkv, wl.bs, wl.dh)


def v_shape(wl):
    """V cache: channel-major tiles [num_blocks][Hkv][dh][bs]."""
    return (wl.paging.num_blocks, wl.Hkv, wl.dh, wl.bs)


def same_codes(fmt: int, a: np.ndarray, b: np.ndarray) -> bool:
    """Bytes equal, except that any two NaN codes count as equal."""
    if np.array_equal(a, b):
        return True
    t = oracle.fp8_decode_table(fmt)
    diff = a != b
    return bool(np.all(np.isnan(t[a[diff]]) & np.isnan(t[b[diff]])))


class DecodeRun:
    """One decode workload through the GPU path (calibrate -> write -> decode)
    and the same inputs through the oracle."""

    def __init__(self, wl, out_dtype="f32", fill: int = SENTINEL):
        import torch
        import quantized_kv_cache_fp8_amd as K
        self.wl, self.K = wl, K
        fmt, gran = FMT_ID[wl.fmt], GRAN_ID[wl.gran]
        self.fmt, self.gran = fmt, gran
        dev = torch_dev()
        nh = wl.Hkv if gran == oracle.GRAN_HEAD else 1
        # ---- oracle scales
        if wl.fixed_scale is not None:
            self.ks_ref = np.full(nh, wl.fixed_scale, np.float32)
            self.vs_ref = self.ks_ref.copy()
        else:
            self.ks_ref = oracle.calibrate(wl.kv.k, fmt, gran)[1]
            self.vs_ref = oracle.calibrate(wl.kv.v, fmt, gran)[1]
        # ---- device inputs
        self.k = to_dev(wl.kv.k)
        self.v = to_dev(wl.kv.v)
        self.q = to_dev(wl.q)
        self.slots = to_dev(wl.kv.slot_mapping)
        self.bt = to_dev(wl.paging.block_tables)
        self.cl = to_dev(wl.paging.context_lens)
        # cache bytes no token writes keep this value (a NaN code tests that
        # slots past a context never reach the output)
        self.fill = fill
        self.kc = torch.full(k_shape(wl), fill, dtype=torch.uint8, device=dev)
        self.vc = torch.full(v_shape(wl), fill, dtype=torch.uint8, device=dev)
        self.ks = torch.empty(nh, dtype=torch.float32, device=dev)
        self.vs = torch.empty(nh, dtype=torch.float32, device=dev)
        self.kamax = torch.empty(nh, dtype=torch.float32, device=dev)
        self.vamax = torch.empty(nh, dtype=torch.float32, device=dev)
        odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
        # NaN until written: a row the kernels never write cannot pass as finite
        self.out = torch.full((wl.B, wl.Hq, wl.dh), float("nan"), dtype=odt, device=dev)
        self.max_ctx = int(wl.paging.context_lens.max()) if wl.B else 0

    def gpu_scales(self):
        import torch
        K = self.K
        if self.wl.fixed_scale is not None:
            self.ks.fill_(self.wl.fixed_scale)
            self.vs.fill_(self.wl.fixed_scale)
        else:
            K.kvq_calibrate_scales(self.k, self.fmt, self.gran, self.kamax, self.ks)
            K.kvq_calibrate_scales(self.v, self.fmt, self.gran, self.vamax, self.vs)
        torch.cuda.synchronize()

    def gpu_write(self):
        import torch
        self.K.kvq_cache_write(self.k, self.v, self.slots, self.kc, self.vc, self.ks, self.vs,
                               self.fmt, self.gran)
        torch.cuda.synchronize()

    def gpu_decode(self, max_ctx=None):
        import torch
        self.K.kvq_decode_attn(self.out, self.q, self.kc, self.vc, self.bt, self.cl,
                               self.max_ctx if max_ctx is None else max_ctx, self.ks, self.vs,
                               self.fmt, self.gran)
        torch.cuda.synchronize()
        return to_np(self.out)

    def oracle_caches(self):
        wl = self.wl
        kc = np.full(k_shape(wl), self.fill, np.uint8)
        vc = np.full(v_shape(wl), self.fill, np.uint8)
        oracle.cache_write(wl.kv.k, wl.kv.v, wl.kv.slot_mapping, kc, vc, self.ks_ref, self.vs_ref,
                           self.fmt, self.gran)
        return kc, vc
