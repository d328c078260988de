"""Reference CPU oracle for the FP8 paged KV cache (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and the
two share no code: the oracle is plain C (``kvq_oracle.c``, fp64) plus this
ctypes marshalling layer, written from the definitions on the pages:

* "10.4 KV Cache 量化: INT8 基础、KIVI 2-bit、FP8 KV" (KV-cache quantization
  textbook chapter): M_KV formula and worked example (10.4.1), write / read /
  attention equations (10.4.2), granularity and metadata table (10.4.3), FP8
  cast path (10.4.5).
  KIVI's per-channel K / per-token V 2-bit grouping and residual (10.4.4).
* "vLLM FP8 量化 KV Cache 完整指南" (vLLM FP8 KV-cache guide): formats, scale
  shapes per granularity, default scale 1.0, Q quantized in the FP8-domain
  (FA3) attention path.

Every function here is pinned by ``tests/test_oracle_*.py`` to something other
than itself (closed forms, torch's float8 dtypes, worked examples printed on
the pages, brute force, invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "liborc.so")

FMT_E4M3 = 0
FMT_E5M2 = 1
FMT_INT8 = 2  # symmetric INT8: clip(round(x / s), -127, 127)
GRAN_TENSOR = 0
GRAN_HEAD = 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (host only, OpenMP over independent rows)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
             SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_num_threads())


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i32, i64, f32, f64, u8 = (ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double,
                                  ctypes.c_uint8)
        L.orc_f16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_double.restype = f64
        L.orc_scale16_from_amax.argtypes = [i32, f32]
        L.orc_scale16_from_amax.restype = ctypes.c_uint16
        L.orc_cache_write_token.argtypes = [P, P, i64, i32, i32, P, P, P, P, P, i64, i32, i32]
        L.orc_decode_token_rows.argtypes = [P, P, i32, P, P, P, P, P, P, i32, P, i32, i32, i32,
                                            i32, i32, f32]
        L.orc_kivi_group.argtypes = [P, i32, P, P, P]
        L.orc_kivi_k_pos.argtypes = [i32, i32, P, P]
        L.orc_kivi_v_pos.argtypes = [i32, i32, P, P]
        L.orc_kivi_quantize.argtypes = [P, P, i64, i32, P, P, i64]
        L.orc_kivi_dequant_tile.argtypes = [P, P, P]
        L.orc_kivi_decode_rows.argtypes = [P, P, i32, P, P, P, i32, P, P, P, P, i32, i32, i32,
                                           f32]
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = i32
        L.orc_fp8_max.argtypes = [i32]
        L.orc_fp8_max.restype = f64
        L.orc_fp8_decode.argtypes = [i32, u8]
        L.orc_fp8_decode.restype = f64
        L.orc_fp8_encode.argtypes = [i32, f32]
        L.orc_fp8_encode.restype = u8
        L.orc_fp8_encode_many.argtypes = [i32, P, P, i64]
        L.orc_fp8_decode_all.argtypes = [i32, P]
        L.orc_quotient.argtypes = [f32, f32]
        L.orc_quotient.restype = f32
        L.orc_quantize.argtypes = [i32, ctypes.c_uint16, f32]
        L.orc_quantize.restype = u8
        L.orc_quantize_many.argtypes = [i32, P, i64, f32, P]
        L.orc_scale_from_amax.argtypes = [i32, f32]
        L.orc_scale_from_amax.restype = f32
        L.orc_calibrate.argtypes = [P, i64, i32, i32, i32, i32, P, P]
        L.orc_cache_write.argtypes = [P, P, i64, i32, i32, P, P, P, i64, i32, P, P, i32, i32]
        L.orc_decode_attn.argtypes = [P, P, P, P, P, i32, P, i32, i32, i32, i32, i32, P, P, i32,
                                      i32, f32]
        L.orc_decode_rows.argtypes = [P, P, i32, P, P, P, P, i32, P, i32, i32, i32, i32, i32, P,
                                      P, i32, i32, f32]
        L.orc_prefill_attn.argtypes = [P, P, P, P, i32, P, P, P, i32, P, i32, i32, i32, i32, i32,
                                       P, P, i32, i32, f32]
        L.orc_prefill_rows.argtypes = [P, P, i32, P, P, P, i32, P, P, P, i32, P, i32, i32, i32,
                                       i32, i32, P, P, i32, i32, f32]
        L.orc_dense_attn.argtypes = [P, P, P, P, i32, i32, i32, i32, f64]
        L.orc_kv_cache_bytes.argtypes = [i32, i32, i32, i64, i32, i32]
        L.orc_kv_cache_bytes.restype = ctypes.c_uint64
        L.orc_token_head_bytes.argtypes = [i32, i32, i32]
        L.orc_token_head_bytes.restype = ctypes.c_uint64
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    """bf16 data as its uint16 bit pattern (accepts torch bf16 or uint16 numpy)."""
    if isinstance(a, np.ndarray):
        assert a.dtype == np.uint16
        return np.ascontiguousarray(a)
    import torch
    assert a.dtype == torch.bfloat16
    return np.ascontiguousarray(a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


# ---------------------------------------------------------------- codec

def fp8_max(fmt: int) -> float:
    return lib().orc_fp8_max(fmt)


def fp8_decode(fmt: int, code: int) -> float:
    return lib().orc_fp8_decode(fmt, code)


def fp8_decode_table(fmt: int) -> np.ndarray:
    out = np.zeros(256, np.float64)
    lib().orc_fp8_decode_all(fmt, _p(out))
    return out


def fp8_encode(fmt: int, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().orc_fp8_encode_many(fmt, _p(x), _p(out), x.size)
    return out


def quotient(x: float, s: float) -> float:
    return lib().orc_quotient(x, s)


def quantize(fmt: int, x_bf16, s: float) -> np.ndarray:
    x = _u16(x_bf16)
    out = np.empty(x.shape, np.uint8)
    lib().orc_quantize_many(fmt, _p(x), x.size, float(s), _p(out))
    return out


def dequantize(fmt: int, codes: np.ndarray, s) -> np.ndarray:
    """x_hat = s * cast_float(code), exact in fp64."""
    return fp8_decode_table(fmt)[codes] * np.float64(s)


def scale_from_amax(fmt: int, amax: float) -> float:
    return lib().orc_scale_from_amax(fmt, amax)


# ---------------------------------------------------------------- path steps

def calibrate(x_bf16, fmt: int, gran: int):
    """amax and scale over bf16 x [T, H, dh]; returns (amax, scale) fp32 arrays."""
    x = _u16(x_bf16)
    T, H, dh = x.shape
    n = H if gran == GRAN_HEAD else 1
    amax = np.zeros(n, np.float32)
    scale = np.zeros(n, np.float32)
    lib().orc_calibrate(_p(x), T, H, dh, fmt, gran, _p(amax), _p(scale))
    return amax, scale


def k_cache_shape(num_blocks: int, Hkv: int, bs: int, dh: int) -> tuple:
    """K cache: tiles of 16-channel chunks, token-major inside a chunk:
    [num_blocks][Hkv][dh/16][bs][16]."""
    return (num_blocks, Hkv, dh // 16, bs, 16)


def v_cache_shape(num_blocks: int, Hkv: int, bs: int, dh: int) -> tuple:
    """V cache: channel-major tiles [num_blocks][Hkv][dh][bs]."""
    return (num_blocks, Hkv, dh, bs)


def k_token_view(k_cache: np.ndarray) -> np.ndarray:
    """The K cache as [num_blocks][Hkv][bs][dh]: element [blk, h, off, d] is the
    code of channel d of the token in slot off (a copy)."""
    nb, Hkv, nc, bs, w = k_cache.shape
    return k_cache.transpose(0, 1, 3, 2, 4).reshape(nb, Hkv, bs, nc * w)


def _kv_dims(k_cache):
    """(num_blocks, Hkv, bs, dh); the K layout needs dh to be a multiple of 16."""
    nb, Hkv, nc, bs, w = k_cache.shape
    assert w == 16
    return nb, Hkv, bs, nc * w


def cache_write(k_bf16, v_bf16, slot_mapping: np.ndarray, k_cache: np.ndarray,
                v_cache: np.ndarray, k_scale, v_scale, fmt: int, gran: int) -> None:
    """Quantize-write (in place) into uint8 caches: K [num_blocks][Hkv][dh/16][bs][16]
    (16-channel chunks, token-major inside a chunk), V [num_blocks][Hkv][dh][bs]
    (channel-major tiles)."""
    k, v = _u16(k_bf16), _u16(v_bf16)
    T, Hkv, dh = k.shape
    nb, hk, bs, dh2 = _kv_dims(k_cache)
    assert hk == Hkv and dh2 == dh and v_cache.shape == (nb, Hkv, dh, bs)
    sm = np.ascontiguousarray(slot_mapping, np.int64)
    ks = np.ascontiguousarray(k_scale, np.float32)
    vs = np.ascontiguousarray(v_scale, np.float32)
    lib().orc_cache_write(_p(k), _p(v), T, Hkv, dh, _p(sm), _p(k_cache), _p(v_cache), nb, bs,
                          _p(ks), _p(vs), fmt, gran)


def decode_attn(q_bf16, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale, fmt,
                gran, softmax_scale: float = 0.0) -> np.ndarray:
    q = _u16(q_bf16)
    B, Hq, dh = q.shape
    _, Hkv, bs, _ = _kv_dims(k_cache)
    bt = np.ascontiguousarray(block_tables, np.int32)
    cl = np.ascontiguousarray(context_lens, np.int32)
    ks = np.ascontiguousarray(k_scale, np.float32)
    vs = np.ascontiguousarray(v_scale, np.float32)
    out = np.zeros((B, Hq, dh), np.float64)
    lib().orc_decode_attn(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(bt), bt.shape[1], _p(cl),
                          B, Hq, Hkv, dh, bs, _p(ks), _p(vs), fmt, gran, softmax_scale)
    return out


def decode_rows(rows: np.ndarray, q_bf16, k_cache, v_cache, block_tables, context_lens, k_scale,
                v_scale, fmt, gran, softmax_scale: float = 0.0) -> np.ndarray:
    """Decode output for the listed (b, hq) pairs only; returns fp64 [n, dh]."""
    q = _u16(q_bf16)
    B, Hq, dh = q.shape
    _, Hkv, bs, _ = _kv_dims(k_cache)
    rows = np.ascontiguousarray(rows, np.int32).reshape(-1, 2)
    bt = np.ascontiguousarray(block_tables, np.int32)
    cl = np.ascontiguousarray(context_lens, np.int32)
    ks = np.ascontiguousarray(k_scale, np.float32)
    vs = np.ascontiguousarray(v_scale, np.float32)
    out = np.zeros((rows.shape[0], dh), np.float64)
    lib().orc_decode_rows(_p(out), _p(rows), rows.shape[0], _p(q), _p(k_cache), _p(v_cache),
                          _p(bt), bt.shape[1], _p(cl), B, Hq, Hkv, dh, bs, _p(ks), _p(vs), fmt,
                          gran, softmax_scale)
    return out


def prefill_attn(q_bf16, cu_seqlens, q_scale, q_gran, k_cache, v_cache, block_tables,
                 context_lens, k_scale, v_scale, fmt, kv_gran,
                 softmax_scale: float = 0.0) -> np.ndarray:
    q = _u16(q_bf16)
    total, Hq, dh = q.shape
    _, Hkv, bs, _ = _kv_dims(k_cache)
    cu = np.ascontiguousarray(cu_seqlens, np.int32)
    B = cu.shape[0] - 1
    bt = np.ascontiguousarray(block_tables, np.int32)
    cl = np.ascontiguousarray(context_lens, np.int32)
    qs = np.ascontiguousarray(q_scale, np.float32)
    ks = np.ascontiguousarray(k_scale, np.float32)
    vs = np.ascontiguousarray(v_scale, np.float32)
    out = np.zeros((total, Hq, dh), np.float64)
    lib().orc_prefill_attn(_p(out), _p(q), _p(cu), _p(qs), q_gran, _p(k_cache), _p(v_cache),
                           _p(bt), bt.shape[1], _p(cl), B, Hq, Hkv, dh, bs, _p(ks), _p(vs), fmt,
                           kv_gran, softmax_scale)
    return out


def prefill_rows(rows: np.ndarray, q_bf16, cu_seqlens, q_scale, q_gran, k_cache, v_cache,
                 block_tables, context_lens, k_scale, v_scale, fmt, kv_gran,
                 softmax_scale: float = 0.0) -> np.ndarray:
    """Prefill output for the listed (query row, hq) pairs only; fp64 [n, dh]."""
    q = _u16(q_bf16)
    total, Hq, dh = q.shape
    _, Hkv, bs, _ = _kv_dims(k_cache)
    rows = np.ascontiguousarray(rows, np.int64).reshape(-1, 2)
    cu = np.ascontiguousarray(cu_seqlens, np.int32)
    B = cu.shape[0] - 1
    bt = np.ascontiguousarray(block_tables, np.int32)
    cl = np.ascontiguousarray(context_lens, np.int32)
    qs = np.ascontiguousarray(q_scale, np.float32)
    ks = np.ascontiguousarray(k_scale, np.float32)
    vs = np.ascontiguousarray(v_scale, np.float32)
    out = np.zeros((rows.shape[0], dh), np.float64)
    lib().orc_prefill_rows(_p(out), _p(rows), rows.shape[0], _p(q), _p(cu), _p(qs), q_gran,
                           _p(k_cache), _p(v_cache), _p(bt), bt.shape[1], _p(cl), B, Hq, Hkv, dh,
                           bs, _p(ks), _p(vs), fmt, kv_gran, softmax_scale)
    return out


def dense_attn(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, sm: float) -> np.ndarray:
    q = np.ascontiguousarray(q, np.float64)
    k = np.ascontiguousarray(k, np.float64)
    v = np.ascontiguousarray(v, np.float64)
    out = np.zeros_like(q)
    lib().orc_dense_attn(_p(out), _p(q), _p(k), _p(v), q.shape[0], k.shape[0], q.shape[1],
                         int(causal), sm)
    return out


# ---------------------------------------------------------------- arithmetic

def kv_cache_bytes(L: int, B: int, Hkv: int, S: int, dh: int, bits_per_elem: int) -> int:
    return int(lib().orc_kv_cache_bytes(L, B, Hkv, S, dh, bits_per_elem))


def token_head_bytes(dh: int, bits_per_elem: int, scale_bytes: int) -> int:
    return int(lib().orc_token_head_bytes(dh, bits_per_elem, scale_bytes))


# ---------------------------------------------------------------- per-token-head scales

def scale16_from_amax(fmt: int, amax: float) -> int:
    """fp16 bits of fl16(clamp(fl32(amax / fmax), 2^-24, 65504)); 1.0 if amax is 0 or not finite."""
    return int(lib().orc_scale16_from_amax(fmt, amax))


def f16_to_double(bits: int) -> float:
    return lib().orc_f16_to_double(bits)


def scale_cache_shape(num_blocks: int, Hkv: int, bs: int) -> tuple:
    """fp16 per-token-head scales (uint16 bit patterns) [num_blocks][Hkv][bs]."""
    return (num_blocks, Hkv, bs)


def cache_write_token(k_bf16, v_bf16, slot_mapping, k_cache, v_cache, k_scale_cache,
                      v_scale_cache, fmt: int) -> None:
    """Quantize-write with one fp16 scale per (token, head), stored beside the codes."""
    k, v = _u16(k_bf16), _u16(v_bf16)
    T, Hkv, dh = k.shape
    nb, hk, bs, dh2 = _kv_dims(k_cache)
    assert hk == Hkv and dh2 == dh and v_cache.shape == (nb, Hkv, dh, bs)
    assert k_scale_cache.shape == (nb, Hkv, bs) and k_scale_cache.dtype == np.uint16
    assert v_scale_cache.shape == (nb, Hkv, bs) and v_scale_cache.dtype == np.uint16
    sm = np.ascontiguousarray(slot_mapping, np.int64)
    lib().orc_cache_write_token(_p(k), _p(v), T, Hkv, dh, _p(sm), _p(k_cache), _p(v_cache),
                                _p(k_scale_cache), _p(v_scale_cache), nb, bs, fmt)


def decode_token_rows(rows, q_bf16, k_cache, v_cache, k_scale_cache, v_scale_cache,
                      block_tables, context_lens, fmt: int, softmax_scale: float = 0.0):
    """Decode output (fp64 [n, dh]) for the listed (b, hq) rows with per-token-head scales."""
    q = _u16(q_bf16)
    B, Hq, dh = q.shape
    _, Hkv, bs, _ = _kv_dims(k_cache)
    rows = np.ascontiguousarray(rows, np.int32).reshape(-1, 2)
    bt = np.ascontiguousarray(block_tables, np.int32)
    cl = np.ascontiguousarray(context_lens, np.int32)
    out = np.zeros((rows.shape[0], dh), np.float64)
    lib().orc_decode_token_rows(_p(out), _p(rows), rows.shape[0], _p(q), _p(k_cache),
                                _p(v_cache), _p(k_scale_cache), _p(v_scale_cache), _p(bt),
                                bt.shape[1], _p(cl), Hq, Hkv, dh, bs, fmt, softmax_scale)
    return out


# ------------------------------------------------------------------ KIVI 2-bit
KIVI_G = 32        # tokens per K group and per cache block; channels per V group
KIVI_DH = 128
KIVI_TILE = 3072   # bytes per (block, head) tile


def kivi_group(x) -> tuple[int, int, np.ndarray]:
    """(s, z) fp16 bits and 2-bit codes of one set of values (fp32)."""
    x = np.ascontiguousarray(x, np.float32)
    s16, z16 = ctypes.c_uint16(), ctypes.c_uint16()
    codes = np.zeros(x.size, np.uint8)
    lib().orc_kivi_group(_p(x), x.size, ctypes.byref(s16), ctypes.byref(z16), _p(codes))
    return s16.value, z16.value, codes


def kivi_k_pos(t: int, c: int) -> tuple[int, int]:
    b, i = ctypes.c_int(), ctypes.c_int()
    lib().orc_kivi_k_pos(t, c, ctypes.byref(b), ctypes.byref(i))
    return b.value, i.value


def kivi_v_pos(t: int, c: int) -> tuple[int, int]:
    b, i = ctypes.c_int(), ctypes.c_int()
    lib().orc_kivi_v_pos(t, c, ctypes.byref(b), ctypes.byref(i))
    return b.value, i.value


def kivi_cache_shape(num_blocks: int, Hkv: int) -> tuple:
    """uint8 [num_blocks][Hkv][3072]: one 32-token tile per (block, head)."""
    return (num_blocks, Hkv, KIVI_TILE)


def kivi_quantize(k_bf16, v_bf16, group_blocks, cache: np.ndarray) -> None:
    """Quantize whole 32-token groups (k, v bf16 [n_groups * 32, Hkv, 128]) into
    the blocks group_blocks[g] of the KIVI cache."""
    k, v = _u16(k_bf16), _u16(v_bf16)
    T, Hkv, dh = k.shape
    assert dh == KIVI_DH and T % KIVI_G == 0 and v.shape == k.shape
    assert cache.shape[1:] == (Hkv, KIVI_TILE) and cache.dtype == np.uint8
    gb = np.ascontiguousarray(group_blocks, np.int32)
    assert gb.size == T // KIVI_G
    lib().orc_kivi_quantize(_p(k), _p(v), gb.size, Hkv, _p(gb), _p(cache), cache.shape[0])


def kivi_dequant_tile(tile: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """k_hat, v_hat fp64 [32, 128] of one (block, head) tile."""
    t = np.ascontiguousarray(tile, np.uint8)
    assert t.size == KIVI_TILE
    kh = np.zeros((KIVI_G, KIVI_DH))
    vh = np.zeros((KIVI_G, KIVI_DH))
    lib().orc_kivi_dequant_tile(_p(t), _p(kh), _p(vh))
    return kh, vh


def kivi_decode_rows(rows, q_bf16, cache, block_tables, quant_groups, res_k, res_v, res_lens,
                     softmax_scale: float = 0.0) -> np.ndarray:
    """Decode output (fp64 [n, 128]) of the listed (b, hq) rows over a KIVI cache
    plus the bf16 residual (res_k / res_v [B, Hkv, R, 128])."""
    q = _u16(q_bf16)
    B, Hq, dh = q.shape
    rk, rv = _u16(res_k), _u16(res_v)
    _, Hkv, R, _ = rk.shape
    rows = np.ascontiguousarray(rows, np.int32).reshape(-1, 2)
    bt = np.ascontiguousarray(block_tables, np.int32)
    qg = np.ascontiguousarray(quant_groups, np.int32)
    rl = np.ascontiguousarray(res_lens, np.int32)
    c = np.ascontiguousarray(cache, np.uint8)
    out = np.zeros((rows.shape[0], dh), np.float64)
    lib().orc_kivi_decode_rows(_p(out), _p(rows), rows.shape[0], _p(q), _p(c), _p(bt),
                               bt.shape[1], _p(qg), _p(rk), _p(rv), _p(rl), R, Hq, Hkv,
                               softmax_scale)
    return out
