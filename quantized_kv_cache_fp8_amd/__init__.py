"""FP8 paged KV cache with fused-dequant attention for AMD Instinct MI355X (gfx950).

Python binding of the C-ABI library ``libkvq.so`` (declared in
``include/kvq.h``).  The functions here carry the C names and only marshal
arguments: they read sizes off torch tensors, pass device pointers and the
current HIP stream, and raise :class:`KvqError` on a non-zero status.  Every
step of the path runs in the library's HIP kernels; if the library is missing
the import of :func:`lib` fails loudly (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

# enums of include/kvq.h
KVQ_OK = 0
KVQ_FMT_E4M3, KVQ_FMT_E5M2, KVQ_FMT_INT8 = 0, 1, 2
KVQ_SCALE_TENSOR, KVQ_SCALE_HEAD = 0, 1
KVQ_OUT_F32, KVQ_OUT_BF16 = 0, 1

# kv_cache_dtype strings of the vLLM FP8 KV-cache guide ("fp8" is an alias of "fp8_e4m3")
FMT_NAMES = {"fp8": KVQ_FMT_E4M3, "fp8_e4m3": KVQ_FMT_E4M3, "e4m3": KVQ_FMT_E4M3,
             "fp8_e5m2": KVQ_FMT_E5M2, "e5m2": KVQ_FMT_E5M2, "int8": KVQ_FMT_INT8}
GRAN_NAMES = {"tensor": KVQ_SCALE_TENSOR, "head": KVQ_SCALE_HEAD,
              "attn_head": KVQ_SCALE_HEAD}

EXPORTS = ["kvq_strerror", "kvq_kv_cache_bytes", "kvq_fp8_encode", "kvq_fp8_decode",
           "kvq_calibrate_scales", "kvq_cache_write", "kvq_decode_workspace_size",
           "kvq_decode_attn", "kvq_prefill_attn", "kvq_cache_write_token_scales",
           "kvq_decode_attn_token_scales", "kvq_kivi_quantize", "kvq_kivi_decode_workspace_size",
           "kvq_kivi_decode_attn", "kvq_cache_write_paged", "kvq_decode_attn_paged",
           "kvq_prefill_attn_paged", "kvq_layer_skipped", "kvq_layer_index", "kvq_page_bytes",
           "kvq_common_page_bytes", "kvq_decode_attn_append", "kvq_decode_attn_append_noalloc",
           "kvq_calibrate_scales_kv"]

# bytes of the device scratch array of kvq_decode_attn_append_noalloc (KVQ_STATIC_SCRATCH_BYTES)
STATIC_SCRATCH_BYTES = 16 << 20


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status} ({kvq_strerror(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvq.so (build it first with ``python -m quantized_kv_cache_fp8_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run "
                              "`python -m quantized_kv_cache_fp8_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
        sz = ctypes.c_size_t
        L.kvq_strerror.argtypes = [i32]
        L.kvq_strerror.restype = ctypes.c_char_p
        L.kvq_kv_cache_bytes.argtypes = [i32, i32, i32, i64, i32, i32]
        L.kvq_kv_cache_bytes.restype = ctypes.c_uint64
        L.kvq_fp8_encode.argtypes = [i32, P, i64, P, P]
        L.kvq_fp8_decode.argtypes = [i32, P, i64, P, P]
        L.kvq_calibrate_scales.argtypes = [P, i64, i32, i32, i32, i32, P, P, i32, P]
        L.kvq_calibrate_scales_kv.argtypes = [P, P, i64, i32, i32, i32, i32, P, P, P, P, i32, P]
        L.kvq_cache_write.argtypes = [P, P, i64, i32, i32, P, P, P, i64, i32, P, P, i32, i32, P]
        L.kvq_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.kvq_decode_workspace_size.restype = sz
        L.kvq_decode_attn.argtypes = [P, i32, P, P, P, i64, P, i32, P, i32, i32, i32, i32, i32,
                                      i32, P, P, i32, i32, f32, P, sz, P]
        L.kvq_cache_write_token_scales.argtypes = [P, P, i64, i32, i32, P, P, P, P, P, i64, i32,
                                                   i32, P]
        L.kvq_decode_attn_token_scales.argtypes = [P, i32, P, P, P, P, P, i64, P, i32, P, i32, i32,
                                                   i32, i32, i32, i32, i32, f32, P, sz, P]
        L.kvq_kivi_quantize.argtypes = [P, P, i64, i32, i32, P, P, i64, P]
        L.kvq_kivi_decode_workspace_size.argtypes = [i32, i32, i32, i32]
        L.kvq_kivi_decode_workspace_size.restype = sz
        L.kvq_kivi_decode_attn.argtypes = [P, i32, P, P, i64, P, i32, P, i32, P, P, P, i32, i32,
                                           i32, i32, i32, f32, P, sz, P]
        L.kvq_cache_write_paged.argtypes = [P, P, i64, i32, i32, P, P, P, i64, i32, i64, P, P,
                                            i32, i32, P]
        L.kvq_decode_attn_paged.argtypes = [P, i32, P, P, P, i64, P, i32, P, i32, i32, i32, i32,
                                            i32, i64, i32, P, P, i32, i32, f32, P, sz, P]
        L.kvq_prefill_attn_paged.argtypes = [P, i32, P, P, i32, P, i32, P, P, i64, P, i32, P, i32,
                                             i32, i32, i32, i32, i64, P, P, i32, i32, f32, P]
        L.kvq_layer_skipped.argtypes = [i32, i32, P, i32]
        L.kvq_layer_index.argtypes = [ctypes.c_char_p]
        L.kvq_page_bytes.argtypes = [i32, i32, i32, i32]
        L.kvq_page_bytes.restype = ctypes.c_uint64
        L.kvq_common_page_bytes.argtypes = [P, i32, i32, i32, i32]
        L.kvq_common_page_bytes.restype = ctypes.c_uint64
        L.kvq_decode_attn_append.argtypes = [P, i32, P, P, P, P, P, i64, P, i32, P, i32, i32,
                                             i32, i32, i32, i32, P, P, i32, i32, f32, P, sz, P]
        L.kvq_decode_attn_append_noalloc.argtypes = [P, i32, P, P, P, P, P, i64, P, i32, P, i32,
                                                     i32, i32, i32, i32, i32, P, P, i32, i32, f32,
                                                     P]
        L.kvq_prefill_attn.argtypes = [P, i32, P, P, i32, P, i32, P, P, i64, P, i32, P, i32, i32,
                                       i32, i32, i32, P, P, i32, i32, f32, P]
        _lib = L
    return _lib


def _fmt(f) -> int:
    return FMT_NAMES[f] if isinstance(f, str) else int(f)


def _gran(g) -> int:
    return GRAN_NAMES[g] if isinstance(g, str) else int(g)


# dtypes each kind of tensor argument may have (names of torch dtypes)
_KINDS = {"bf16": ("bfloat16",), "u8": ("uint8",), "f32": ("float32",), "i32": ("int32",),
          "i64": ("int64",), "s16": ("int16", "uint16", "float16"),
          "out": ("float32", "bfloat16")}


def _ptr(t, kind: str | None = None, dense: bool = True) -> int | None:
    """Device address of tensor t (None passes NULL, which the library
    rejects where a pointer is required).  t must live on the GPU, be
    contiguous unless dense is False (padded-page cache views, whose layout
    the caller checks), and have a dtype of the given kind."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("kvq: tensor arguments must be on the GPU")
    if dense and not t.is_contiguous():
        raise ValueError("kvq: tensor arguments must be contiguous")
    if kind is not None and t.dtype not in _kind_dtypes(kind):
        raise TypeError(f"kvq: dtype {t.dtype} where {'/'.join(_KINDS[kind])} is expected")
    return t.data_ptr()


_KIND_DTYPES: dict = {}


def _kind_dtypes(kind: str) -> frozenset:
    """The torch dtypes of a kind, built once (the per-call check allocates nothing)."""
    s = _KIND_DTYPES.get(kind)
    if s is None:
        import torch
        s = _KIND_DTYPES[kind] = frozenset(getattr(torch, n) for n in _KINDS[kind])
    return s


def _cache_dims(k_cache, v_cache):
    """(num_blocks, Hkv, bs, dh) of a cache pair: K uint8 [nb, Hkv, dh/16, bs, 16]
    (16-channel chunks, token-major inside a chunk), V uint8 [nb, Hkv, dh, bs]."""
    if k_cache.dim() != 5 or k_cache.shape[4] != 16 or v_cache.dim() != 4:
        raise ValueError("k_cache must be [nb, Hkv, dh/16, bs, 16] and v_cache [nb, Hkv, dh, bs]")
    nb, Hkv, nc, bs, _ = k_cache.shape
    dh = nc * 16
    if tuple(v_cache.shape) != (nb, Hkv, dh, bs):
        raise ValueError(f"v_cache shape {tuple(v_cache.shape)} does not match k_cache "
                         f"{tuple(k_cache.shape)}")
    return nb, Hkv, bs, dh


def _shape(name: str, t, want) -> None:
    """Raise ValueError unless tensor t has exactly the shape want."""
    if tuple(t.shape) != tuple(want):
        raise ValueError(f"kvq: {name} has shape {tuple(t.shape)}, expected {tuple(want)}")


def _rows(name: str, t, dim: int, n: int) -> None:
    """Raise ValueError unless t has `dim` dimensions and at least n rows."""
    if t.dim() != dim or t.shape[0] < n:
        raise ValueError(f"kvq: {name} must have {dim} dimension(s) and at least {n} rows, "
                         f"got shape {tuple(t.shape)}")


def _scales(name: str, t, gran, H: int) -> None:
    """A scale tensor holds one value (per tensor) or H values (per head)."""
    n = H if _gran(gran) == KVQ_SCALE_HEAD else 1
    if t is not None and t.numel() != n:
        raise ValueError(f"kvq: {name} must hold {n} value(s) for this granularity, "
                         f"got {t.numel()}")


def _attn_shapes(out, q, Hkv, dh, block_tables, context_lens, B):
    """Shape checks shared by the decode calls: q [B, Hq, dh] with dh the
    cache's and Hq a multiple of Hkv, out like q, at least B block-table rows
    and context lengths."""
    if q.dim() != 3 or q.shape[2] != dh or q.shape[1] % Hkv:
        raise ValueError(f"kvq: q has shape {tuple(q.shape)}; expected [B, Hq, {dh}] with Hq a "
                         f"multiple of Hkv = {Hkv}")
    _shape("out", out, q.shape)
    _rows("block_tables", block_tables, 2, B)
    _rows("context_lens", context_lens, 1, B)


def _write_shapes(k, v, slot_mapping, Hkv, dh) -> int:
    """k and v [T, Hkv, dh] with the cache's Hkv and dh, slot_mapping [T]; returns T."""
    if k.dim() != 3:
        raise ValueError(f"kvq: k must be [T, Hkv, dh], got shape {tuple(k.shape)}")
    T = k.shape[0]
    _shape("k", k, (T, Hkv, dh))
    _shape("v", v, (T, Hkv, dh))
    _shape("slot_mapping", slot_mapping, (T,))
    return T


def _prefill_shapes(out, q, cu_seqlens_q, q_scale, q_gran, Hkv, dh, block_tables, context_lens,
                    k_scale, v_scale, kv_gran) -> int:
    """Shape checks of the prefill calls; returns B (cu_seqlens_q holds B + 1 offsets)."""
    if q.dim() != 3 or q.shape[2] != dh or q.shape[1] % Hkv:
        raise ValueError(f"kvq: q has shape {tuple(q.shape)}; expected [total_q, Hq, {dh}] with "
                         f"Hq a multiple of Hkv = {Hkv}")
    _shape("out", out, q.shape)
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.shape[0] < 2:
        raise ValueError("kvq: cu_seqlens_q must be [B + 1] with B >= 1")
    B = cu_seqlens_q.shape[0] - 1
    _rows("block_tables", block_tables, 2, B)
    _rows("context_lens", context_lens, 1, B)
    _scales("q_scale", q_scale, q_gran, q.shape[1])
    _scales("k_scale", k_scale, kv_gran, Hkv)
    _scales("v_scale", v_scale, kv_gran, Hkv)
    return B


def _stream(stream) -> int | None:
    if stream is not None:
        return int(stream)
    import torch
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(fn: str, st: int) -> None:
    if st != KVQ_OK:
        raise KvqError(fn, st)


def kvq_strerror(status: int) -> str:
    return lib().kvq_strerror(int(status)).decode()


def kvq_kv_cache_bytes(L: int, B: int, Hkv: int, S: int, dh: int, bits_per_elem: int) -> int:
    return int(lib().kvq_kv_cache_bytes(L, B, Hkv, S, dh, bits_per_elem))


def kvq_fp8_encode(x, fmt, out, stream=None) -> None:
    """out (uint8, same numel) <- saturating RNE codes of fp32 x."""
    if out.numel() != x.numel():
        raise ValueError("kvq: out must have as many elements as x")
    _check("kvq_fp8_encode", lib().kvq_fp8_encode(_fmt(fmt), _ptr(x, "f32"), x.numel(),
                                                  _ptr(out, "u8"), _stream(stream)))


def kvq_fp8_decode(codes, fmt, out, stream=None) -> None:
    """out (fp32, same numel) <- exact values of uint8 codes."""
    if out.numel() != codes.numel():
        raise ValueError("kvq: out must have as many elements as codes")
    _check("kvq_fp8_decode", lib().kvq_fp8_decode(_fmt(fmt), _ptr(codes, "u8"), codes.numel(),
                                                  _ptr(out, "f32"), _stream(stream)))


def kvq_calibrate_scales(x, fmt, gran, amax_io, scale_out, accumulate=False, stream=None) -> None:
    """x: bf16 [T, H, dh]; amax_io / scale_out: fp32 [1] or [H]."""
    if x.dim() != 3:
        raise ValueError(f"kvq: x must be [T, H, dh], got shape {tuple(x.shape)}")
    T, H, dh = x.shape
    _scales("amax_io", amax_io, gran, H)
    _scales("scale_out", scale_out, gran, H)
    _check("kvq_calibrate_scales",
           lib().kvq_calibrate_scales(_ptr(x, "bf16"), T, H, dh, _fmt(fmt), _gran(gran),
                                      _ptr(amax_io, "f32"), _ptr(scale_out, "f32"),
                                      int(bool(accumulate)), _stream(stream)))


def kvq_calibrate_scales_kv(k, v, fmt, gran, k_amax_io, v_amax_io, k_scale_out, v_scale_out,
                            accumulate=False, stream=None) -> None:
    """k, v: bf16 [T, H, dh] of one shape; the four arrays fp32 [1] or [H]."""
    if k.dim() != 3 or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"kvq: k and v must be [T, H, dh] of one shape, got {tuple(k.shape)} "
                         f"and {tuple(v.shape)}")
    T, H, dh = k.shape
    for name, a in (("k_amax_io", k_amax_io), ("v_amax_io", v_amax_io),
                    ("k_scale_out", k_scale_out), ("v_scale_out", v_scale_out)):
        _scales(name, a, gran, H)
    _check("kvq_calibrate_scales_kv",
           lib().kvq_calibrate_scales_kv(_ptr(k, "bf16"), _ptr(v, "bf16"), T, H, dh, _fmt(fmt),
                                         _gran(gran), _ptr(k_amax_io, "f32"),
                                         _ptr(v_amax_io, "f32"), _ptr(k_scale_out, "f32"),
                                         _ptr(v_scale_out, "f32"), int(bool(accumulate)),
                                         _stream(stream)))


def kvq_cache_write(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale, fmt, gran,
                    stream=None) -> None:
    """k, v: bf16 [T, Hkv, dh]; slot_mapping int64 [T]; caches: K uint8
    [nb, Hkv, dh/16, bs, 16], V uint8 [nb, Hkv, dh, bs]."""
    nb, Hkv, bs, dh = _cache_dims(k_cache, v_cache)
    T = _write_shapes(k, v, slot_mapping, Hkv, dh)
    _scales("k_scale", k_scale, gran, Hkv)
    _scales("v_scale", v_scale, gran, Hkv)
    _check("kvq_cache_write",
           lib().kvq_cache_write(_ptr(k, "bf16"), _ptr(v, "bf16"), T, Hkv, dh,
                                 _ptr(slot_mapping, "i64"), _ptr(k_cache, "u8"),
                                 _ptr(v_cache, "u8"), nb, bs, _ptr(k_scale, "f32"),
                                 _ptr(v_scale, "f32"), _fmt(fmt), _gran(gran), _stream(stream)))


def kvq_decode_workspace_size(B: int, Hq: int, dh: int, max_context_len: int, bs: int) -> int:
    return int(lib().kvq_decode_workspace_size(B, Hq, dh, max_context_len, bs))


def kvq_decode_attn(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                    k_scale, v_scale, fmt, gran, softmax_scale=0.0, workspace=None,
                    stream=None) -> None:
    """out: fp32 or bf16 [B, Hq, dh]; q bf16 [B, Hq, dh]; block_tables int32 [B, max_blocks]."""
    import torch
    nb, Hkv, bs, dh = _cache_dims(k_cache, v_cache)
    _attn_shapes(out, q, Hkv, dh, block_tables, context_lens, q.shape[0])
    B, Hq, _ = q.shape
    _scales("k_scale", k_scale, gran, Hkv)
    _scales("v_scale", v_scale, gran, Hkv)
    ws_bytes = kvq_decode_workspace_size(B, Hq, dh, max_context_len, bs)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    out_dt = KVQ_OUT_BF16 if out.dtype == torch.bfloat16 else KVQ_OUT_F32
    _check("kvq_decode_attn",
           lib().kvq_decode_attn(_ptr(out, "out"), out_dt, _ptr(q, "bf16"), _ptr(k_cache, "u8"),
                                 _ptr(v_cache, "u8"), nb, _ptr(block_tables, "i32"),
                                 block_tables.shape[1], _ptr(context_lens, "i32"), B, Hq, Hkv, dh,
                                 bs, int(max_context_len), _ptr(k_scale, "f32"),
                                 _ptr(v_scale, "f32"), _fmt(fmt), _gran(gran),
                                 float(softmax_scale), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))


def _scale_cache_dims(k_scale_cache, v_scale_cache, nb, Hkv, bs):
    want = (nb, Hkv, bs)
    for t in (k_scale_cache, v_scale_cache):
        if tuple(t.shape) != want or t.element_size() != 2:
            raise ValueError(f"scale caches must be 16-bit {want}, got {tuple(t.shape)}")


def kvq_cache_write_token_scales(k, v, slot_mapping, k_cache, v_cache, k_scale_cache,
                                 v_scale_cache, fmt, stream=None) -> None:
    """As kvq_cache_write with one fp16 scale per (token, KV head), computed from
    the row and stored in k_scale_cache / v_scale_cache (16-bit [nb, Hkv, bs])."""
    nb, Hkv, bs, dh = _cache_dims(k_cache, v_cache)
    T = _write_shapes(k, v, slot_mapping, Hkv, dh)
    _scale_cache_dims(k_scale_cache, v_scale_cache, nb, Hkv, bs)
    _check("kvq_cache_write_token_scales",
           lib().kvq_cache_write_token_scales(_ptr(k, "bf16"), _ptr(v, "bf16"), T, Hkv, dh,
                                              _ptr(slot_mapping, "i64"), _ptr(k_cache, "u8"),
                                              _ptr(v_cache, "u8"), _ptr(k_scale_cache, "s16"),
                                              _ptr(v_scale_cache, "s16"), nb, bs, _fmt(fmt),
                                              _stream(stream)))


def kvq_decode_attn_token_scales(out, q, k_cache, v_cache, k_scale_cache, v_scale_cache,
                                 block_tables, context_lens, max_context_len, fmt,
                                 softmax_scale=0.0, workspace=None, stream=None) -> None:
    """kvq_decode_attn over a cache with per-token-head fp16 scales (Hq / Hkv <= 4)."""
    import torch
    nb, Hkv, bs, dh = _cache_dims(k_cache, v_cache)
    _attn_shapes(out, q, Hkv, dh, block_tables, context_lens, q.shape[0])
    B, Hq, _ = q.shape
    _scale_cache_dims(k_scale_cache, v_scale_cache, nb, Hkv, bs)
    ws_bytes = kvq_decode_workspace_size(B, Hq, dh, max_context_len, bs)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    out_dt = KVQ_OUT_BF16 if out.dtype == torch.bfloat16 else KVQ_OUT_F32
    _check("kvq_decode_attn_token_scales",
           lib().kvq_decode_attn_token_scales(_ptr(out, "out"), out_dt, _ptr(q, "bf16"),
                                              _ptr(k_cache, "u8"), _ptr(v_cache, "u8"),
                                              _ptr(k_scale_cache, "s16"),
                                              _ptr(v_scale_cache, "s16"), nb,
                                              _ptr(block_tables, "i32"), block_tables.shape[1],
                                              _ptr(context_lens, "i32"), B, Hq, Hkv, dh, bs,
                                              int(max_context_len), _fmt(fmt),
                                              float(softmax_scale), _ptr(workspace),
                                              workspace.numel() * workspace.element_size(),
                                              _stream(stream)))


def kvq_prefill_attn(out, q, cu_seqlens_q, max_q_len, q_scale, q_gran, k_cache, v_cache,
                     block_tables, context_lens, k_scale, v_scale, fmt, kv_gran,
                     softmax_scale=0.0, stream=None) -> None:
    """out: fp32 or bf16 [total_q, Hq, dh]; q bf16 [total_q, Hq, dh]; cu_seqlens_q int32 [B+1]."""
    import torch
    nb, Hkv, bs, dh = _cache_dims(k_cache, v_cache)
    B = _prefill_shapes(out, q, cu_seqlens_q, q_scale, q_gran, Hkv, dh, block_tables,
                        context_lens, k_scale, v_scale, kv_gran)
    Hq = q.shape[1]
    out_dt = KVQ_OUT_BF16 if out.dtype == torch.bfloat16 else KVQ_OUT_F32
    _check("kvq_prefill_attn",
           lib().kvq_prefill_attn(_ptr(out, "out"), out_dt, _ptr(q, "bf16"),
                                  _ptr(cu_seqlens_q, "i32"), int(max_q_len), _ptr(q_scale, "f32"),
                                  _gran(q_gran), _ptr(k_cache, "u8"), _ptr(v_cache, "u8"), nb,
                                  _ptr(block_tables, "i32"), block_tables.shape[1],
                                  _ptr(context_lens, "i32"), B, Hq, Hkv, dh, bs,
                                  _ptr(k_scale, "f32"), _ptr(v_scale, "f32"), _fmt(fmt),
                                  _gran(kv_gran), float(softmax_scale), _stream(stream)))


KIVI_TILE = 3072  # bytes per (32-token block, head) tile of the 2-bit cache


def kvq_kivi_quantize(k, v, group_blocks, kivi_cache, stream=None) -> None:
    """k, v: bf16 [n_groups * 32, Hkv, 128]; group_blocks int32 [n_groups];
    kivi_cache uint8 [num_blocks, Hkv, 3072]."""
    if k.dim() != 3 or kivi_cache.dim() != 3 or kivi_cache.shape[2] != KIVI_TILE:
        raise ValueError("kvq: k must be [T, Hkv, 128] and kivi_cache [nb, Hkv, 3072]")
    T, Hkv, dh = k.shape
    if T % 32:
        raise ValueError("kvq: k must hold whole 32-token groups")
    _shape("v", v, k.shape)
    _shape("group_blocks", group_blocks, (T // 32,))
    if kivi_cache.shape[1] != Hkv:
        raise ValueError(f"kvq: kivi_cache has {kivi_cache.shape[1]} KV heads, k has {Hkv}")
    _check("kvq_kivi_quantize",
           lib().kvq_kivi_quantize(_ptr(k, "bf16"), _ptr(v, "bf16"), T // 32, Hkv, dh,
                                   _ptr(group_blocks, "i32"), _ptr(kivi_cache, "u8"),
                                   kivi_cache.shape[0], _stream(stream)))


def kvq_kivi_decode_workspace_size(B: int, Hq: int, Hkv: int, max_groups: int) -> int:
    return int(lib().kvq_kivi_decode_workspace_size(B, Hq, Hkv, max_groups))


def kvq_kivi_decode_attn(out, q, kivi_cache, block_tables, quant_groups, max_groups, res_k,
                         res_v, res_lens, softmax_scale=0.0, workspace=None,
                         stream=None) -> None:
    """out: fp32 or bf16 [B, Hq, 128]; q bf16 [B, Hq, 128]; res_k / res_v bf16
    [B, Hkv, R, 128]; quant_groups / res_lens int32 [B]."""
    import torch
    if q.dim() != 3 or res_k.dim() != 4 or kivi_cache.dim() != 3:
        raise ValueError("kvq: q must be [B, Hq, 128], res_k [B, Hkv, R, 128] and kivi_cache "
                         "[nb, Hkv, 3072]")
    B, Hq, dh = q.shape
    _, Hkv, R, _ = res_k.shape
    _shape("res_k", res_k, (B, Hkv, R, dh))
    _shape("res_v", res_v, res_k.shape)
    _shape("out", out, q.shape)
    _shape("kivi_cache", kivi_cache, (kivi_cache.shape[0], Hkv, KIVI_TILE))
    if Hq % Hkv:
        raise ValueError(f"kvq: Hq = {Hq} is not a multiple of Hkv = {Hkv}")
    _rows("block_tables", block_tables, 2, B)
    _rows("quant_groups", quant_groups, 1, B)
    _rows("res_lens", res_lens, 1, B)
    ws_bytes = kvq_kivi_decode_workspace_size(B, Hq, Hkv, max_groups)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    out_dt = KVQ_OUT_BF16 if out.dtype == torch.bfloat16 else KVQ_OUT_F32
    _check("kvq_kivi_decode_attn",
           lib().kvq_kivi_decode_attn(_ptr(out, "out"), out_dt, _ptr(q, "bf16"),
                                      _ptr(kivi_cache, "u8"), kivi_cache.shape[0],
                                      _ptr(block_tables, "i32"), block_tables.shape[1],
                                      _ptr(quant_groups, "i32"), int(max_groups),
                                      _ptr(res_k, "bf16"), _ptr(res_v, "bf16"),
                                      _ptr(res_lens, "i32"), R, B, Hq, Hkv, dh,
                                      float(softmax_scale), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream)))


# ------------------------------------------------------------------ skip-layers, padded pages

def kvq_layer_skipped(layer_index: int, is_sliding_window: bool, skip_list) -> bool:
    """The guide's skip rule: sliding-window layers when "sliding_window" is
    listed, or the layer whose decimal index is listed."""
    arr = (ctypes.c_char_p * max(1, len(skip_list)))(*[str(x).encode() for x in skip_list])
    return bool(lib().kvq_layer_skipped(int(layer_index), int(bool(is_sliding_window)),
                                        ctypes.cast(arr, ctypes.c_void_p), len(skip_list)))


def kvq_layer_index(prefix: str) -> int:
    return int(lib().kvq_layer_index(prefix.encode()))


def kvq_page_bytes(Hkv: int, dh: int, bs: int, bits_per_elem: int) -> int:
    return int(lib().kvq_page_bytes(Hkv, dh, bs, bits_per_elem))


def kvq_common_page_bytes(layer_bits, Hkv: int, dh: int, bs: int) -> int:
    arr = (ctypes.c_int * max(1, len(layer_bits)))(*[int(b) for b in layer_bits])
    return int(lib().kvq_common_page_bytes(ctypes.cast(arr, ctypes.c_void_p), len(layer_bits), Hkv,
                                           dh, bs))


def _paged_dims(k_cache, v_cache):
    """(num_blocks, Hkv, bs, dh, block_stride) of a K/V cache pair that may be
    views into a pool of padded pages: inside a block the tensors must be
    dense; the block stride (bytes) is stride(0), the same for K and V."""
    nb, Hkv, bs, dh = _cache_dims(k_cache, v_cache)
    if (k_cache.stride()[1:] != (dh * bs, 16 * bs, 16, 1)
            or v_cache.stride()[1:] != (dh * bs, bs, 1)):
        raise ValueError("caches must be dense inside each block")
    if k_cache.stride(0) != v_cache.stride(0):
        raise ValueError("k_cache and v_cache must share one block stride")
    return nb, Hkv, bs, dh, k_cache.stride(0)


def kvq_cache_write_paged(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale, fmt, gran,
                          stream=None) -> None:
    """kvq_cache_write on caches whose blocks sit block_stride = k_cache.stride(0)
    bytes apart (views into a pool of padded pages)."""
    nb, Hkv, bs, dh, bst = _paged_dims(k_cache, v_cache)
    T = _write_shapes(k, v, slot_mapping, Hkv, dh)
    _scales("k_scale", k_scale, gran, Hkv)
    _scales("v_scale", v_scale, gran, Hkv)
    _check("kvq_cache_write_paged",
           lib().kvq_cache_write_paged(_ptr(k, "bf16"), _ptr(v, "bf16"), T, Hkv, dh,
                                       _ptr(slot_mapping, "i64"), _ptr(k_cache, "u8", False),
                                       _ptr(v_cache, "u8", False), nb, bs, bst,
                                       _ptr(k_scale, "f32"), _ptr(v_scale, "f32"), _fmt(fmt),
                                       _gran(gran), _stream(stream)))


def kvq_decode_attn_paged(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                          k_scale, v_scale, fmt, gran, softmax_scale=0.0, workspace=None,
                          stream=None) -> None:
    import torch
    nb, Hkv, bs, dh, bst = _paged_dims(k_cache, v_cache)
    _attn_shapes(out, q, Hkv, dh, block_tables, context_lens, q.shape[0])
    B, Hq, _ = q.shape
    _scales("k_scale", k_scale, gran, Hkv)
    _scales("v_scale", v_scale, gran, Hkv)
    ws_bytes = kvq_decode_workspace_size(B, Hq, dh, max_context_len, bs)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    out_dt = KVQ_OUT_BF16 if out.dtype == torch.bfloat16 else KVQ_OUT_F32
    _check("kvq_decode_attn_paged",
           lib().kvq_decode_attn_paged(_ptr(out, "out"), out_dt, _ptr(q, "bf16"),
                                       _ptr(k_cache, "u8", False), _ptr(v_cache, "u8", False), nb,
                                       _ptr(block_tables, "i32"), block_tables.shape[1],
                                       _ptr(context_lens, "i32"), B, Hq, Hkv, dh, bs, bst,
                                       int(max_context_len), _ptr(k_scale, "f32"),
                                       _ptr(v_scale, "f32"), _fmt(fmt), _gran(gran),
                                       float(softmax_scale), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(stream)))


def kvq_prefill_attn_paged(out, q, cu_seqlens_q, max_q_len, q_scale, q_gran, k_cache, v_cache,
                           block_tables, context_lens, k_scale, v_scale, fmt, kv_gran,
                           softmax_scale=0.0, stream=None) -> None:
    import torch
    nb, Hkv, bs, dh, bst = _paged_dims(k_cache, v_cache)
    B = _prefill_shapes(out, q, cu_seqlens_q, q_scale, q_gran, Hkv, dh, block_tables,
                        context_lens, k_scale, v_scale, kv_gran)
    Hq = q.shape[1]
    out_dt = KVQ_OUT_BF16 if out.dtype == torch.bfloat16 else KVQ_OUT_F32
    _check("kvq_prefill_attn_paged",
           lib().kvq_prefill_attn_paged(_ptr(out, "out"), out_dt, _ptr(q, "bf16"),
                                        _ptr(cu_seqlens_q, "i32"), int(max_q_len),
                                        _ptr(q_scale, "f32"), _gran(q_gran),
                                        _ptr(k_cache, "u8", False), _ptr(v_cache, "u8", False), nb,
                                        _ptr(block_tables, "i32"), block_tables.shape[1],
                                        _ptr(context_lens, "i32"), B, Hq, Hkv, dh, bs, bst,
                                        _ptr(k_scale, "f32"), _ptr(v_scale, "f32"), _fmt(fmt),
                                        _gran(kv_gran), float(softmax_scale), _stream(stream)))


def kvq_decode_attn_append(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                           max_context_len, k_scale, v_scale, fmt, gran, softmax_scale=0.0,
                           workspace=None, stream=None) -> None:
    """kvq_decode_attn with the new token (k_new / v_new bf16 [B, Hkv, dh]) quantized
    into position context_lens[b] - 1 by the same kernel."""
    import torch
    nb, Hkv, bs, dh = _cache_dims(k_cache, v_cache)
    _attn_shapes(out, q, Hkv, dh, block_tables, context_lens, q.shape[0])
    B, Hq, _ = q.shape
    _shape("k_new", k_new, (B, Hkv, dh))
    _shape("v_new", v_new, (B, Hkv, dh))
    _scales("k_scale", k_scale, gran, Hkv)
    _scales("v_scale", v_scale, gran, Hkv)
    if workspace is None:
        ws_bytes = kvq_decode_workspace_size(B, Hq, dh, max_context_len, bs)
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    out_dt = KVQ_OUT_BF16 if out.dtype == torch.bfloat16 else KVQ_OUT_F32
    _check("kvq_decode_attn_append",
           lib().kvq_decode_attn_append(_ptr(out, "out"), out_dt, _ptr(q, "bf16"),
                                        _ptr(k_new, "bf16"), _ptr(v_new, "bf16"),
                                        _ptr(k_cache, "u8"), _ptr(v_cache, "u8"), nb,
                                        _ptr(block_tables, "i32"), block_tables.shape[1],
                                        _ptr(context_lens, "i32"), B, Hq, Hkv, dh, bs,
                                        int(max_context_len), _ptr(k_scale, "f32"),
                                        _ptr(v_scale, "f32"), _fmt(fmt), _gran(gran),
                                        float(softmax_scale), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(stream)))


def kvq_decode_attn_append_noalloc(out, q, k_new, v_new, k_cache, v_cache, block_tables,
                                   context_lens, max_context_len, k_scale, v_scale, fmt, gran,
                                   softmax_scale=0.0, stream=None) -> None:
    """kvq_decode_attn_append with its split partials in the library's static
    device scratch: no workspace argument, nothing allocated (for code under
    graph capture or loops that may not allocate).  Calls that overlap on one
    GPU share that scratch and must be ordered by the caller."""
    import torch
    nb, Hkv, bs, dh = _cache_dims(k_cache, v_cache)
    _attn_shapes(out, q, Hkv, dh, block_tables, context_lens, q.shape[0])
    B, Hq, _ = q.shape
    _shape("k_new", k_new, (B, Hkv, dh))
    _shape("v_new", v_new, (B, Hkv, dh))
    _scales("k_scale", k_scale, gran, Hkv)
    _scales("v_scale", v_scale, gran, Hkv)
    out_dt = KVQ_OUT_BF16 if out.dtype == torch.bfloat16 else KVQ_OUT_F32
    _check("kvq_decode_attn_append_noalloc",
           lib().kvq_decode_attn_append_noalloc(
               _ptr(out, "out"), out_dt, _ptr(q, "bf16"), _ptr(k_new, "bf16"),
               _ptr(v_new, "bf16"), _ptr(k_cache, "u8"), _ptr(v_cache, "u8"), nb,
               _ptr(block_tables, "i32"), block_tables.shape[1], _ptr(context_lens, "i32"), B, Hq,
               Hkv, dh, bs, int(max_context_len), _ptr(k_scale, "f32"), _ptr(v_scale, "f32"),
               _fmt(fmt), _gran(gran), float(softmax_scale), _stream(stream)))
