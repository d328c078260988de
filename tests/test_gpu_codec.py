"""GPU parity of the device FP8 and INT8 codec against the oracle (bit-exact).

Decode: all 256 codes.  Encode: every one of the 2^32 fp32 bit patterns, in
chunks, through the library's kvq_fp8_encode (the same device codec the cache
kernels inline), compared byte for byte with the oracle's bit-level encoder
(NaN inputs must give a NaN code on both sides).
"""
import numpy as np
import pytest

import oracle
from helpers import same_codes, to_dev, to_np

pytestmark = pytest.mark.gpu
FMTS = [oracle.FMT_E4M3, oracle.FMT_E5M2, oracle.FMT_INT8]


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_all_256_codes(fmt):
    import torch
    import quantized_kv_cache_fp8_amd as K
    codes = to_dev(np.arange(256, dtype=np.uint8))
    out = torch.empty(256, dtype=torch.float32, device=codes.device)
    K.kvq_fp8_decode(codes, fmt, out)
    torch.cuda.synchronize()
    got = to_np(out).astype(np.float64)
    ref = oracle.fp8_decode_table(fmt)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))  # -0 kept


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_every_fp32_pattern(fmt):
    import torch
    import quantized_kv_cache_fp8_amd as K
    chunk = 1 << 28
    step = np.arange(chunk, dtype=np.uint32)
    out = torch.empty(chunk, dtype=torch.uint8, device="cuda:0")
    for i in range(1 << 32 >> 28):
        u = step + np.uint32(i * chunk)
        x = u.view(np.float32)
        xd = to_dev(x)
        K.kvq_fp8_encode(xd, fmt, out)
        torch.cuda.synchronize()
        got = to_np(out)
        ref = oracle.fp8_encode(fmt, x)
        assert same_codes(fmt, got, ref), f"chunk {i}: first diff at {np.flatnonzero(got != ref)[:5]}"
        del xd


@pytest.mark.parametrize("n", [1, 3, 5, 1027, 4097])
def test_encode_ragged_lengths(n):
    import torch
    import quantized_kv_cache_fp8_amd as K
    g = np.random.Generator(np.random.PCG64(n))
    x = (g.standard_normal(n) * 100).astype(np.float32)
    out = torch.full((n + 8,), 0xA5, dtype=torch.uint8, device="cuda:0")
    K.kvq_fp8_encode(to_dev(x), oracle.FMT_E4M3, out[:n])
    torch.cuda.synchronize()
    got = to_np(out)
    assert np.array_equal(got[:n], oracle.fp8_encode(oracle.FMT_E4M3, x))
    assert np.all(got[n:] == 0xA5)  # nothing written past the end


def test_binding_rejects_strided_and_mistyped_tensors():
    """A non-contiguous view or a tensor of the wrong dtype is refused by the
    binding before any launch."""
    import torch
    import quantized_kv_cache_fp8_amd as K
    dev = torch.device("cuda:0")
    x = torch.zeros(16, dtype=torch.float32, device=dev)
    out = torch.zeros(16, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="contiguous"):
        K.kvq_fp8_encode(x[::2], "e4m3", out[:8])
    with pytest.raises(TypeError, match="float32"):
        K.kvq_fp8_encode(x.to(torch.bfloat16), "e4m3", out)
    with pytest.raises(TypeError, match="uint8"):
        K.kvq_fp8_encode(x, "e4m3", out.to(torch.int8))
    K.kvq_fp8_encode(x, "e4m3", out)
    torch.cuda.synchronize()
    assert int(out.sum()) == 0
