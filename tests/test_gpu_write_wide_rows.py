"""GPU parity of long writes (more than 512 tokens, the LDS-staged kernel) at
the headline row shapes, where a token's row of all heads holds 1024 values
(Hkv = 8 at dh = 128, Hkv = 16 at dh = 64), against the oracle: cache bytes
(and per-token-head scales) bit-exact.

Slot layouts cover runs of consecutive slots (whole blocks, and partial blocks
where a write starts or ends inside a block, as a chunked prefill continuing a
cached prefix does) and scattered slots (every token its own block, as in a
decode step of many sequences), with padding and out-of-pool slots.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import FMT_ID, SENTINEL, same_codes, to_dev, to_np
from test_gpu_write_calibrate import ALL_BF16, SCALES

pytestmark = pytest.mark.gpu

FMTS = ["e4m3", "e5m2", "int8"]
SHORT_WRITE = 512  # longer writes take the LDS-staged kernels
SHAPES = {128: 8, 64: 16}  # dh -> Hkv with 1024 values per token row


def pad_long(k, v, slots):
    """Pad a write with skipped tokens (slot -1) past the one-pass kernel's size."""
    if k.shape[0] > SHORT_WRITE:
        return k, v, slots
    n = SHORT_WRITE + 1 - k.shape[0]
    z = np.zeros((n,) + k.shape[1:], np.uint16)
    return (np.concatenate([k, z]), np.concatenate([v, z]),
            np.concatenate([slots, np.full(n, -1, np.int64)]))


def gpu_write(k, v, slots, nb, Hkv, dh, ks, vs, fmt, gran):
    import torch
    import quantized_kv_cache_fp8_amd as K
    kc = torch.full(oracle.k_cache_shape(nb, Hkv, 16, dh), SENTINEL, dtype=torch.uint8,
                    device="cuda:0")
    vc = torch.full(oracle.v_cache_shape(nb, Hkv, 16, dh), SENTINEL, dtype=torch.uint8,
                    device="cuda:0")
    K.kvq_cache_write(to_dev(k), to_dev(v), to_dev(slots), kc, vc,
                      to_dev(np.asarray(ks, np.float32)), to_dev(np.asarray(vs, np.float32)),
                      fmt, gran)
    torch.cuda.synchronize()
    return to_np(kc), to_np(vc)


def oracle_write(k, v, slots, nb, Hkv, dh, ks, vs, fmt, gran):
    kc = np.full(oracle.k_cache_shape(nb, Hkv, 16, dh), SENTINEL, np.uint8)
    vc = np.full(oracle.v_cache_shape(nb, Hkv, 16, dh), SENTINEL, np.uint8)
    oracle.cache_write(k, v, slots, kc, vc, np.asarray(ks, np.float32),
                       np.asarray(vs, np.float32), fmt, gran)
    return kc, vc


def chunked_tokens(seed, Hkv, dh, contexts):
    """Sequences in shuffled 16-slot blocks, each written from a random token
    onwards (as a chunked prefill continues a cached prefix), so its first run
    starts inside a block; a padding token and an out-of-pool slot mixed in."""
    g = W.rng(seed)
    paging = W.make_paging(g, contexts, 16)
    kv = W.make_kv(g, paging, Hkv, dh, k_outliers=(4, 10.0), head_range=(0.5, 20.0))
    keep, start = [], 0
    for c in contexts:
        o = int(g.integers(0, max(1, c // 2)))
        keep.extend(range(start + o, start + c))
        start += c
    keep = np.asarray(keep)
    k, v, slots = kv.k[keep].copy(), kv.v[keep].copy(), kv.slot_mapping[keep].copy()
    slots[len(slots) // 3] = -1
    slots[len(slots) // 2] = paging.num_blocks * 16 + 5
    return k, v, slots, paging.num_blocks


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("gran", ["tensor", "head"])
def test_every_bf16_input_every_scale(fmt, gran):
    """All 65536 bf16 patterns as K (and reversed as V) in 64 tokens of 8 x 128,
    written from slot 5 (a partial first block, whole blocks, a partial last
    one), for every scale of the write tests (per head: eight of them in turn)."""
    k = ALL_BF16.reshape(64, 8, 128)
    v = ALL_BF16[::-1].copy().reshape(64, 8, 128)
    slots = np.arange(5, 69, dtype=np.int64)
    kp, vp, sp = pad_long(k, v, slots)
    f = FMT_ID[fmt]
    gid = oracle.GRAN_HEAD if gran == "head" else oracle.GRAN_TENSOR
    for i in range(0, len(SCALES), 8 if gran == "head" else 1):
        sc = [np.float32(SCALES[(i + j) % len(SCALES)]) for j in range(8 if gran == "head" else 1)]
        gk, gv = gpu_write(kp, vp, sp, 6, 8, 128, sc, sc[::-1], f, gid)
        rk, rv = oracle_write(k, v, slots, 6, 8, 128, sc, sc[::-1], f, gid)
        assert same_codes(f, gk, rk), f"K differs at scales {sc!r}"
        assert same_codes(f, gv, rv), f"V differs at scales {sc!r}"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dh", [128, 64])
@pytest.mark.parametrize("gran", ["tensor", "head"])
def test_runs_of_chunked_sequences(fmt, dh, gran):
    Hkv = SHAPES[dh]
    k, v, slots, nb = chunked_tokens(700 + dh, Hkv, dh, [300, 17, 1, 64, 700, 33, 129])
    assert k.shape[0] > SHORT_WRITE
    f = FMT_ID[fmt]
    gid = oracle.GRAN_HEAD if gran == "head" else oracle.GRAN_TENSOR
    n = Hkv if gran == "head" else 1
    ks = oracle.calibrate(k, f, gid)[1][:n]
    vs = oracle.calibrate(v, f, gid)[1][:n]
    gk, gv = gpu_write(k, v, slots, nb, Hkv, dh, ks, vs, f, gid)
    rk, rv = oracle_write(k, v, slots, nb, Hkv, dh, ks, vs, f, gid)
    assert np.array_equal(gk, rk) and np.array_equal(gv, rv)
    assert (gk == SENTINEL).any()  # the skipped slots stay untouched


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dh", [128, 64])
def test_scattered_slots(fmt, dh):
    """Every token in its own slot of a random block, with padding and
    out-of-pool slots; then a mapping where runs of random length 1..16 at
    random offsets of distinct blocks follow one another."""
    Hkv = SHAPES[dh]
    g = W.rng(720 + dh)
    T, nb = 700, 90
    k = W.normal_bf16(g, (T, Hkv, dh))
    v = W.normal_bf16(g, (T, Hkv, dh))
    slots = g.permutation(nb * 16)[:T].astype(np.int64)
    slots[g.choice(T, 20, replace=False)] = -1
    slots[3] = nb * 16 + 1
    f = FMT_ID[fmt]
    gk, gv = gpu_write(k, v, slots, nb, Hkv, dh, [0.03], [0.02], f, oracle.GRAN_TENSOR)
    rk, rv = oracle_write(k, v, slots, nb, Hkv, dh, [0.03], [0.02], f, oracle.GRAN_TENSOR)
    assert np.array_equal(gk, rk) and np.array_equal(gv, rv)
    # runs of random lengths at random offsets of distinct blocks
    slots, t = np.full(T, -1, np.int64), 0
    blocks = g.permutation(nb)
    for b in blocks:
        o = int(g.integers(0, 16))
        n = min(int(g.integers(1, 17 - o)), T - t)
        slots[t:t + n] = b * 16 + o + np.arange(n)
        t += n
        if t >= T:
            break
    gk, gv = gpu_write(k, v, slots, nb, Hkv, dh, [0.03], [0.02], f, oracle.GRAN_TENSOR)
    rk, rv = oracle_write(k, v, slots, nb, Hkv, dh, [0.03], [0.02], f, oracle.GRAN_TENSOR)
    assert np.array_equal(gk, rk) and np.array_equal(gv, rv)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dh", [128, 64])
@pytest.mark.parametrize("layout", ["chunked", "scattered"])
def test_per_token_head_scales(fmt, dh, layout):
    """One fp16 scale per (token, head): codes and scales bit-exact, rows
    spanning 1e-9 .. 1e10, zero rows, NaN and Inf."""
    import torch
    import quantized_kv_cache_fp8_amd as K
    Hkv = SHAPES[dh]
    if layout == "chunked":
        k, v, slots, nb = chunked_tokens(740 + dh, Hkv, dh, [300, 17, 1, 64, 300, 33])
    else:
        g = W.rng(750 + dh)
        nb = 60
        k = W.normal_bf16(g, (600, Hkv, dh))
        v = W.normal_bf16(g, (600, Hkv, dh))
        slots = g.permutation(nb * 16)[:600].astype(np.int64)
    g = W.rng(760 + dh)
    k = W.scale_rows(g, k, 1e-9, 1e10)
    v = W.scale_rows(g, v, 1e-9, 1e10)
    k[5] = 0
    k[7, 2, 3] = 0x7FC0  # NaN
    v[8, 0, 9] = 0xFF80  # -Inf
    f = FMT_ID[fmt]
    kc = np.full(oracle.k_cache_shape(nb, Hkv, 16, dh), SENTINEL, np.uint8)
    vc = np.full(oracle.v_cache_shape(nb, Hkv, 16, dh), SENTINEL, np.uint8)
    ksc = np.full(oracle.scale_cache_shape(nb, Hkv, 16), 0xBEEF, np.uint16)
    vsc = ksc.copy()
    gkc, gvc = to_dev(kc), to_dev(vc)
    gks, gvs = to_dev(ksc).view(torch.int16), to_dev(vsc).view(torch.int16)
    K.kvq_cache_write_token_scales(to_dev(k), to_dev(v), to_dev(slots), gkc, gvc, gks, gvs, f)
    torch.cuda.synchronize()
    oracle.cache_write_token(k, v, slots, kc, vc, ksc, vsc, f)
    assert np.array_equal(to_np(gks).view(np.uint16), ksc)
    assert np.array_equal(to_np(gvs).view(np.uint16), vsc)
    assert same_codes(f, to_np(gkc), kc) and same_codes(f, to_np(gvc), vc)


def test_padded_pages():
    """Writing into padded pages (block stride above the layer's own bytes) at
    Hkv = 8: codes bit-exact, the padding and other layers untouched."""
    from test_gpu_paged import FILL, make_pool, write_layer
    wl = W.decode_workload("paged8", 930, 3, 32, 8, 128, [17, 600, 129], 16, "e4m3", "head",
                           k_outliers=(4, 10.0))
    pool, page, skipped = make_pool(wl)
    nat = wl.Hkv * 16 * wl.dh
    for layer, fmt in ((0, "e4m3"), (2, "e5m2")):
        kc, vc, ks, vs = write_layer(wl, pool, layer, page, fmt)
        rk = np.full(oracle.k_cache_shape(wl.paging.num_blocks, wl.Hkv, 16, wl.dh), FILL, np.uint8)
        rv = np.full(oracle.v_cache_shape(wl.paging.num_blocks, wl.Hkv, 16, wl.dh), FILL, np.uint8)
        oracle.cache_write(wl.kv.k, wl.kv.v, wl.kv.slot_mapping, rk, rv, to_np(ks), to_np(vs),
                           FMT_ID[fmt], oracle.GRAN_HEAD)
        assert same_codes(FMT_ID[fmt], to_np(kc), rk) and same_codes(FMT_ID[fmt], to_np(vc), rv)
    p = to_np(pool)
    assert np.array_equal(p[:, 1, :], to_np(skipped))
    assert np.all(p[:, 0, 2 * nat:] == FILL) and np.all(p[:, 2, 2 * nat:] == FILL)
