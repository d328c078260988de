"""GPU parity of scale calibration and quantize-on-write (bit-exact against the oracle)."""
import numpy as np
import pytest

import oracle
import workloads as W
from helpers import SENTINEL, DecodeRun, same_codes, to_dev, to_np

pytestmark = pytest.mark.gpu
FMTS = [oracle.FMT_E4M3, oracle.FMT_E5M2, oracle.FMT_INT8]
ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)

# scales in the supported range (positive, below 2^126): powers of two, amax/fmax-like
# values, the extremes (quotients overflow / underflow), scales below 2^-100 whose
# reciprocal leaves the fp32 range (subnormal ones down to 2^-149 included: an E5M2
# calibration of a tensor with amax below 2^-110 gives one) and a seeded
# log-uniform spread
SCALES = ([1.0, 0.5, 2.0 ** -9, 1.0 / 448, 10.0 / 448, 3.0, 0.0123, 123.456, 1e-30, 3.3e20,
           1.1754944e-38, 6.0e37, 2.0 ** -101, 3.1e-33, 2.0 ** -130, 1.0e-40, 2.0 ** -149]
          + list(np.exp(W.rng(77).uniform(np.log(1e-6), np.log(1e6), 48)).astype(np.float32)))


# Writes of up to 512 tokens take the one-pass kernel, longer ones the
# LDS-staged kernel; "long" pads a short write with skipped tokens (slot -1) so
# the same cases also run through the second kernel.
SHORT_WRITE = 512


def gpu_write(k_bits, v_bits, slots, nb, Hkv, dh, ks, vs, fmt, gran, path="short"):
    import torch
    import quantized_kv_cache_fp8_amd as K
    if path == "long" and k_bits.shape[0] <= SHORT_WRITE:
        pad = SHORT_WRITE + 1 - k_bits.shape[0]
        z = np.zeros((pad, Hkv, dh), np.uint16)
        k_bits, v_bits = np.concatenate([k_bits, z]), np.concatenate([v_bits, z])
        slots = np.concatenate([slots, np.full(pad, -1, np.int64)])
    kc = torch.full(oracle.k_cache_shape(nb, Hkv, 16, dh), SENTINEL, dtype=torch.uint8,
                    device="cuda:0")
    vc = torch.full((nb, Hkv, dh, 16), SENTINEL, dtype=torch.uint8, device="cuda:0")
    K.kvq_cache_write(to_dev(k_bits), to_dev(v_bits), to_dev(slots), kc, vc,
                      to_dev(np.asarray(ks, np.float32)), to_dev(np.asarray(vs, np.float32)),
                      fmt, gran)
    torch.cuda.synchronize()
    return to_np(kc), to_np(vc)


def oracle_write(k_bits, v_bits, slots, nb, Hkv, dh, ks, vs, fmt, gran):
    kc = np.full(oracle.k_cache_shape(nb, Hkv, 16, dh), SENTINEL, np.uint8)
    vc = np.full((nb, Hkv, dh, 16), SENTINEL, np.uint8)
    oracle.cache_write(k_bits, v_bits, slots, kc, vc, np.asarray(ks, np.float32),
                       np.asarray(vs, np.float32), fmt, gran)
    return kc, vc


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("path", ["short", "long"])
def test_write_every_bf16_input_for_every_scale(fmt, path):
    """All 65536 bf16 patterns (as K, and reversed as V) for each scale: the
    cache bytes equal the oracle's, i.e. fp8(fl32(x / s)) exactly."""
    k = ALL_BF16.reshape(512, 1, 128)
    v = ALL_BF16[::-1].copy().reshape(512, 1, 128)
    slots = np.arange(512, dtype=np.int64)
    for s in SCALES:
        s = np.float32(s)
        gk, gv = gpu_write(k, v, slots, 32, 1, 128, [s], [s], fmt, oracle.GRAN_TENSOR, path)
        rk, rv = oracle_write(k, v, slots, 32, 1, 128, [s], [s], fmt, oracle.GRAN_TENSOR)
        assert same_codes(fmt, gk, rk), f"K differs at scale {s!r}"
        assert same_codes(fmt, gv, rv), f"V differs at scale {s!r}"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("path", ["short", "long"])
def test_write_per_head_scales(fmt, path):
    g = W.rng(5)
    Hkv, dh = 4, 64
    k = g.permutation(ALL_BF16).reshape(256, Hkv, dh)
    v = g.permutation(ALL_BF16).reshape(256, Hkv, dh)
    ks = np.array([0.25, 1.0 / 448, 7.0, 3.1e-3], np.float32)
    vs = np.array([1.5e-2, 2.0, 1.0, 9.9e3], np.float32)
    slots = g.permutation(256 + 48)[:256].astype(np.int64)  # scattered over a larger pool
    gk, gv = gpu_write(k, v, slots, 19, Hkv, dh, ks, vs, fmt, oracle.GRAN_HEAD, path)
    rk, rv = oracle_write(k, v, slots, 19, Hkv, dh, ks, vs, fmt, oracle.GRAN_HEAD)
    assert same_codes(fmt, gk, rk) and same_codes(fmt, gv, rv)


@pytest.mark.parametrize("path", ["short", "long"])
def test_write_skips_padding_and_out_of_range_slots(path):
    g = W.rng(6)
    Hkv, dh = 2, 128
    k = W.normal_bf16(g, (40, Hkv, dh))
    v = W.normal_bf16(g, (40, Hkv, dh))
    slots = g.permutation(64)[:40].astype(np.int64)
    slots[[3, 17]] = -1  # padding
    slots[[5, 30]] = [64, 1 << 40]  # beyond the pool of 4 blocks: skipped, never written
    gk, gv = gpu_write(k, v, slots, 4, Hkv, dh, [0.01], [0.02], 0, 0, path)
    rk, rv = oracle_write(k, v, slots, 4, Hkv, dh, [0.01], [0.02], 0, 0)
    assert np.array_equal(gk, rk) and np.array_equal(gv, rv)
    assert (gk == SENTINEL).sum() == (rk == SENTINEL).sum() > 0


@pytest.mark.parametrize("start", [0, 2, 5])
@pytest.mark.parametrize("path", ["short", "long"])
def test_write_partial_and_misaligned_runs(start, path):
    """Consecutive slots that start off a 4-token boundary, a ragged token count
    and a gap in the middle: every mix of the dword and byte store paths."""
    g = W.rng(9 + start)
    Hkv, dh, T = 3, 128, 37
    k = W.normal_bf16(g, (T, Hkv, dh))
    v = W.normal_bf16(g, (T, Hkv, dh))
    slots = np.arange(start, start + T, dtype=np.int64)
    slots[20:] += 7  # a gap: later tokens land in other blocks at other offsets
    gk, gv = gpu_write(k, v, slots, 5, Hkv, dh, [0.02, 0.03, 0.05], [0.01, 0.04, 0.2], 1,
                       oracle.GRAN_HEAD, path)
    rk, rv = oracle_write(k, v, slots, 5, Hkv, dh, [0.02, 0.03, 0.05], [0.01, 0.04, 0.2], 1,
                          oracle.GRAN_HEAD)
    assert np.array_equal(gk, rk) and np.array_equal(gv, rv)


@pytest.mark.parametrize("path", ["short", "long"])
def test_duplicate_slots_land_one_of_the_writers(path):
    """Tokens that name the same slot (the header leaves which one lands
    unspecified): every 16-byte K piece of such a slot, one thread's store, is
    the piece of one of its writers, every V byte is one of their bytes, and
    every other slot is bit-exact.  The candidates are the oracle's cache with
    the first writers alone and with the second writers written over them."""
    g = W.rng(31)
    Hkv, dh, T = 2, 128, 120
    k = W.normal_bf16(g, (T, Hkv, dh))
    v = W.normal_bf16(g, (T, Hkv, dh))
    slots = g.permutation(8 * 16)[:T].astype(np.int64)
    slots[90:] = slots[10:40]  # tokens 90..119 land on the slots of tokens 10..39
    ks, vs = [0.02, 0.05], [0.03, 0.01]
    gk, gv = gpu_write(k, v, slots, 8, Hkv, dh, ks, vs, 0, oracle.GRAN_HEAD, path)
    first = slots.copy()
    first[90:] = -1
    ak, av = oracle_write(k, v, first, 8, Hkv, dh, ks, vs, 0, oracle.GRAN_HEAD)
    bk, bv = ak.copy(), av.copy()
    second = np.full(T, -1, np.int64)
    second[90:] = slots[90:]
    oracle.cache_write(k, v, second, bk, bv, np.asarray(ks, np.float32),
                       np.asarray(vs, np.float32), 0, oracle.GRAN_HEAD)
    # K: [blk][h][chunk][off][16] -- compare whole 16-byte pieces
    pk = lambda c: c.reshape(-1, 16)
    ok_k = np.all(pk(gk) == pk(ak), axis=1) | np.all(pk(gk) == pk(bk), axis=1)
    assert ok_k.all(), f"{(~ok_k).sum()} K pieces match neither writer"
    assert np.all((gv == av) | (gv == bv)), "a V byte matches neither writer"
    # slots with one writer (or none) are exact: there the two candidates agree
    assert np.array_equal(gk[ak == bk], ak[ak == bk]) and np.array_equal(gv[av == bv], av[av == bv])
    assert (ak != bk).any()  # the duplicates really differ


def test_write_empty_batch_is_a_no_op():
    gk, gv = gpu_write(np.zeros((0, 2, 64), np.uint16), np.zeros((0, 2, 64), np.uint16),
                       np.zeros(0, np.int64), 2, 2, 64, [1.0], [1.0], 0, 0)
    assert np.all(gk == SENTINEL) and np.all(gv == SENTINEL)


# ------------------------------------------------------------------ calibration

def gpu_calibrate(x_bits, fmt, gran, amax_in=None):
    import torch
    import quantized_kv_cache_fp8_amd as K
    n = x_bits.shape[1] if gran == oracle.GRAN_HEAD else 1
    amax = to_dev(np.asarray(amax_in, np.float32)) if amax_in is not None else \
        torch.full((n,), 12345.0, device="cuda:0")
    sc = torch.empty(n, dtype=torch.float32, device="cuda:0")
    K.kvq_calibrate_scales(to_dev(x_bits), fmt, gran, amax, sc, accumulate=amax_in is not None)
    torch.cuda.synchronize()
    return to_np(amax), to_np(sc)


def same_f32(a, b):
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(
        a[~np.isnan(a)].view(np.uint32), b[~np.isnan(b)].view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("gran", [oracle.GRAN_TENSOR, oracle.GRAN_HEAD])
@pytest.mark.parametrize("shape", [(1, 1, 64), (333, 6, 64), (4099, 8, 128), (50, 32, 128), (77, 5, 64),
                                   (7, 300, 64)])
def test_calibrate_matches_oracle(fmt, gran, shape):
    g = W.rng(sum(shape) + fmt)
    x = W.normal_bf16(g, shape, 1, W.log_uniform(g, shape[1], 0.5, 20.0), g.choice(shape[2], 2),
                      10.0)
    ga, gs = gpu_calibrate(x, fmt, gran)
    ra, rs = oracle.calibrate(x, fmt, gran)
    assert same_f32(ga, ra) and same_f32(gs, rs)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("gran", [oracle.GRAN_TENSOR, oracle.GRAN_HEAD])
@pytest.mark.parametrize("shape", [(1, 1, 64), (333, 6, 64), (4099, 8, 128), (7, 300, 64),
                                   (0, 3, 64)])
def test_calibrate_kv_equals_two_calls(fmt, gran, shape):
    """K and V in one call: both results match the oracle per tensor and are
    bit-identical to two single calls; accumulation continues both."""
    import torch
    import quantized_kv_cache_fp8_amd as K
    g = W.rng(900 + sum(shape) + fmt)
    k = W.normal_bf16(g, shape, 1, W.log_uniform(g, shape[1], 0.5, 20.0), g.choice(shape[2], 2), 10.0)
    v = W.normal_bf16(g, shape, 1, W.log_uniform(g, shape[1], 1e-3, 5.0))
    if shape[0] > 5:
        v[5, 0, 3] = 0x7FC0  # a NaN in V only
    n = shape[1] if gran == oracle.GRAN_HEAD else 1
    arrs = [torch.full((n,), 12345.0, device="cuda:0") for _ in range(4)]
    K.kvq_calibrate_scales_kv(to_dev(k), to_dev(v), fmt, gran, *arrs)
    torch.cuda.synchronize()
    ka, va, ks, vs = (to_np(a) for a in arrs)
    for x, a, sc in ((k, ka, ks), (v, va, vs)):
        ra, rs = oracle.calibrate(x, fmt, gran)
        assert same_f32(a, ra) and same_f32(sc, rs)
        ga, gs = gpu_calibrate(x, fmt, gran)
        assert same_f32(a, ga) and same_f32(sc, gs)
    # a second batch accumulates into both
    k2 = W.normal_bf16(g, (9,) + shape[1:], 1, np.full(shape[1], 30.0))
    v2 = W.normal_bf16(g, (9,) + shape[1:], 1, np.full(shape[1], 0.01))
    K.kvq_calibrate_scales_kv(to_dev(k2), to_dev(v2), fmt, gran, *arrs, accumulate=True)
    torch.cuda.synchronize()
    for x, x2, a, sc in ((k, k2, arrs[0], arrs[2]), (v, v2, arrs[1], arrs[3])):
        ra, rs = oracle.calibrate(np.concatenate([x, x2]), fmt, gran)
        assert same_f32(to_np(a), ra) and same_f32(to_np(sc), rs)


def test_calibrate_accumulates_across_batches():
    g = W.rng(8)
    a = W.normal_bf16(g, (100, 4, 64), 1, np.array([1, 2, 3, 4.0]))
    b = W.normal_bf16(g, (70, 4, 64), 1, np.array([4, 3, 2, 1.0]))
    ga, _ = gpu_calibrate(a, 0, oracle.GRAN_HEAD)
    ga2, gs2 = gpu_calibrate(b, 0, oracle.GRAN_HEAD, amax_in=ga)
    ra, rs = oracle.calibrate(np.concatenate([a, b]), 0, oracle.GRAN_HEAD)
    assert same_f32(ga2, ra) and same_f32(gs2, rs)


def test_calibrate_degenerate_sets():
    z = np.zeros((64, 3, 64), np.uint16)
    z[:, 2, :] = 0x8000  # -0 only
    z[7, 1, 9] = 0x7FC0  # NaN in head 1
    ga, gs = gpu_calibrate(z, 0, oracle.GRAN_HEAD)
    ra, rs = oracle.calibrate(z, 0, oracle.GRAN_HEAD)
    assert same_f32(ga, ra) and same_f32(gs, rs)
    assert gs[0] == 1.0 and np.isnan(ga[1]) and gs[1] == 1.0 and gs[2] == 1.0
    z[7, 1, 9] = 0xFF80  # -Inf
    ga, gs = gpu_calibrate(z, 1, oracle.GRAN_TENSOR)
    assert np.isinf(ga[0]) and gs[0] == 1.0
    ga, gs = gpu_calibrate(np.zeros((0, 3, 64), np.uint16), 1, oracle.GRAN_HEAD)
    assert np.all(ga == 0) and np.all(gs == 1.0)


@pytest.mark.parametrize("fmt", FMTS)
def test_tiny_amax_gives_a_usable_subnormal_scale(fmt):
    """A tensor whose amax is tiny (bf16 values near 2^-120, zeros among
    them) calibrates to a scale below 2^-126 for E5M2 (amax / 57344) and near
    it for the other formats; the scale and every code written with it, zeros
    included, equal the oracle's (zeros stay code 0, not NaN)."""
    g = W.rng(31 + fmt)
    Hkv, dh = 2, 128
    mant = g.integers(0, 128, (64, Hkv, dh)).astype(np.uint16)
    expo = g.integers(1, 12, (64, Hkv, dh)).astype(np.uint16)  # 2^-126 .. 2^-116
    k = (expo << 7) | mant | (g.integers(0, 2, (64, Hkv, dh)).astype(np.uint16) << 15)
    k[:, :, :9] = 0  # zeros among them
    k[3, 1, 20:30] = g.integers(1, 128, 10)  # bf16 subnormals
    ga, gs = gpu_calibrate(k, fmt, oracle.GRAN_TENSOR)
    ra, rs = oracle.calibrate(k, fmt, oracle.GRAN_TENSOR)
    assert same_f32(ga, ra) and same_f32(gs, rs)
    if fmt == oracle.FMT_E5M2:
        assert 0 < rs[0] < 2.0 ** -126
    slots = np.arange(64, dtype=np.int64)
    for path in ("short", "long"):
        gk, gv = gpu_write(k, k, slots, 4, Hkv, dh, rs, rs, fmt, oracle.GRAN_TENSOR, path)
        rk, rv = oracle_write(k, k, slots, 4, Hkv, dh, rs, rs, fmt, oracle.GRAN_TENSOR)
        assert np.array_equal(gk, rk) and np.array_equal(gv, rv)
        assert np.all(gk.reshape(4, Hkv, dh // 16, 16, 16)[0, :, 0, :, :9] == 0)


# ------------------------------------------------------------------ full-size workloads

@pytest.mark.parametrize("which", ["llama", "long-e4m3", "long-e5m2"])
def test_full_size_calibrate_and_write(which):
    """The Llama-3-8B-shaped layer (B=32, ctx ~ U[512, 8192], per-tensor) and
    the long-context batch (B=4, S=32768, per-head): GPU scales and every cache
    byte equal the oracle's."""
    wl = {"llama": W.llama_layer_decode, "long-e4m3": lambda: W.long_context_decode("e4m3"),
          "long-e5m2": lambda: W.long_context_decode("e5m2")}[which]()
    print(f"[{which}] tokens={wl.kv.k.shape[0]}", flush=True)
    run = DecodeRun(wl)
    run.gpu_scales()
    assert same_f32(to_np(run.ks), run.ks_ref) and same_f32(to_np(run.vs), run.vs_ref)
    run.gpu_write()
    rk, rv = run.oracle_caches()
    assert np.array_equal(to_np(run.kc), rk)
    assert np.array_equal(to_np(run.vc), rv)
