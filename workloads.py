"""Seeded synthetic inputs for the FP8 paged KV-cache path.

This module only draws random data and lays out block tables; it holds none of
the method's arithmetic (no quantization, no scales, no attention), so both the
CPU oracle and the GPU library can be fed from it.

Data recipe (the pages measure on no public data set; these synthetic tensors
stand in for real Llama-shaped activations):

* numpy ``Generator(PCG64(seed))``; values drawn as fp32 N(0, 1) and rounded to
  bf16 with round-to-nearest-even; tensors are returned as the uint16 bit
  pattern of the bf16 values.
* Outlier channels: a seeded set of channel indices, shared by every token and
  head of one tensor, multiplied by a constant (K outliers sit in fixed
  channels, textbook 10.4.4 on KIVI).
* Per-head ranges: head h of a tensor is multiplied by r_h = exp(U(ln lo, ln hi)),
  drawn independently for the Q, K and V heads.
* Paging: sequence b owns ceil(ctx_b / bs) physical blocks; physical ids are a
  seeded permutation of the pool.  One extra "trap" block holds random bytes,
  and every unused block-table entry points at it, so a kernel that reads past
  a sequence's context picks up garbage and fails parity (without touching
  memory outside the pool).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 20260


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); return the uint16 bits.  Finite input only."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(g: np.random.Generator, shape, head_axis: int | None = None,
                head_mult: np.ndarray | None = None, outlier_channels: np.ndarray | None = None,
                outlier_mult: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if outlier_channels is not None and len(outlier_channels):
        x[..., outlier_channels] *= np.float32(outlier_mult)
    if head_mult is not None:
        sh = [1] * len(shape)
        sh[head_axis] = shape[head_axis]
        x *= head_mult.astype(np.float32).reshape(sh)
    return f32_to_bf16_bits(x)


def log_uniform(g: np.random.Generator, n: int, lo: float, hi: float) -> np.ndarray:
    return np.exp(g.uniform(np.log(lo), np.log(hi), size=n)).astype(np.float32)


@dataclass
class Paging:
    """Block pool for a batch of sequences of given context lengths."""
    context_lens: np.ndarray  # int32 [B]
    block_tables: np.ndarray  # int32 [B, max_blocks]
    num_blocks: int
    bs: int
    trap_block: int

    def slots(self, b: int, positions: np.ndarray) -> np.ndarray:
        blk = self.block_tables[b, positions // self.bs].astype(np.int64)
        return blk * self.bs + positions % self.bs


def make_paging(g: np.random.Generator, context_lens, bs: int = 16,
                max_blocks: int | None = None) -> Paging:
    cl = np.asarray(context_lens, np.int32)
    nb_seq = (cl.astype(np.int64) + bs - 1) // bs
    need = int(nb_seq.sum())
    num_blocks = need + 1
    if max_blocks is None:
        max_blocks = max(1, int(nb_seq.max()) if len(cl) else 1)
    perm = g.permutation(num_blocks).astype(np.int32)
    trap = int(perm[-1])
    bt = np.full((len(cl), max_blocks), trap, np.int32)
    o = 0
    for b, n in enumerate(nb_seq):
        bt[b, :n] = perm[o:o + n]
        o += n
    return Paging(cl, bt, num_blocks, bs, trap)


@dataclass
class KVBatch:
    """K/V of every cached token of a batch, in sequence order, plus where each goes."""
    k: np.ndarray  # uint16 (bf16 bits) [T, Hkv, dh]
    v: np.ndarray
    slot_mapping: np.ndarray  # int64 [T]
    seq_offsets: np.ndarray  # int64 [B+1]: token rows of sequence b


def make_kv(g: np.random.Generator, paging: Paging, Hkv: int, dh: int,
            k_outliers: tuple[int, float] = (0, 1.0), v_outliers: tuple[int, float] = (0, 1.0),
            head_range: tuple[float, float] | None = None) -> KVBatch:
    cl = paging.context_lens.astype(np.int64)
    T = int(cl.sum())
    k_ch = g.choice(dh, size=k_outliers[0], replace=False) if k_outliers[0] else None
    v_ch = g.choice(dh, size=v_outliers[0], replace=False) if v_outliers[0] else None
    k_mult = log_uniform(g, Hkv, *head_range) if head_range else None
    v_mult = log_uniform(g, Hkv, *head_range) if head_range else None
    k = normal_bf16(g, (T, Hkv, dh), 1, k_mult, k_ch, k_outliers[1])
    v = normal_bf16(g, (T, Hkv, dh), 1, v_mult, v_ch, v_outliers[1])
    offs = np.concatenate([[0], np.cumsum(cl)]).astype(np.int64)
    slots = np.empty(T, np.int64)
    for b in range(len(cl)):
        slots[offs[b]:offs[b + 1]] = paging.slots(b, np.arange(cl[b]))
    return KVBatch(k, v, slots, offs)


def scale_rows(g: np.random.Generator, x: np.ndarray, lo: float, hi: float) -> np.ndarray:
    """bf16 [T, H, dh] with every (token, head) row multiplied by its own
    log-uniform factor in [lo, hi] (rows of very different magnitudes, the case
    per-token scales are for); re-rounded to bf16."""
    T, H, _ = x.shape
    f = log_uniform(g, T * H, lo, hi).reshape(T, H, 1)
    return f32_to_bf16_bits(bf16_bits_to_f32(x) * f)


@dataclass
class DecodeWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    dh: int
    bs: int
    fmt: str  # "e4m3" | "e5m2" | "int8"
    gran: str  # "tensor" | "head"
    paging: Paging
    kv: KVBatch
    q: np.ndarray  # uint16 [B, Hq, dh]
    fixed_scale: float | None = None  # scale used as-is (no calibration)
    meta: dict = field(default_factory=dict)


def decode_workload(name: str, seed: int, B: int, Hq: int, Hkv: int, dh: int, context_lens,
                    bs: int = 16, fmt: str = "e4m3", gran: str = "tensor",
                    k_outliers=(0, 1.0), v_outliers=(0, 1.0), head_range=None,
                    fixed_scale: float | None = None) -> DecodeWorkload:
    g = rng(seed)
    paging = make_paging(g, context_lens, bs)
    kv = make_kv(g, paging, Hkv, dh, k_outliers, v_outliers, head_range)
    q_mult = log_uniform(g, Hq, *head_range) if head_range else None
    q = normal_bf16(g, (B, Hq, dh), 1, q_mult)
    return DecodeWorkload(name, B, Hq, Hkv, dh, bs, fmt, gran, paging, kv, q, fixed_scale)


def uniform_context_lens(g_seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    """ctx_b ~ U{lo..hi} inclusive, from its own seeded stream."""
    return rng(g_seed).integers(lo, hi + 1, size=B).astype(np.int32)


# ------------------------------------------------------------------ named workloads

def tiny_decode(seed: int = BASE_SEED + 0) -> DecodeWorkload:
    """B=1, Hq=4, Hkv=2, dh=64, context 256 in 16 shuffled blocks of 16; two
    outlier K channels x8; per-tensor scale fixed at 1.0; E4M3."""
    return decode_workload("tiny-decode-b1-h4-kv2-d64-ctx256", seed, 1, 4, 2, 64, [256], 16,
                           "e4m3", "tensor", k_outliers=(2, 8.0), fixed_scale=1.0)


def llama_layer_decode(seed: int = BASE_SEED + 1, B: int = 32, lo: int = 512,
                       hi: int = 8192) -> DecodeWorkload:
    """Llama-3-8B-shaped layer: B=32, Hq=32, Hkv=8, dh=128, ctx ~ U{512..8192},
    bs=16; K and V each with 4 outlier channels x10; per-tensor scales from amax; E4M3."""
    cl = uniform_context_lens(seed * 7 + 1, B, lo, hi)
    return decode_workload(f"llama3-8b-layer-decode-b{B}-ctx{lo}-{hi}", seed, B, 32, 8, 128, cl,
                           16, "e4m3", "tensor", k_outliers=(4, 10.0), v_outliers=(4, 10.0))


def long_context_decode(fmt: str = "e4m3", seed: int = BASE_SEED + 2, B: int = 4,
                        S: int = 32768) -> DecodeWorkload:
    """B=4, Hq=32, Hkv=8, dh=128, S=32768 per sequence; per-head scales for K/V
    [8] and Q [32]; head ranges log-uniform in [0.5, 20]."""
    return decode_workload(f"long-context-decode-b{B}-s{S}-{fmt}", seed, B, 32, 8, 128, [S] * B,
                           16, fmt, "head", head_range=(0.5, 20.0))


@dataclass
class PrefillWorkload:
    name: str
    Hq: int
    Hkv: int
    dh: int
    bs: int
    fmt: str
    paging: Paging
    kv: KVBatch  # every cached token: prefix and chunk
    q: np.ndarray  # uint16 [total_q, Hq, dh]: the chunk's queries
    cu_seqlens: np.ndarray  # int32 [B+1]
    prefix_lens: np.ndarray  # int32 [B]


def prefill_workload(name: str, seed: int, prefix_lens, chunk_lens, Hq: int = 32, Hkv: int = 8,
                     dh: int = 128, bs: int = 16, fmt: str = "e4m3") -> PrefillWorkload:
    g = rng(seed)
    pl = np.asarray(prefix_lens, np.int32)
    ch = np.asarray(chunk_lens, np.int32)
    paging = make_paging(g, pl + ch, bs)
    kv = make_kv(g, paging, Hkv, dh)
    cu = np.concatenate([[0], np.cumsum(ch)]).astype(np.int32)
    q = normal_bf16(g, (int(cu[-1]), Hq, dh))
    return PrefillWorkload(name, Hq, Hkv, dh, bs, fmt, paging, kv, q, cu, pl)


def ragged_chunked_prefill(seed: int = BASE_SEED + 7) -> PrefillWorkload:
    """8 sequences whose chunk and cached prefix are equal and range from 256 to
    4096 tokens (work per sequence differs 16-fold); Hq=32, Hkv=8, dh=128."""
    lens = [4096, 512, 2048, 1024, 4096, 256, 3072, 1536]
    return prefill_workload("fp8-chunked-prefill-ragged-b8-256-4096", seed, lens, lens)


def fp8_chunked_prefill(seed: int = BASE_SEED + 3, B: int = 8, prefix: int = 4096,
                        chunk: int = 4096) -> PrefillWorkload:
    """8 sequences, a 4096-token chunk each on top of 4096 cached tokens;
    Hq=32, Hkv=8, dh=128; N(0,1); per-head E4M3 scales for Q, K and V."""
    return prefill_workload(f"fp8-chunked-prefill-b{B}-prefix{prefix}-chunk{chunk}", seed,
                            [prefix] * B, [chunk] * B)


# ------------------------------------------------------------------ KIVI 2-bit

@dataclass
class KiviWorkload:
    """Sequences whose first quant_groups[b] 32-token groups are quantized into
    a paged 2-bit cache (block = group) and whose next res_lens[b] tokens sit in
    a bf16 residual [B, Hkv, R, dh]."""
    name: str
    B: int
    Hq: int
    Hkv: int
    R: int
    paging: Paging  # bs = 32; context_lens = 32 * quant_groups
    k: np.ndarray  # uint16 [sum(quant_groups) * 32, Hkv, dh]: quantized tokens, group order
    v: np.ndarray
    group_blocks: np.ndarray  # int32 [n_groups]: block of each group
    quant_groups: np.ndarray  # int32 [B]
    res_k: np.ndarray  # uint16 [B, Hkv, R, dh]
    res_v: np.ndarray
    res_lens: np.ndarray  # int32 [B]
    q: np.ndarray  # uint16 [B, Hq, dh]


def kivi_workload(name: str, seed: int, Hq: int, Hkv: int, quant_groups, res_lens, R: int = 128,
                  dh: int = 128, k_outliers=(4, 10.0), head_range=(0.5, 4.0),
                  max_blocks: int | None = None) -> KiviWorkload:
    """K with a few fixed outlier channels (the per-channel structure KIVI's K
    grouping is for), V plain; per-head magnitudes log-uniform; N(0,1) q."""
    g = rng(seed)
    qg = np.asarray(quant_groups, np.int32)
    rl = np.asarray(res_lens, np.int32)
    B = len(qg)
    paging = make_paging(g, qg * 32, 32, max_blocks)
    n = int(qg.sum())
    gb = np.concatenate([paging.block_tables[b, :qg[b]] for b in range(B)]).astype(np.int32) \
        if n else np.zeros(0, np.int32)
    k_ch = g.choice(dh, size=k_outliers[0], replace=False) if k_outliers[0] else None
    km = log_uniform(g, Hkv, *head_range)
    vm = log_uniform(g, Hkv, *head_range)
    k = normal_bf16(g, (n * 32, Hkv, dh), 1, km, k_ch, k_outliers[1])
    v = normal_bf16(g, (n * 32, Hkv, dh), 1, vm)
    rk = normal_bf16(g, (B, Hkv, R, dh), 1, km, k_ch, k_outliers[1])
    rv = normal_bf16(g, (B, Hkv, R, dh), 1, vm)
    q = normal_bf16(g, (B, Hq, dh))
    return KiviWorkload(name, B, Hq, Hkv, R, paging, k, v, gb, qg, rk, rv, rl, q)


def kivi_2bit_decode(seed: int = BASE_SEED + 5, B: int = 8, S: int = 16384,
                     R: int = 128) -> KiviWorkload:
    """B=8, Hq=32, Hkv=8, dh=128, S=16384 tokens per sequence: the first
    S - 128 in 2-bit groups of 32, the newest 128 in the bf16 residual."""
    return kivi_workload(f"kivi-2bit-decode-b{B}-s{S}-res{R}", seed, 32, 8,
                         [(S - R) // 32] * B, [R] * B, R)
