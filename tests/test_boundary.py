"""The C-ABI library on the host (no GPU needed): it loads, exports every
function include/kvq.h declares, and rejects invalid arguments with the
documented status before making any HIP call."""
import ctypes
import os
import re

import pytest

import quantized_kv_cache_fp8_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")
FAKE = 0x10000  # a non-NULL pointer value; only ever passed to calls that must fail validation


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["kvq_calibrate_scales", "kvq_cache_write", "kvq_decode_attn", "kvq_prefill_attn",
              "kvq_decode_workspace_size", "kvq_kv_cache_bytes", "kvq_strerror"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = K.lib()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(K.EXPORTS)


def test_header_is_plain_c_and_links():
    """include/kvq.h compiles as strict C99 (no C++, no HIP headers needed) and
    every function it declares resolves at link time against the library the
    binding loads."""
    import subprocess
    names = declared_functions()
    work = os.path.join(ROOT, "tests", "c_client", "_build")  # git-ignored
    os.makedirs(work, exist_ok=True)
    src = os.path.join(work, "uses_every_symbol.c")
    with open(src, "w") as fh:
        fh.write("#include \"kvq.h\"\n"
                 "typedef void (*fn)(void);\n"
                 "fn table[] = {\n" + "".join(f"  (fn){n},\n" for n in names) + "};\n"
                 "int main(void) { return table[0] == 0; }\n")
    exe = os.path.join(work, "uses_every_symbol")
    r = subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                        "-I", os.path.join(ROOT, "include"), src, "-o", exe, K.LIB_PATH, "-Wl,--unresolved-symbols=ignore-in-shared-libs"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@pytest.mark.parametrize("B,Hq,Hkv", [(8, 32, 8), (1, 4, 1), (3, 6, 2), (64, 32, 8)])
def test_kivi_workspace_size_never_shrinks_as_groups_grow(B, Hq, Hkv):
    """The same promise for the 2-bit decode: non-decreasing in max_groups, a
    whole number of (b, hq, split) partials, at least the residual split plus
    one 32-group split per 32 groups."""
    unit = B * Hq * (128 + 2) * 4
    prev = 0
    for mg in range(0, 3001, 3):
        ws = K.kvq_kivi_decode_workspace_size(B, Hq, Hkv, mg)
        assert ws >= prev, f"max_groups {mg}: {ws} < {prev}"
        assert ws % unit == 0 and ws // unit >= 1 + -(-mg // 32)
        prev = ws


def test_strerror_covers_every_status():
    for st in range(-7, 1):
        assert K.kvq_strerror(st) and K.kvq_strerror(st) != "unknown status"
    assert K.kvq_strerror(-99) == "unknown status"


def test_kv_cache_bytes_worked_example():
    # KV-cache quantization textbook 10.4.1: 4 GiB bf16, 2 GiB FP8 for this shape
    assert K.kvq_kv_cache_bytes(32, 1, 8, 32768, 128, 16) == 4 << 30
    assert K.kvq_kv_cache_bytes(32, 1, 8, 32768, 128, 8) == 2 << 30
    assert K.kvq_kv_cache_bytes(32, 1, 8, 32768, 128, 2) == 1 << 29
    assert K.kvq_kv_cache_bytes(-1, 1, 8, 32768, 128, 8) == 0


def test_workspace_size_is_positive_and_monotone():
    a = K.kvq_decode_workspace_size(32, 32, 128, 8192, 16)
    b = K.kvq_decode_workspace_size(32, 32, 128, 16384, 16)
    assert 0 < a <= b
    assert K.kvq_decode_workspace_size(0, 32, 128, 8192, 16) == 0
    # (m, l) pair plus dh partial sums per (b, hq, split)
    assert a % (32 * 32 * (128 + 2) * 4) == 0


@pytest.mark.parametrize("B,Hq,dh", [(32, 32, 128), (4, 32, 128), (1, 4, 64), (8, 64, 128),
                                     (3, 6, 64), (128, 32, 128)])
def test_workspace_size_never_shrinks_as_the_context_grows(B, Hq, dh):
    """A workspace sized for the longest context serves every shorter call:
    across every split-size threshold of the plan, the size is non-decreasing
    in max_context_len, a whole number of (b, hq, split) partials, and at least
    one 40-block split per 640 tokens."""
    unit = B * Hq * (dh + 2) * 4
    prev = 0
    for ctx in range(0, 40001, 7):
        ws = K.kvq_decode_workspace_size(B, Hq, dh, ctx, 16)
        assert ws >= prev, f"max_context_len {ctx}: {ws} < {prev}"
        assert ws % unit == 0 and ws // unit >= max(1, -(-ctx // 640))
        prev = ws


def status_of_decode(**over):
    L = K.lib()
    args = dict(out=FAKE, odt=0, q=FAKE, kc=FAKE, vc=FAKE, nb=10, bt=FAKE, mb=4, cl=FAKE, B=2,
                Hq=8, Hkv=2, dh=128, bs=16, maxctx=64, ks=FAKE, vs=FAKE, fmt=0, gran=0, sm=0.0,
                ws=FAKE, wsb=0, stream=None)
    args.update(over)
    return L.kvq_decode_attn(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(q=None), -1), (dict(ks=None), -1), (dict(bt=None), -1), (dict(ws=None, wsb=1 << 20), -1),
    (dict(Hq=6, Hkv=4), -2), (dict(B=0), -2), (dict(maxctx=65), -2), (dict(maxctx=-1), -2),
    (dict(nb=0), -2), (dict(dh=96), -3), (dict(bs=32), -3), (dict(fmt=3), -3), (dict(gran=5), -3),
    (dict(odt=3), -3), (dict(Hq=64, Hkv=2), -3), (dict(wsb=16), -4),
])
def test_decode_validation(over, status):
    assert status_of_decode(**over) == status


def test_write_validation():
    L = K.lib()
    base = [FAKE, FAKE, 4, 2, 128, FAKE, FAKE, FAKE, 8, 16, FAKE, FAKE, 0, 0, None]
    def st(**kw):
        a = list(base)
        idx = dict(k=0, v=1, T=2, Hkv=3, dh=4, slots=5, kc=6, vc=7, nb=8, bs=9, ks=10, vs=11,
                   fmt=12, gran=13)
        for k, v in kw.items():
            a[idx[k]] = v
        return L.kvq_cache_write(*a)
    assert st(kc=None) == -1 and st(slots=None) == -1 and st(ks=None) == -1
    assert st(T=-1) == -2 and st(nb=0) == -2 and st(Hkv=0) == -2
    assert st(dh=80) == -3 and st(bs=8) == -3 and st(fmt=7) == -3
    assert st(k=FAKE + 2) == -3 and st(kc=FAKE + 8) == -3  # misaligned
    assert st(T=0) == 0  # empty batch: nothing to launch


def test_calibrate_and_codec_validation():
    L = K.lib()
    assert L.kvq_calibrate_scales(FAKE, 4, 2, 128, 0, 0, None, FAKE, 0, None) == -1
    assert L.kvq_calibrate_scales(FAKE, -4, 2, 128, 0, 0, FAKE, FAKE, 0, None) == -2
    assert L.kvq_calibrate_scales(FAKE, 4, 2, 12, 0, 0, FAKE, FAKE, 0, None) == -2
    assert L.kvq_calibrate_scales(FAKE, 4, 2, 128, 3, 0, FAKE, FAKE, 0, None) == -3
    kv = L.kvq_calibrate_scales_kv
    assert kv(FAKE, FAKE, 4, 2, 128, 0, 0, FAKE, FAKE, FAKE, None, 0, None) == -1
    assert kv(FAKE, None, 4, 2, 128, 0, 0, FAKE, FAKE, FAKE, FAKE, 0, None) == -1
    assert kv(FAKE, FAKE, -1, 2, 128, 0, 0, FAKE, FAKE, FAKE, FAKE, 0, None) == -2
    assert kv(FAKE, FAKE, 4, 0, 128, 0, 0, FAKE, FAKE, FAKE, FAKE, 0, None) == -2
    assert kv(FAKE, FAKE, 4, 2, 128, 0, 7, FAKE, FAKE, FAKE, FAKE, 0, None) == -3
    assert L.kvq_fp8_encode(0, None, 8, FAKE, None) == -1
    assert L.kvq_fp8_encode(0, FAKE, -8, FAKE, None) == -2
    assert L.kvq_fp8_encode(0, FAKE, 0, FAKE, None) == 0
    assert L.kvq_fp8_decode(9, FAKE, 8, FAKE, None) == -3


def test_prefill_validation():
    L = K.lib()
    base = dict(out=FAKE, odt=0, q=FAKE, cu=FAKE, maxq=8, qs=FAKE, qg=0, kc=FAKE, vc=FAKE, nb=4,
                bt=FAKE, mb=4, cl=FAKE, B=1, Hq=8, Hkv=2, dh=128, bs=16, ks=FAKE, vs=FAKE, fmt=0,
                kvg=0, sm=0.0, stream=None)
    def st(**kw):
        a = dict(base)
        a.update(kw)
        return L.kvq_prefill_attn(*a.values())
    assert st(cu=None) == -1 and st(qs=None) == -1
    assert st(maxq=-1) == -2 and st(Hq=7) == -2
    assert st(qg=4) == -3 and st(dh=256) == -3
    assert st(fmt=2) == -3  # INT8 caches: the FP8-domain prefill does not take them
    assert st(maxq=0) == 0


def test_token_scale_write_validation():
    L = K.lib()
    base = dict(k=FAKE, v=FAKE, T=4, Hkv=2, dh=128, slots=FAKE, kc=FAKE, vc=FAKE, ksc=FAKE,
                vsc=FAKE, nb=8, bs=16, fmt=0, stream=None)
    def st(**kw):
        a = dict(base)
        a.update(kw)
        return L.kvq_cache_write_token_scales(*a.values())
    assert st(ksc=None) == -1 and st(vsc=None) == -1 and st(slots=None) == -1
    assert st(T=-1) == -2 and st(nb=0) == -2 and st(T=1 << 28, Hkv=8) == -2
    assert st(dh=96) == -3 and st(bs=32) == -3 and st(fmt=3) == -3
    assert st(ksc=FAKE + 1) == -3 and st(vc=FAKE + 8) == -3  # misaligned
    assert st(T=0) == 0


def test_token_scale_decode_validation():
    L = K.lib()
    base = dict(out=FAKE, odt=0, q=FAKE, kc=FAKE, vc=FAKE, ksc=FAKE, vsc=FAKE, nb=10, bt=FAKE,
                mb=4, cl=FAKE, B=2, Hq=8, Hkv=2, dh=128, bs=16, maxctx=64, fmt=0, sm=0.0,
                ws=FAKE, wsb=0, stream=None)
    def st(**kw):
        a = dict(base)
        a.update(kw)
        return L.kvq_decode_attn_token_scales(*a.values())
    assert st(ksc=None) == -1 and st(vsc=None) == -1 and st(ws=None, wsb=1 << 20) == -1
    assert st(Hq=6, Hkv=4) == -2 and st(maxctx=65) == -2
    assert st(Hq=16, Hkv=2) == -3  # groups of more than 4 query heads
    assert st(fmt=3) == -3 and st(dh=80) == -3 and st(vsc=FAKE + 1) == -3
    assert st(wsb=16) == -4


def test_kivi_quantize_validation():
    L = K.lib()
    base = dict(k=FAKE, v=FAKE, ng=4, Hkv=2, dh=128, gb=FAKE, cache=FAKE, nb=8, stream=None)
    def st(**kw):
        a = dict(base)
        a.update(kw)
        return L.kvq_kivi_quantize(*a.values())
    assert st(gb=None) == -1 and st(cache=None) == -1 and st(k=None) == -1
    assert st(ng=-1) == -2 and st(nb=0) == -2 and st(Hkv=0) == -2
    assert st(dh=64) == -3 and st(k=FAKE + 4) == -3
    assert st(ng=0) == 0


def test_kivi_decode_validation():
    L = K.lib()
    base = dict(out=FAKE, odt=0, q=FAKE, cache=FAKE, nb=10, bt=FAKE, mb=8, qg=FAKE, mg=6,
                rk=FAKE, rv=FAKE, rl=FAKE, R=128, B=2, Hq=8, Hkv=2, dh=128, sm=0.0, ws=FAKE,
                wsb=0, stream=None)
    def st(**kw):
        a = dict(base)
        a.update(kw)
        return L.kvq_kivi_decode_attn(*a.values())
    assert st(rk=None) == -1 and st(qg=None) == -1 and st(ws=None, wsb=1 << 24) == -1
    assert st(mg=9) == -2 and st(R=0) == -2 and st(Hq=6, Hkv=4) == -2
    assert st(Hq=16, Hkv=2) == -3 and st(dh=64) == -3 and st(R=300) == -3 and st(odt=5) == -3
    assert st(rv=FAKE + 2) == -3
    assert st(wsb=16) == -4
    assert K.kvq_kivi_decode_workspace_size(2, 8, 2, 6) > 0
    assert K.kvq_kivi_decode_workspace_size(2, 7, 2, 6) == 0


def test_skip_rule_follows_the_guide_examples():
    # vLLM FP8 KV-cache guide, skip-layers section: "sliding_window" skips every
    # sliding-window layer; "0 1 23" skips exactly those layer indices
    sw = ["sliding_window"]
    assert K.kvq_layer_skipped(3, True, sw) and not K.kvq_layer_skipped(3, False, sw)
    idx = ["0", "1", "23"]
    assert [i for i in range(40) if K.kvq_layer_skipped(i, False, idx)] == [0, 1, 23]
    assert not K.kvq_layer_skipped(5, True, idx)  # a sliding layer not named by index
    assert K.kvq_layer_skipped(23, True, ["sliding_window", "23"])
    assert not K.kvq_layer_skipped(2, False, []) and not K.kvq_layer_skipped(2, False, ["02"])
    assert not K.kvq_layer_skipped(-1, False, ["-1"])


def test_layer_index_from_module_prefix():
    assert K.kvq_layer_index("model.layers.0.self_attn") == 0
    assert K.kvq_layer_index("model.layers.23.self_attn.attn") == 23
    assert K.kvq_layer_index("lm_head") == -1
    assert K.kvq_layer_index("model.layers.1.mlp.experts.7") == -1  # ambiguous
    assert K.kvq_layer_index("model.layers.x1.attn") == -1


def test_page_bytes_and_common_page():
    # bf16 pages are twice the FP8 ones; every layer pads to the largest
    assert K.kvq_page_bytes(8, 128, 16, 8) == 2 * 8 * 128 * 16
    assert K.kvq_page_bytes(8, 128, 16, 16) == 2 * K.kvq_page_bytes(8, 128, 16, 8)
    assert K.kvq_common_page_bytes([8, 16, 8], 8, 128, 16) == K.kvq_page_bytes(8, 128, 16, 16)
    assert K.kvq_common_page_bytes([8, 8], 8, 128, 16) == K.kvq_page_bytes(8, 128, 16, 8)
    assert K.kvq_common_page_bytes([2], 1, 8, 1) == 16  # 4 bytes of 2-bit codes, rounded to 16
    assert K.kvq_common_page_bytes([], 8, 128, 16) == 0


def test_paged_stride_validation():
    L = K.lib()
    nat = 2 * 16 * 128
    w = [FAKE, FAKE, 4, 2, 128, FAKE, FAKE, FAKE, 8, 16, nat, FAKE, FAKE, 0, 0, None]
    assert L.kvq_cache_write_paged(*w) != -2
    w[10] = nat - 16
    assert L.kvq_cache_write_paged(*w) == -2
    w[10] = nat + 8
    assert L.kvq_cache_write_paged(*w) == -3
    d = dict(out=FAKE, odt=0, q=FAKE, kc=FAKE, vc=FAKE, nb=10, bt=FAKE, mb=4, cl=FAKE, B=2, Hq=8,
             Hkv=2, dh=128, bs=16, bst=nat - 16, maxctx=64, ks=FAKE, vs=FAKE, fmt=0, gran=0,
             sm=0.0, ws=FAKE, wsb=0, stream=None)
    assert L.kvq_decode_attn_paged(*d.values()) == -2
    p = dict(out=FAKE, odt=0, q=FAKE, cu=FAKE, maxq=8, qs=FAKE, qg=0, kc=FAKE, vc=FAKE, nb=4,
             bt=FAKE, mb=4, cl=FAKE, B=1, Hq=8, Hkv=2, dh=128, bs=16, bst=nat + 4, ks=FAKE,
             vs=FAKE, fmt=0, kvg=0, sm=0.0, stream=None)
    assert L.kvq_prefill_attn_paged(*p.values()) == -3


def test_binding_rejects_host_tensors():
    """The Python binding passes device addresses only: a host tensor is
    refused before the library is called."""
    import torch
    x = torch.zeros(8, dtype=torch.float32)
    out = torch.zeros(8, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        K.kvq_fp8_encode(x, "e4m3", out)


def _host_case():
    """Host tensors of a consistent decode / write / prefill case (2 sequences,
    Hq = 8, Hkv = 2, dh = 128, a pool of 10 blocks); the shape checks run
    before any pointer is taken, so host tensors reach them."""
    import torch
    bf, u8, i32 = torch.bfloat16, torch.uint8, torch.int32
    c = dict(kc=torch.zeros(10, 2, 8, 16, 16, dtype=u8), vc=torch.zeros(10, 2, 128, 16, dtype=u8),
             q=torch.zeros(2, 8, 128, dtype=bf), out=torch.zeros(2, 8, 128),
             bt=torch.zeros(2, 4, dtype=i32), cl=torch.zeros(2, dtype=i32),
             k=torch.zeros(5, 2, 128, dtype=bf), v=torch.zeros(5, 2, 128, dtype=bf),
             slots=torch.zeros(5, dtype=torch.int64), s1=torch.ones(1), s2=torch.ones(2),
             kn=torch.zeros(2, 2, 128, dtype=bf), vn=torch.zeros(2, 2, 128, dtype=bf))
    return c


def _bad(c, **over):
    d = dict(c)
    d.update(over)
    return d


@pytest.mark.parametrize("over,match", [
    (dict(k="k3"), "k has shape"),          # more KV heads than the cache
    (dict(v="vshort"), "v has shape"),
    (dict(slots="slots4"), "slot_mapping"),
    (dict(s1="s2"), "k_scale"),              # per-tensor call with two scales
])
def test_binding_checks_write_shapes(over, match):
    import torch
    c = _host_case()
    alt = dict(k3=torch.zeros(5, 3, 128, dtype=torch.bfloat16),
               vshort=torch.zeros(4, 2, 128, dtype=torch.bfloat16),
               slots4=torch.zeros(4, dtype=torch.int64), s2=c["s2"])
    d = _bad(c, **{k: alt[v] for k, v in over.items()})
    with pytest.raises(ValueError, match=match):
        K.kvq_cache_write(d["k"], d["v"], d["slots"], d["kc"], d["vc"], d["s1"], c["s1"],
                          "e4m3", "tensor")


@pytest.mark.parametrize("over,match", [
    (dict(out="out_small"), "out has shape"),
    (dict(q="q_dh64"), "q has shape"),      # head dim other than the cache's
    (dict(q="q_hq6"), "q has shape"),       # Hq not a multiple of Hkv
    (dict(bt="bt1"), "block_tables"),       # fewer rows than sequences
    (dict(cl="cl1"), "context_lens"),
    (dict(s2="s1"), "k_scale"),             # per-head call with one scale
])
def test_binding_checks_decode_shapes(over, match):
    import torch
    c = _host_case()
    alt = dict(out_small=torch.zeros(1, 8, 128), q_dh64=torch.zeros(2, 8, 64, dtype=torch.bfloat16),
               q_hq6=torch.zeros(2, 7, 128, dtype=torch.bfloat16),
               bt1=torch.zeros(1, 4, dtype=torch.int32), cl1=torch.zeros(1, dtype=torch.int32),
               s1=c["s1"])
    d = _bad(c, **{k: alt[v] for k, v in over.items()})
    if over.get("out") or over.get("q"):
        d["out"] = d["out"] if over.get("out") else torch.zeros(d["q"].shape)
    with pytest.raises(ValueError, match=match):
        K.kvq_decode_attn(d["out"], d["q"], d["kc"], d["vc"], d["bt"], d["cl"], 64, d["s2"],
                          c["s2"], "e4m3", "head")


def test_binding_checks_append_and_prefill_shapes():
    import torch
    c = _host_case()
    with pytest.raises(ValueError, match="k_new"):
        K.kvq_decode_attn_append(c["out"], c["q"], c["k"], c["vn"], c["kc"], c["vc"], c["bt"],
                                 c["cl"], 64, c["s1"], c["s1"], "e4m3", "tensor")
    cu = torch.tensor([0, 3, 5], dtype=torch.int32)
    q = torch.zeros(5, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out has shape"):
        K.kvq_prefill_attn(torch.zeros(4, 8, 128), q, cu, 3, c["s1"], "tensor", c["kc"], c["vc"],
                           c["bt"], c["cl"], c["s1"], c["s1"], "e4m3", "tensor")
    with pytest.raises(ValueError, match="q_scale"):
        K.kvq_prefill_attn(torch.zeros(5, 8, 128), q, cu, 3, c["s2"], "head", c["kc"], c["vc"],
                           c["bt"], c["cl"], c["s1"], c["s1"], "e4m3", "tensor")
    with pytest.raises(ValueError, match="block_tables"):
        K.kvq_prefill_attn(torch.zeros(5, 8, 128), q, torch.tensor([0, 1, 2, 5], dtype=torch.int32),
                           3, c["s1"], "tensor", c["kc"], c["vc"], c["bt"], c["cl"], c["s1"],
                           c["s1"], "e4m3", "tensor")


def test_binding_checks_calibrate_and_kivi_shapes():
    import torch
    x = torch.zeros(4, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="scale_out"):
        K.kvq_calibrate_scales(x, "e4m3", "head", torch.zeros(2), torch.zeros(1))
    with pytest.raises(ValueError, match="one shape"):
        K.kvq_calibrate_scales_kv(x, x[:2], "e4m3", "tensor", *[torch.zeros(1)] * 4)
    with pytest.raises(ValueError, match="v_scale_out"):
        K.kvq_calibrate_scales_kv(x, x, "e4m3", "head", *[torch.zeros(2)] * 3, torch.zeros(1))
    k = torch.zeros(64, 2, 128, dtype=torch.bfloat16)
    cache = torch.zeros(4, 2, K.KIVI_TILE, dtype=torch.uint8)
    with pytest.raises(ValueError, match="group_blocks"):
        K.kvq_kivi_quantize(k, k, torch.zeros(3, dtype=torch.int32), cache)
    with pytest.raises(ValueError, match="KV heads"):
        K.kvq_kivi_quantize(k, k, torch.zeros(2, dtype=torch.int32),
                            torch.zeros(4, 3, K.KIVI_TILE, dtype=torch.uint8))
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    rk = torch.zeros(2, 2, 16, 128, dtype=torch.bfloat16)
    i32 = torch.int32
    with pytest.raises(ValueError, match="res_v"):
        K.kvq_kivi_decode_attn(torch.zeros(2, 8, 128), q, cache, torch.zeros(2, 4, dtype=i32),
                               torch.zeros(2, dtype=i32), 4, rk, rk[:, :, :8], torch.zeros(2, dtype=i32))
