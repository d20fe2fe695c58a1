"""The C ABI library loads without a GPU, exports exactly what include/moe.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

m = pytest.importorskip("moe_expert_ffn_router_amd")
lib = m.lib
OK, NULL, SHAPE, ALIGN, WORKSPACE, UNSUP = 0, 1, 2, 3, 4, 5


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(moe_\w+)\s*\(", text, flags=re.M))


def exported_functions():
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    return {ln.split()[-1] for ln in out.splitlines() if " T " in ln}


def test_exports_match_header_exactly():
    decl = declared_functions()
    assert decl == set(m.EXPORTS)
    assert exported_functions() == decl
    for name in decl:
        assert hasattr(lib, name)


def test_abi_version_and_status_strings():
    assert lib.moe_abi_version() == 1
    for s in range(7):
        assert m.status_str(s).startswith("MOE_")
    assert "UNKNOWN" in m.status_str(99)


P = 0x1000  # a 4 KiB-aligned fake device address: never dereferenced on these paths


def test_route_validation():
    f = lib.moe_route_topk
    assert f(P, 4, 0, 1, 0, P, P, None) == SHAPE          # E < 1
    assert f(P, 4, 1025, 1, 0, P, P, None) == SHAPE       # E > 1024
    assert f(P, 4, 8, 0, 0, P, P, None) == SHAPE          # k < 1
    assert f(P, 4, 8, 9, 0, P, P, None) == SHAPE          # k > E
    assert f(P, -1, 8, 2, 0, P, P, None) == SHAPE         # T < 0
    assert f(None, 4, 8, 2, 0, P, P, None) == NULL
    assert f(P, 4, 8, 2, 0, None, P, None) == NULL
    assert f(P + 2, 4, 8, 2, 0, P, P, None) == ALIGN
    assert f(None, 0, 8, 2, 0, None, None, None) == OK    # T = 0: nothing to do


def test_route_align_validation():
    f = lib.moe_route_align
    assert f(P, 4, 0, 1, 0, 16, P, P, P, P, P, None) == SHAPE      # E < 1
    assert f(P, 4, 8, 9, 0, 16, P, P, P, P, P, None) == SHAPE      # k > E
    assert f(P, 4, 8, 2, 0, 12, P, P, P, P, P, None) == SHAPE      # block_m not a power of 2
    assert f(None, 4, 8, 2, 0, 16, P, P, P, P, P, None) == NULL    # logits
    assert f(P, 4, 8, 2, 0, 16, P, None, P, P, P, None) == NULL    # topk_weights
    assert f(P, 4, 8, 2, 0, 16, P, P, None, P, P, None) == NULL    # sorted_ids
    assert f(P, 4, 8, 2, 0, 16, P, P, P, P, None, None) == NULL    # num_padded
    assert f(P, 4, 8, 2, 0, 16, P, P, P + 2, P, P, None) == ALIGN


def test_align_validation_and_capacity():
    cap = lib.moe_align_capacity
    assert cap(16, 8, 64, 64) == 128 + 64 * 63           # S + min(E,S)(M-1), a multiple of M
    assert cap(4, 2, 8, 16) == 128
    assert cap(0, 2, 8, 16) == 0
    assert cap(3, 2, 8, 1) == 6
    assert cap(16, 8, 64, 3) == 0                          # block_m not a power of two
    assert cap(16, 8, 64, 512) == 0                        # block_m > 256
    f = lib.moe_align_block
    assert f(P, 4, 2, 8, 3, P, P, P, None) == SHAPE
    assert f(P, 4, 2, 8, 16, P, P, None, None) == NULL
    assert f(None, 4, 2, 8, 16, P, P, P, None) == NULL
    assert f(P, 4, 2, 8, 16, None, P, P, None) == NULL
    assert f(P, 4, 2, 8, 16, P, P, P + 1, None) == ALIGN
    assert f(P, 1 << 22, 8, 64, 16, P, P, P, None) == SHAPE   # T*k >= 2^24


def _ffn_args(**kw):
    a = dict(x=P, w1=P, w2=P, ids=P, wts=P, sid=P, be=P, npad=P, T=4, E=8, H=256, I=512, k=2,
             M=16, flags=0, ws=P, wsb=1 << 30, out=P)
    a.update(kw)
    return a


def call_bf16(**kw):
    a = _ffn_args(**kw)
    return lib.moe_ffn_bf16(a["x"], a["w1"], a["w2"], a["ids"], a["wts"], a["sid"], a["be"],
                            a["npad"], a["T"], a["E"], a["H"], a["I"], a["k"], a["M"], a["flags"],
                            a["ws"], a["wsb"], a["out"], None)


def call_fp8(s1=P, s2=P, **kw):
    a = _ffn_args(**kw)
    return lib.moe_ffn_fp8(a["x"], a["w1"], s1, a["w2"], s2, a["ids"], a["wts"], a["sid"],
                           a["be"], a["npad"], a["T"], a["E"], a["H"], a["I"], a["k"], a["M"],
                           a["flags"], a["ws"], a["wsb"], a["out"], None)


def call_w8a16(s1=P, s2=P, **kw):
    a = _ffn_args(**kw)
    return lib.moe_ffn_w8a16(a["x"], a["w1"], s1, a["w2"], s2, a["ids"], a["wts"], a["sid"],
                             a["be"], a["npad"], a["T"], a["E"], a["H"], a["I"], a["k"], a["M"],
                             a["flags"], a["ws"], a["wsb"], a["out"], None)


def call_fp8_block(s1=P, s2=P, **kw):
    a = _ffn_args(**kw)
    return lib.moe_ffn_fp8_block(a["x"], a["w1"], s1, a["w2"], s2, a["ids"], a["wts"],
                                 a["sid"], a["be"], a["npad"], a["T"], a["E"], a["H"], a["I"],
                                 a["k"], a["M"], a["flags"], a["ws"], a["wsb"], a["out"], None)


def call_f32(**kw):
    a = _ffn_args(**kw)
    return lib.moe_ffn_f32(a["x"], a["w1"], a["w2"], a["ids"], a["wts"], a["sid"], a["be"],
                           a["npad"], a["T"], a["E"], a["H"], a["I"], a["k"], a["M"], a["flags"],
                           a["ws"], a["wsb"], a["out"], None)


# the multiple of 8 H and I must be (bf16, fp8: any; weight-only and
# block-scaled fp8: 128; f32: 4)
MULT = {call_bf16: 8, call_fp8: 8, call_w8a16: 128, call_fp8_block: 128, call_f32: 4}


@pytest.mark.parametrize("call", [call_bf16, call_fp8, call_w8a16, call_fp8_block, call_f32])
def test_ffn_shape_multiples(call):
    m = MULT[call]
    assert call(H=m, I=m, wsb=16) == WORKSPACE               # the smallest allowed shape passes
    assert call(H=200 if m < 128 else 256, I=m * 3, wsb=16) == WORKSPACE
    for bad in (m // 2, m + m // 2, 202, 129):
        if bad % m:
            assert call(H=bad) == SHAPE, bad
            assert call(I=bad) == SHAPE, bad
    if m == 128:
        assert call(H=200) == SHAPE and call(I=136) == SHAPE


@pytest.mark.parametrize("call", [call_bf16, call_fp8, call_w8a16, call_fp8_block, call_f32])
def test_ffn_validation(call):
    assert call(H=202) == SHAPE
    assert call(I=0) == SHAPE
    assert call(k=9) == SHAPE
    assert call(E=2000) == SHAPE
    assert call(M=12) == SHAPE
    assert call(x=None) == NULL
    assert call(npad=None) == NULL
    assert call(ws=None) == NULL
    assert call(out=P + 8) == ALIGN
    assert call(ws=P + 128) == ALIGN
    assert call(wsb=16) == WORKSPACE
    assert call(flags=1 << 20) == UNSUP
    # every documented flag is accepted (the workspace check comes after the flag check)
    for f in (1, 2, 4, 8, 1 | (1 << 11), 1 << 8, 1 << 10):
        assert call(flags=f, wsb=16) == WORKSPACE, f
    assert call(flags=1 << 9, wsb=16) == UNSUP              # moe_forward_small's flag
    assert call(T=0, x=None, out=None, ws=None) == OK       # empty batch: nothing launched


@pytest.mark.parametrize("call", [call_fp8, call_w8a16])
def test_fp8_scale_pointers_validated(call):
    assert call(s1=None) == NULL
    assert call(s2=P + 4) == ALIGN
    assert call(T=0, x=None, out=None, ws=None, s1=None, s2=None) == OK


def test_block_scale_pointers_validated():
    assert call_fp8_block(s1=None) == NULL
    assert call_fp8_block(s2=P + 2) == ALIGN


def call_small(logits=P, x=P, w1=P, s1=P, w2=P, s2=P, T=16, E=64, H=4096, I=1536, k=8,
               renorm=0, dtype=1, flags=0, ids=P, wts=P, ws=P, wsb=1 << 40, out=P):
    return lib.moe_forward_small(logits, x, w1, s1, w2, s2, T, E, H, I, k, renorm, dtype, flags,
                                 ids, wts, ws, wsb, out, None)


def test_small_path_validation():
    assert lib.moe_small_max_tokens() == 64
    assert call_small(T=65) == SHAPE
    assert call_small(T=64, k=9, E=64) == SHAPE           # T * k > 512
    # accepted shapes get as far as the workspace check (no GPU here to run them)
    assert call_small(T=16, k=17, E=64, wsb=100) == WORKSPACE  # 272 slots: aligned launches
    assert call_small(T=64, k=8, E=128, wsb=100) == WORKSPACE
    assert call_small(T=17, flags=1 << 9) == UNSUP        # one kernel: 16 tokens at most
    assert call_small(T=16, k=17, E=64, flags=1 << 9) == UNSUP  # ... and 256 slots
    assert call_small(T=16, flags=1 << 9, wsb=100) == WORKSPACE
    assert call_small(E=1025, k=2) == SHAPE
    assert call_small(H=200) == SHAPE
    assert call_small(dtype=0) == UNSUP                   # f32
    assert call_small(dtype=3) == UNSUP
    assert call_small(flags=1) == UNSUP                   # stage flags are not taken
    assert call_small(flags=1 << 10) == UNSUP
    assert call_small(logits=None) == NULL
    assert call_small(dtype=2, s1=None) == NULL
    assert call_small(dtype=2, s2=P + 4) == ALIGN
    assert call_small(ws=P + 64) == ALIGN
    assert call_small(wsb=100) == WORKSPACE
    assert call_small(T=0, logits=None, x=None, out=None, ws=None) == OK
    wsb = lib.moe_forward_small_workspace_bytes
    assert wsb(16, 64, 4096, 1536, 8, 1) > lib.moe_ffn_workspace_bytes(16, 64, 4096, 1536, 8, 64, 1)
    # beyond the small kernels: the alignment outputs plus the FFN workspace
    for T, E, dt in [(17, 64, 1), (64, 128, 1), (64, 128, 2), (32, 8, 2)]:
        bm = lib.moe_default_block_m(T, E, 8)
        assert wsb(T, E, 7168, 2048, 8, dt) >= (lib.moe_ffn_workspace_bytes(T, E, 7168, 2048, 8, bm, dt)
                                              + 4 * oracle.align_capacity(T * 8, E, bm))
    assert wsb(65, 64, 4096, 1536, 8, 1) == 0 and wsb(16, 64, 4096, 1536, 8, 0) == 0


def call_small_static(logits=P, x=P, w1=P, s1=P, w2=P, s2=P, T=16, E=64, H=4096, I=1536, k=8,
                      renorm=0, dtype=1, flags=0, ids=P, wts=P, out=P):
    return lib.moe_forward_small_static(logits, x, w1, s1, w2, s2, T, E, H, I, k, renorm, dtype,
                                        flags, ids, wts, out, None)


def test_small_static_validation():
    # every rejection happens on the host, before the scratch's device address
    # is looked up (no GPU here)
    assert call_small_static(T=65) == SHAPE
    assert call_small_static(T=17, flags=1 << 9) == UNSUP
    assert call_small_static(H=200) == SHAPE
    assert call_small_static(dtype=0) == UNSUP
    assert call_small_static(flags=1) == UNSUP
    assert call_small_static(logits=None) == NULL
    assert call_small_static(out=None) == NULL
    assert call_small_static(dtype=2, s1=None) == NULL
    assert call_small_static(x=P + 2) == ALIGN
    assert call_small_static(T=0, logits=None, x=None, out=None) == OK
    # intermediates beyond the static scratch (32 MiB): y alone is
    # 256 slots x 32768 x 4 bytes = 32 MiB
    wsb = lib.moe_forward_small_workspace_bytes
    assert wsb(16, 16, 32768, 4096, 16, 2) > m.STATIC_SCRATCH_BYTES
    assert call_small_static(T=16, E=16, H=32768, I=4096, k=16, dtype=2) == WORKSPACE
    assert wsb(16, 64, 4096, 1536, 8, 2) <= m.STATIC_SCRATCH_BYTES  # the decode workloads fit
    assert wsb(64, 128, 7168, 2048, 8, 2) <= m.STATIC_SCRATCH_BYTES  # (the skewed one too)


def test_default_block_m():
    f = lib.moe_default_block_m
    assert f(16, 64, 8) == 64          # decode: 2 slots per expert
    assert f(64, 128, 8) == 64
    assert f(4096, 128, 8) == 256      # prefill: 256 slots per expert
    assert f(16, 1, 8) == 0            # k > E
    assert f(2048, 128, 8) == 256 and f(2047, 128, 8) == 64


def test_workspace_bytes():
    ws = lib.moe_ffn_workspace_bytes
    S, H, I = 16 * 8, 4096, 1536
    bf = ws(16, 64, H, I, 8, 64, 1)
    assert bf >= S * I * 2 + S * H * 2 and bf % 256 == 0      # h, y bf16
    f8 = ws(16, 64, H, I, 8, 64, 2)
    assert f8 >= S * I * 4 + S * I + S * 4 + 16 * H + 16 * 4 + S * H * 4
    assert ws(16, 64, H, I, 8, 64, 3) == bf                  # W8A16 keeps bf16 intermediates
    fb = ws(16, 64, H, I, 8, 64, 4)                          # block FP8: group scales
    assert fb > f8
    assert fb >= S * I * 4 + S * I + S * (I // 128) * 4 + 16 * H + 16 * (H // 128) * 4 + S * H * 4
    assert ws(16, 64, H, I, 8, 64, 7) == 0
    assert ws(0, 64, H, I, 8, 64, 1) == 0
