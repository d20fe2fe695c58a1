"""GPU parity of the block-scaled FP8 path (128 x 128 weight blocks, 1 x 128
activation groups) against the oracle: the 16-token decode workload's shapes,
small ragged shapes over block sizes, the group quantisers bit-exact, extreme
block scales, determinism and stage splitting, an empty batch."""
import numpy as np
import pytest
import torch

import oracle
from synth import config_inputs, make_inputs
from tests.gpu_util import TOL, moe, out_f64, say

pytestmark = pytest.mark.gpu

TOL_BLOCK = TOL["fp8"]


def _run(inp, block_m, flags=0, workspace=None, out=None):
    m = moe()
    ids, w, sid, be, npad = m.route_align(inp.logits, inp.k, block_m)
    out = m.ffn_fp8_block(inp.x, inp.w1, inp.w1_scale, inp.w2, inp.w2_scale, ids, w, sid, be,
                          npad, block_m, flags, workspace, out)
    torch.cuda.synchronize()
    return ids, w, out


def _oracle(inp, tokens=None):
    ids, w = oracle.route(inp.host_logits(), inp.k)
    return ids, oracle.ffn_fp8_block(inp.host_x(), inp.host_w1, inp.host_w1_scale(),
                                     inp.host_w2, inp.host_w2_scale(), ids, w, tokens)


def test_decode_block_fp8_parity():
    inp = config_inputs(3, device="cuda", dtype="fp8_block")
    bm = moe().default_block_m(inp.T, inp.E, inp.k)
    say(f"fp8 block decode T={inp.T} E={inp.E} H={inp.H} I={inp.I} k={inp.k} block_m={bm}")
    ids, w, out = _run(inp, bm)
    ids_o, ref = _oracle(inp)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    err = oracle.normwise_rel_err(out_f64(out), ref)
    say(f"  normwise rel err {err:.3e} (tol {TOL_BLOCK})")
    assert err <= TOL_BLOCK


CASES = [  # T, E, H, I, k, routing
    (37, 16, 256, 384, 3, "normal"),
    (5, 4, 128, 128, 4, "normal"),
    (1, 1, 256, 128, 1, "normal"),
    (16, 2, 256, 128, 2, "normal"),
    (12, 3, 384, 256, 2, "zipf"),
    (90, 8, 640, 384, 2, "zipf"),
]


@pytest.mark.parametrize("block_m", [1, 16, 64, 256])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}_E{}_H{}_I{}_k{}_{}".format(*c))
def test_small_ragged_parity(case, block_m):
    T, E, H, I, k, routing = case
    say(f"fp8 block small T={T} E={E} H={H} I={I} k={k} {routing} block_m={block_m}")
    inp = make_inputs(T, E, H, I, k, dtype="fp8_block", routing=routing,
                      seed=T + 5 * E + block_m, device="cuda")
    _, _, out = _run(inp, block_m)
    _, ref = _oracle(inp)
    err = oracle.normwise_rel_err(out_f64(out), ref)
    say(f"  normwise rel err {err:.3e}")
    assert err <= TOL_BLOCK


def _regions(T, H, I, k):
    S = T * k
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    o, reg = 0, {}
    for name, n in (("h", S * I * 4), ("hq", S * I), ("hs", S * (I // 128) * 4), ("xq", T * H),
                    ("xs", T * (H // 128) * 4), ("y", S * H * 4)):
        reg[name] = (o, n)
        o = up(o + n)
    return reg


def test_group_quantisers():
    # x groups bit-exact against the oracle's quantiser (same fp32 decisions);
    # h groups satisfy their definition on the GPU's own h
    m = moe()
    inp = make_inputs(6, 8, 512, 256, 2, dtype="fp8_block", seed=2, device="cuda")
    x = inp.x.float()
    x[1] = 0.0                                 # all groups zero
    x[2, 130] = 3e4                            # one outlier group
    x[3, :128] *= 1e-3                         # a group near the subnormal range
    inp.x = x.to(torch.bfloat16)
    say("fp8 block quantisers")
    M = 16
    ids, w, sid, be, npad = m.route_align(inp.logits, inp.k, M)
    ws = m.alloc_workspace(inp.T, inp.E, inp.H, inp.I, inp.k, M, m.MOE_DTYPE_FP8_BLOCK, "cuda")
    m.ffn_fp8_block(inp.x, inp.w1, inp.w1_scale, inp.w2, inp.w2_scale, ids, w, sid, be, npad, M,
                    m.STAGE_FC1 | m.STAGE_FC2, ws)
    torch.cuda.synchronize()
    reg = _regions(inp.T, inp.H, inp.I, inp.k)
    wsh = ws.cpu().numpy()

    def grab(name, dtype):
        o, n = reg[name]
        return wsh[o:o + n].view(dtype)

    xq = grab("xq", np.uint8).reshape(inp.T, inp.H)
    xs = grab("xs", np.float32).reshape(inp.T, inp.H // 128)
    x32 = oracle.bf16_bits_to_f64(inp.host_x()).astype(np.float32)
    q_o, s_o = oracle.quant_groups_e4m3(x32)
    assert np.array_equal(xs, s_o), "x group scales differ"
    assert np.array_equal(oracle.e4m3fn_decode(xq), oracle.e4m3fn_decode(q_o)), "x codes differ"
    h = grab("h", np.float32).reshape(inp.S, inp.I)
    hq = grab("hq", np.uint8).reshape(inp.S, inp.I)
    hs = grab("hs", np.float32).reshape(inp.S, inp.I // 128)
    q_h, s_h = oracle.quant_groups_e4m3(h)
    assert np.array_equal(hs, s_h), "h group scales differ"
    assert np.array_equal(oracle.e4m3fn_decode(hq), oracle.e4m3fn_decode(q_h)), "h codes differ"


def test_extreme_block_scales():
    # block scales spanning 2^-20 .. 2^10 within one expert
    T, E, H, I, k = 8, 2, 384, 256, 2
    inp = make_inputs(T, E, H, I, k, dtype="fp8_block", seed=6, device="cuda")
    g = torch.Generator().manual_seed(1)
    e1 = torch.randint(-20, 11, inp.w1_scale.shape, generator=g).float()
    e2 = torch.randint(-20, 11, inp.w2_scale.shape, generator=g).float()
    inp.w1_scale = (inp.w1_scale.cpu() * torch.exp2(e1)).cuda()
    inp.w2_scale = (inp.w2_scale.cpu() * torch.exp2(e2)).cuda()
    say("fp8 block extreme scales")
    _, _, out = _run(inp, 16)
    _, ref = _oracle(inp)
    got = out_f64(out)
    assert np.all(np.isfinite(got))
    err = oracle.normwise_rel_err(got, ref)
    say(f"  normwise rel err {err:.3e}")
    assert err <= TOL_BLOCK


def test_determinism_and_stages():
    m = moe()
    inp = make_inputs(40, 16, 512, 256, 4, dtype="fp8_block", routing="zipf", seed=4,
                      device="cuda")
    say("fp8 block determinism/stages")
    M = 16
    ids, w, sid, be, npad = m.route_align(inp.logits, inp.k, M)
    call = lambda **kw: m.ffn_fp8_block(inp.x, inp.w1, inp.w1_scale, inp.w2,  # noqa: E731
                                        inp.w2_scale, ids, w, sid, be, npad, M, **kw)
    a = call()
    b = call(flags=m.NO_XCD_REMAP)
    ws = m.alloc_workspace(inp.T, inp.E, inp.H, inp.I, inp.k, M, m.MOE_DTYPE_FP8_BLOCK, "cuda")
    d = torch.empty_like(a)
    for st in (m.STAGE_FC1, m.STAGE_FC2, m.STAGE_COMBINE):
        call(flags=st, workspace=ws, out=d)
    f = torch.empty_like(a)  # PREP in a call of its own
    for st in (m.STAGE_PREP, m.STAGE_FC1 | m.PREPARED, m.STAGE_FC2 | m.STAGE_COMBINE):
        call(flags=st, workspace=ws, out=f)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), d.view(torch.int16))
    assert torch.equal(a.view(torch.int16), f.view(torch.int16))


def test_empty_batch_and_null_scales():
    m = moe()
    say("fp8 block T=0 and null scales")
    inp = make_inputs(2, 4, 128, 128, 2, dtype="fp8_block", seed=0, device="cuda")
    ids, w, sid, be, npad = m.route_align(inp.logits[:0], 2, 16)
    out = m.ffn_fp8_block(inp.x[:0], inp.w1, inp.w1_scale, inp.w2, inp.w2_scale, ids, w, sid,
                          be, npad, 16)
    assert out.shape == (0, 128)
    ids, w, sid, be, npad = m.route_align(inp.logits, 2, 16)
    ws = m.alloc_workspace(2, 4, 128, 128, 2, 16, m.MOE_DTYPE_FP8_BLOCK, "cuda")
    out = torch.empty((2, 128), dtype=torch.bfloat16, device="cuda")
    st = m.lib.moe_ffn_fp8_block(m._ptr(inp.x), m._ptr(inp.w1), m._ptr(inp.w1_scale),
                                 m._ptr(inp.w2), None, m._ptr(ids), m._ptr(w), m._ptr(sid),
                                 m._ptr(be), m._ptr(npad), 2, 4, 128, 128, 2, 16, 0, m._ptr(ws),
                                 ws.numel(), m._ptr(out), None)
    assert st != m.MOE_OK
