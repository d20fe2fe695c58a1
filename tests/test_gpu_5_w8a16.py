"""GPU parity of the weight-only FP8 (W8A16) path against the oracle: the
16-token decode workload's FP8 weights with bf16 activations, small ragged
shapes over block sizes, every e4m3fn weight code, determinism and stage
splitting, an empty batch."""
import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs
from tests.gpu_util import TOL, cfg_inputs, moe, out_f64, say

pytestmark = pytest.mark.gpu

TOL_W8A16 = TOL["bf16"]   # h and y are rounded to bf16 as on the bf16 path


def _run(inp, block_m, flags=0):
    m = moe()
    ids, w, sid, be, npad = m.route_align(inp.logits, inp.k, block_m)
    out = m.ffn_w8a16(inp.x, inp.w1, inp.w1_scale, inp.w2, inp.w2_scale, ids, w, sid, be, npad,
                      block_m, flags)
    torch.cuda.synchronize()
    return ids, w, out


def _oracle(inp, ids, w, tokens=None):
    return oracle.ffn_w8a16(inp.host_x(), inp.host_w1, inp.host_w1_scale(), inp.host_w2,
                            inp.host_w2_scale(), ids, w, tokens)


def test_decode_fp8_weights_parity():
    inp = cfg_inputs(3)
    bm = moe().default_block_m(inp.T, inp.E, inp.k)
    say(f"w8a16 decode T={inp.T} E={inp.E} H={inp.H} I={inp.I} k={inp.k} block_m={bm}")
    ids, w, out = _run(inp, bm)
    ids_o, w_o = oracle.route(inp.host_logits(), inp.k)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    err = oracle.normwise_rel_err(out_f64(out), _oracle(inp, ids_o, w_o))
    say(f"  normwise rel err {err:.3e} (tol {TOL_W8A16})")
    assert err <= TOL_W8A16


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
    say(f"w8a16 small T={T} E={E} H={H} I={I} k={k} {routing} block_m={block_m}")
    inp = make_inputs(T, E, H, I, k, dtype="fp8", routing=routing, seed=T + 3 * E + block_m,
                      device="cuda")
    ids, w, out = _run(inp, block_m)
    ids_o, w_o = oracle.route(inp.host_logits(), k)
    err = oracle.normwise_rel_err(out_f64(out), _oracle(inp, ids_o, w_o))
    say(f"  normwise rel err {err:.3e}")
    assert err <= TOL_W8A16


def test_every_weight_code():
    # each FC1 row holds all 254 finite e4m3fn codes (in a rotated order) and
    # two zeros; FC2 likewise: every code's widening to bf16 is exercised
    T, E, H, I, k = 8, 2, 256, 256, 2
    inp = make_inputs(T, E, H, I, k, dtype="fp8", routing="normal", seed=5, device="cuda")
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    line = np.concatenate([finite, np.zeros(2, np.uint8)])
    w1 = np.stack([[np.roll(line, 3 * n + e) for n in range(2 * I)] for e in range(E)])
    w2 = np.stack([[np.roll(line, 5 * n + e) for n in range(H)] for e in range(E)])
    inp.w1 = torch.from_numpy(w1).cuda()
    inp.w2 = torch.from_numpy(w2).cuda()
    inp.w1_scale = torch.full((E, 2 * I), 2.0 ** -9, device="cuda")
    inp.w2_scale = torch.full((E, H), 2.0 ** -8, device="cuda")
    say("w8a16 every weight code")
    ids, w, out = _run(inp, 16)
    ids_o, w_o = oracle.route(inp.host_logits(), k)
    ref = _oracle(inp, ids_o, w_o)
    got = out_f64(out)
    assert np.all(np.isfinite(got))
    err = oracle.normwise_rel_err(got, ref)
    say(f"  normwise rel err {err:.3e}")
    assert err <= TOL_W8A16


def test_determinism_and_stages():
    m = moe()
    inp = make_inputs(40, 16, 512, 256, 4, dtype="fp8", routing="zipf", seed=4, device="cuda")
    say("w8a16 determinism/stages")
    M = 16
    ids, w, sid, be, npad = m.route_align(inp.logits, inp.k, M)
    call = lambda **kw: m.ffn_w8a16(inp.x, inp.w1, inp.w1_scale, inp.w2, inp.w2_scale,  # noqa
                                    ids, w, sid, be, npad, M, **kw)
    a = call()
    b = call(flags=m.NO_XCD_REMAP)
    ws = m.alloc_workspace(inp.T, inp.E, inp.H, inp.I, inp.k, M, m.MOE_DTYPE_W8A16, "cuda")
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


def test_empty_batch_and_bad_scales():
    m = moe()
    say("w8a16 T=0 and null scales")
    inp = make_inputs(2, 4, 128, 128, 2, dtype="fp8", seed=0, device="cuda")
    ids, w, sid, be, npad = m.route_align(inp.logits[:0], 2, 16)
    out = m.ffn_w8a16(inp.x[:0], inp.w1, inp.w1_scale, inp.w2, inp.w2_scale, ids, w, sid, be,
                      npad, 16)
    assert out.shape == (0, 128)
    ids, w, sid, be, npad = m.route_align(inp.logits, 2, 16)
    ws = m.alloc_workspace(2, 4, 128, 128, 2, 16, m.MOE_DTYPE_W8A16, "cuda")
    out = torch.empty((2, 128), dtype=torch.bfloat16, device="cuda")
    st = m.lib.moe_ffn_w8a16(m._ptr(inp.x), m._ptr(inp.w1), None, m._ptr(inp.w2),
                             m._ptr(inp.w2_scale), m._ptr(ids), m._ptr(w), m._ptr(sid),
                             m._ptr(be), m._ptr(npad), 2, 4, 128, 128, 2, 16, 0, m._ptr(ws),
                             ws.numel(), m._ptr(out), None)
    assert st != m.MOE_OK
