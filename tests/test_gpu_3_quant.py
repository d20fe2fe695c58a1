"""GPU checks of the W8A8 activation quantisers: per-token x quantisation and
per-slot h quantisation (on the GPU's own h) are bit-exact against the
oracle's quantiser (same fp32 decisions), and the h codes also satisfy the
defining half-step bound."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import cfg_inputs, moe, say

pytestmark = pytest.mark.gpu


def _regions(T, H, I, k):
    S = T * k
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    o, reg = 0, {}
    for name, n in (("h", S * I * 4), ("hq", S * I), ("hs", S * 4), ("xq", T * H), ("xs", T * 4),
                    ("y", S * H * 4)):
        reg[name] = (o, n)
        o = up(o + n)
    return reg


@pytest.mark.parametrize("which", ["config3", "edge"])
def test_fp8_quantisers(which):
    m = moe()
    if which == "config3":
        inp = cfg_inputs(3)
    else:
        from synth import make_inputs
        inp = make_inputs(6, 8, 512, 256, 2, dtype="fp8", seed=2, device="cuda")
        x = inp.x.float()
        x[1] = 0.0                                     # an all-zero row: scale 1, codes 0
        x[2, 7] = 3e4                                  # a large outlier
        x[3] *= 1e-3                                   # small values near the subnormal range
        inp.x = x.to(torch.bfloat16)
    say(f"fp8 quantisers {which}")
    M = 16
    ids, w = m.route_topk(inp.logits, inp.k)
    sid, be, npad = m.align_block(ids, inp.E, M)
    ws = m.alloc_workspace(inp.T, inp.E, inp.H, inp.I, inp.k, M, m.MOE_DTYPE_FP8, "cuda")
    m.ffn_fp8(inp.x, inp.w1, inp.w1_scale, inp.w2, inp.w2_scale, ids, w, sid, be, npad, M,
              m.STAGE_FC1 | m.STAGE_FC2, ws)
    torch.cuda.synchronize()
    reg = _regions(inp.T, inp.H, inp.I, inp.k)
    wsh = ws.cpu().numpy()

    def grab(name, dtype):
        o, n = reg[name]
        return wsh[o:o + n].view(dtype)

    xq = grab("xq", np.uint8).reshape(inp.T, inp.H)
    xs = grab("xs", np.float32)
    x32 = oracle.bf16_bits_to_f64(inp.host_x()).astype(np.float32)
    q_o, s_o = oracle.quant_rows_e4m3(x32)
    assert np.array_equal(xs, s_o), "x scales differ"
    # codes equal as values (a negative value rounding to zero may carry either sign)
    assert np.array_equal(oracle.e4m3fn_decode(xq), oracle.e4m3fn_decode(q_o)), "x codes differ"

    S = inp.S
    h = grab("h", np.float32).reshape(S, inp.I)
    hq = grab("hq", np.uint8).reshape(S, inp.I)
    hs = grab("hs", np.float32)
    hq_o, hs_o = oracle.quant_rows_e4m3(h)
    assert np.array_equal(hs, hs_o), "h scales differ"
    assert np.array_equal(oracle.e4m3fn_decode(hq), oracle.e4m3fn_decode(hq_o)), "h codes differ"
    dq = oracle.e4m3fn_decode(hq) * hs[:, None].astype(np.float64)
    # within half an e4m3 step: relative 2^-4 for normals, 2^-10 * scale for subnormals
    assert np.all(np.abs(dq - h) <= np.abs(h) * 2.0 ** -4 + hs[:, None] * 2.0 ** -10 * 1.0001)
