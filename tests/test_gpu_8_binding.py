"""The binding checks every tensor argument against the others before calling
the library (the C ABI sees only addresses): mismatched shapes, dtypes,
devices and alignment buffers too small for the block size are refused with
an exception and nothing is launched (the outputs keep their sentinels)."""
import pytest
import torch

from synth import make_inputs
from tests.gpu_util import moe, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def setup():
    m = moe()
    inp = make_inputs(12, 8, 256, 128, 2, dtype="bf16", routing="normal", seed=5, device="cuda")
    ids, w, sid, be, npad = m.route_align(inp.logits, inp.k, 16)
    torch.cuda.synchronize()
    return m, inp, (ids, w, sid, be, npad)


def _expect(exc, fn):
    with pytest.raises(exc):
        fn()


def test_ffn_argument_checks(setup):
    m, inp, (ids, w, sid, be, npad) = setup
    say("binding: FFN argument checks")
    out = torch.full((inp.T, inp.H), 0x7F7F, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    call = lambda **kw: m.ffn_bf16(**{**dict(  # noqa: E731
        x=inp.x, w1=inp.w1, w2=inp.w2, topk_ids=ids, topk_weights=w, sorted_ids=sid,
        block_expert=be, num_padded=npad, block_m=16, out=out), **kw})
    _expect(ValueError, lambda: call(w1=inp.w1[:, :, :128].contiguous()))       # H mismatch
    _expect(ValueError, lambda: call(w2=inp.w2[:4]))                            # E mismatch
    _expect(ValueError, lambda: call(w2=inp.w2.transpose(1, 2).contiguous()))   # [E, I, H]
    _expect(ValueError, lambda: call(topk_ids=ids[:5].contiguous()))            # T mismatch
    _expect(ValueError, lambda: call(topk_weights=w[:, :1].contiguous()))       # k mismatch
    _expect(TypeError, lambda: call(topk_weights=w.double()))
    _expect(TypeError, lambda: call(x=inp.x.float()))
    # alignment made for 16-token blocks, FFN asked to run 64-token blocks:
    # the buffers are too small for that block size's capacity
    _expect(ValueError, lambda: call(block_m=64))
    _expect(ValueError, lambda: call(out=torch.empty((inp.T, inp.H + 8), dtype=torch.bfloat16,
                                                     device="cuda")))
    _expect(TypeError, lambda: call(out=torch.empty((inp.T, inp.H), dtype=torch.float32,
                                                    device="cuda")))
    _expect(ValueError, lambda: call(out=torch.empty((inp.T, inp.H), dtype=torch.bfloat16)))
    _expect(ValueError, lambda: call(workspace=torch.empty(64, dtype=torch.uint8,
                                                           device="cuda")))
    _expect(ValueError, lambda: call(workspace=torch.empty(1 << 20, dtype=torch.uint8)))
    _expect(ValueError, lambda: call(x=inp.x[:, ::2]))                          # not contiguous
    torch.cuda.synchronize()
    assert bool((out.view(torch.int16) == 0x7F7F).all()), "a refused call wrote its output"
    call()                                                                      # the good call
    torch.cuda.synchronize()
    assert not bool((out.view(torch.int16) == 0x7F7F).all())


def test_scaled_and_small_argument_checks(setup):
    m, _, _ = setup
    say("binding: fp8 scale and small-path checks")
    inp = make_inputs(6, 8, 256, 128, 2, dtype="fp8", routing="normal", seed=6, device="cuda")
    ids, w, sid, be, npad = m.route_align(inp.logits, inp.k, 16)
    call = lambda **kw: m.ffn_fp8(**{**dict(  # noqa: E731
        x=inp.x, w1=inp.w1, w1_scale=inp.w1_scale, w2=inp.w2, w2_scale=inp.w2_scale,
        topk_ids=ids, topk_weights=w, sorted_ids=sid, block_expert=be, num_padded=npad,
        block_m=16), **kw})
    _expect(ValueError, lambda: call(w1_scale=inp.w1_scale[:, :128].contiguous()))
    _expect(ValueError, lambda: call(w2_scale=inp.w2_scale[:4]))
    _expect(TypeError, lambda: call(w1_scale=inp.w1_scale.half()))
    # block scales given to the per-row entry point
    _expect(ValueError, lambda: call(w1_scale=torch.ones((8, 2, 2), device="cuda")))
    small = lambda **kw: m.forward_small(**{**dict(  # noqa: E731
        logits=inp.logits, x=inp.x, w1=inp.w1, w2=inp.w2, k=inp.k, w1_scale=inp.w1_scale,
        w2_scale=inp.w2_scale), **kw})
    _expect(ValueError, lambda: small(logits=inp.logits[:, :4].contiguous()))
    _expect(ValueError, lambda: small(workspace=torch.empty(256, dtype=torch.uint8,
                                                            device="cuda")))
    _expect(ValueError, lambda: small(topk_ids=torch.empty((6, 3), dtype=torch.int32,
                                                           device="cuda")))
    _expect(ValueError, lambda: m.forward_small_static(inp.logits, inp.x, inp.w1, inp.w2, inp.k,
                                                       w1_scale=inp.w1_scale,
                                                       w2_scale=inp.w2_scale[:, :64].contiguous()))
    _expect(ValueError, lambda: m.route_topk(inp.logits, 2, out=(ids[:3].contiguous(), w)))
    _expect(ValueError, lambda: m.align_block(ids, inp.E, 16, out=(sid[:8], be, npad)))
    call()
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_prepared_calls_match_direct_calls(setup, dtype):
    # prepare=True checks and marshals once; the prepared calls, run several
    # times, give the bits of the direct calls
    m, _, _ = setup
    say(f"binding: prepared calls {dtype}")
    inp = make_inputs(24, 16, 256, 256, 4, dtype=dtype, routing="zipf", seed=8, device="cuda")
    bm = 64
    ref = m.forward(inp.x, inp.logits, inp.w1, inp.w2, inp.k, bm, w1_scale=inp.w1_scale,
                    w2_scale=inp.w2_scale)
    ids, w, sid, be, npad = m.route_align(inp.logits, inp.k, bm)
    route = m.route_align(inp.logits, inp.k, bm, out=(ids, w, sid, be, npad), prepare=True)
    code = m.MOE_DTYPE_FP8 if dtype == "fp8" else m.MOE_DTYPE_BF16
    ws = m.alloc_workspace(inp.T, inp.E, inp.H, inp.I, inp.k, bm, code, "cuda")
    out = torch.empty_like(ref)
    if dtype == "fp8":
        ffn = m.ffn_fp8(inp.x, inp.w1, inp.w1_scale, inp.w2, inp.w2_scale, ids, w, sid, be,
                        npad, bm, 0, ws, out, prepare=True)
    else:
        ffn = m.ffn_bf16(inp.x, inp.w1, inp.w2, ids, w, sid, be, npad, bm, 0, ws, out,
                         prepare=True)
    small = m.forward_small(inp.logits, inp.x, inp.w1, inp.w2, inp.k, False, inp.w1_scale,
                            inp.w2_scale, prepare=True)
    assert isinstance(route, m.Prepared) and isinstance(ffn, m.Prepared)
    for _ in range(3):
        out.zero_()
        route()
        ffn()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    small()
    torch.cuda.synchronize()
