"""GPU check of moe_forward_small_static, the allocation-free variant of
moe_forward_small for callers that cannot allocate device memory: called
through the C ABI, its outputs equal moe_forward_small's bit for bit (and the
oracle's within tolerance) on two calls in a row, the second with a smaller
batch, in both modes and both weight formats; a batch that needs more than the
static scratch is refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs
from tests.gpu_util import TOL, moe, oracle_forward, out_f64, say

pytestmark = pytest.mark.gpu


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _static_call(inp, flags):
    """moe_forward_small_static straight through the C ABI (ctypes), on
    caller-allocated outputs."""
    m = moe()
    T, E, H, I, k = inp.T, inp.E, inp.H, inp.I, inp.k
    fp8 = inp.dtype == "fp8"
    out = torch.full((T, H), 0x7F7F, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    wts = torch.full((T, k), -1.0, dtype=torch.float32, device="cuda")
    st = m.lib.moe_forward_small_static(
        _ptr(inp.logits), _ptr(inp.x), _ptr(inp.w1), _ptr(inp.w1_scale) if fp8 else None,
        _ptr(inp.w2), _ptr(inp.w2_scale) if fp8 else None, T, E, H, I, k, 0,
        m.MOE_DTYPE_FP8 if fp8 else m.MOE_DTYPE_BF16, flags, _ptr(ids), _ptr(wts), _ptr(out),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == m.MOE_OK, m.status_str(st)
    return out, ids, wts


def _reference(inp, flags):
    m = moe()
    out, ids, wts = m.forward_small(inp.logits, inp.x, inp.w1, inp.w2, inp.k, False,
                                    inp.w1_scale, inp.w2_scale, flags)
    return out, ids, wts


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("mode", ["split", "one_kernel"])
def test_static_scratch_matches_workspace_entry_point(dtype, mode):
    m = moe()
    flags = m.FORWARD_ONE_KERNEL if mode == "one_kernel" else 0
    # a batch at the small path's limits first, then a smaller one that reuses
    # (and must not be disturbed by) what the first left in the scratch
    cases = [(16, 64, 1024, 512, 8, 11), (3, 20, 512, 256, 4, 12)]
    for T, E, H, I, k, seed in cases:
        say(f"static-scratch forward {dtype} {mode} T={T} E={E} H={H} I={I} k={k}")
        inp = make_inputs(T, E, H, I, k, dtype=dtype, routing="normal", seed=seed,
                          device="cuda")
        got, ids, wts = _static_call(inp, flags)
        ref, ids_r, wts_r = _reference(inp, flags)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_r), "topk_ids differ from moe_forward_small"
        assert torch.equal(wts.view(torch.int32), wts_r.view(torch.int32)), \
            "topk_weights differ from moe_forward_small"
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), \
            "out differs from moe_forward_small"
        ids_o, w_o, ref_o = oracle_forward(inp)
        assert np.array_equal(ids.cpu().numpy(), ids_o)
        err = oracle.normwise_rel_err(out_f64(got), ref_o)
        say(f"  bitwise equal to moe_forward_small; vs oracle {err:.3e}")
        assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_static_scratch_beyond_small_kernels(dtype):
    # batches past the small kernels (routing, alignment and the FFN launches
    # inside the scratch), a smaller one of them second, then one that takes
    # the small kernels: each bit-equal to moe_forward_small
    cases = [(64, 64, 512, 256, 8, 31, "zipf"), (24, 16, 256, 256, 4, 32, "zipf"),
             (5, 16, 256, 256, 4, 33, "normal")]
    for T, E, H, I, k, seed, routing in cases:
        say(f"static-scratch forward {dtype} T={T} E={E} H={H} I={I} k={k} {routing}")
        inp = make_inputs(T, E, H, I, k, dtype=dtype, routing=routing, seed=seed,
                          device="cuda")
        got, ids, wts = _static_call(inp, 0)
        ref, ids_r, wts_r = _reference(inp, 0)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_r) and torch.equal(wts.view(torch.int32),
                                                       wts_r.view(torch.int32))
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), \
            "out differs from moe_forward_small"
        ids_o, w_o, ref_o = oracle_forward(inp)
        err = oracle.normwise_rel_err(out_f64(got), ref_o)
        say(f"  bitwise equal to moe_forward_small; vs oracle {err:.3e}")
        assert err <= TOL[dtype]


def test_static_scratch_size_limit():
    # the layer's intermediates would not fit in the static scratch: refused on
    # the host with MOE_ERR_WORKSPACE, nothing launched, outputs untouched
    m = moe()
    T, E, H, I, k = 16, 16, 32768, 4096, 16
    need = m.forward_small_workspace_bytes(T, E, H, I, k, m.MOE_DTYPE_FP8)
    assert need > m.STATIC_SCRATCH_BYTES
    logits = torch.zeros((T, E), dtype=torch.float32, device="cuda")
    x = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(16, dtype=torch.uint8, device="cuda")  # never read
    s = torch.zeros(16, dtype=torch.float32, device="cuda")
    ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    wts = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    out = torch.zeros((T, H), dtype=torch.bfloat16, device="cuda")
    st = m.lib.moe_forward_small_static(_ptr(logits), _ptr(x), _ptr(w), _ptr(s), _ptr(w),
                                        _ptr(s), T, E, H, I, k, 0, m.MOE_DTYPE_FP8, 0, _ptr(ids),
                                        _ptr(wts), _ptr(out), None)
    assert st == 4  # MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((ids == -7).all())
