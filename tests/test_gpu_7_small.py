"""GPU checks of the small-batch forward, in both of its modes (separate
launches without alignment, and one cooperative launch): parity with the
oracle, bit-for-bit equality with routing + alignment + FFN at the same T, the
one-kernel status word, determinism, the XCD-remap switch and an empty batch."""
import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs
from tests.gpu_util import TOL, cfg_inputs, moe, oracle_forward, oracle_full, out_f64, say

pytestmark = pytest.mark.gpu


MODES = ["split", "one_kernel"]


def _small(inp, renormalize=False, flags=0, workspace=None):
    m = moe()
    dt = m.MOE_DTYPE_FP8 if inp.dtype == "fp8" else m.MOE_DTYPE_BF16
    n = m.forward_small_workspace_bytes(inp.T, inp.E, inp.H, inp.I, inp.k, dt)
    if workspace is None:
        workspace = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")  # not zero
    out, ids, wts = m.forward_small(inp.logits, inp.x, inp.w1, inp.w2, inp.k, renormalize,
                                    inp.w1_scale, inp.w2_scale, flags, workspace=workspace)
    torch.cuda.synchronize()
    # the status word is written by the one-kernel mode only
    # (the last 4 of the n bytes this batch needs, also in a larger workspace)
    status = int(workspace[n - 4:n].view(torch.int32).item()) if flags & m.FORWARD_ONE_KERNEL else 0
    return out, ids, wts, status


def _separate(inp, renormalize=False):
    m = moe()
    bm = m.default_block_m(inp.T, inp.E, inp.k)
    ids, w, sid, be, npad = m.route_align(inp.logits, inp.k, bm, renormalize)
    if inp.dtype == "fp8":
        out = m.ffn_fp8(inp.x, inp.w1, inp.w1_scale, inp.w2, inp.w2_scale, ids, w, sid, be,
                        npad, bm)
    else:
        out = m.ffn_bf16(inp.x, inp.w1, inp.w2, ids, w, sid, be, npad, bm)
    torch.cuda.synchronize()
    return out, ids, w


def _flags(mode):
    return moe().FORWARD_ONE_KERNEL if mode == "one_kernel" else 0


def _check(inp, mode, renormalize=False):
    out, ids, wts, status = _small(inp, renormalize, flags=_flags(mode))
    assert status == 0, f"device-side barrier wait gave up (status {status})"
    ids_o, w_o, ref = oracle_forward(inp, renormalize=renormalize)
    assert np.array_equal(ids.cpu().numpy(), ids_o), "topk_ids differ from the oracle"
    assert np.max(np.abs(wts.cpu().numpy() - w_o), initial=0.0) <= 1e-5
    err = oracle.normwise_rel_err(out_f64(out), ref)
    say(f"  normwise rel err {err:.3e} (tol {TOL[inp.dtype]})")
    assert err <= TOL[inp.dtype]
    out_s, ids_s, w_s = _separate(inp, renormalize)
    assert torch.equal(ids, ids_s) and torch.equal(wts, w_s)
    assert torch.equal(out.view(torch.int16), out_s.view(torch.int16)), \
        f"small path ({mode}) differs from routing + alignment + FFN"


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("n", [2, 3])
def test_decode_workloads(n, mode):
    inp = cfg_inputs(n)
    say(f"small path {mode} config {n} ({inp.dtype}) T={inp.T} E={inp.E} H={inp.H} I={inp.I} "
        f"k={inp.k}")
    _check(inp, mode)


CASES = [  # T, E, H, I, k, routing
    (1, 1, 128, 128, 1, "normal"),
    (5, 4, 128, 256, 4, "normal"),
    (16, 2, 256, 128, 2, "normal"),
    (12, 3, 384, 256, 2, "zipf"),
    (16, 256, 256, 128, 16, "normal"),    # 256 slots: one per thread of a workgroup
    (7, 1000, 128, 128, 3, "normal"),     # wide router
    (16, 64, 512, 384, 8, "zipf"),
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}_E{}_H{}_I{}_k{}_{}".format(*c))
def test_small_shapes(case, dtype, mode):
    T, E, H, I, k, routing = case
    say(f"small path {mode} {dtype} T={T} E={E} H={H} I={I} k={k} {routing}")
    inp = make_inputs(T, E, H, I, k, dtype=dtype, routing=routing, seed=T + E, device="cuda")
    _check(inp, mode)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_renormalize_determinism_remap(dtype, mode):
    m = moe()
    f = _flags(mode)
    inp = make_inputs(16, 32, 256, 256, 4, dtype=dtype, routing="normal", seed=3, device="cuda")
    say(f"small path {mode} renormalize/determinism/remap {dtype}")
    _check(inp, mode, renormalize=True)
    a = _small(inp, flags=f)
    b = _small(inp, flags=f)
    c = _small(inp, flags=f | m.NO_XCD_REMAP)
    for r in (a, b, c):
        assert r[3] == 0
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[0].view(torch.int16), c[0].view(torch.int16))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_modes_agree_on_a_reused_workspace(dtype):
    """Both modes on one workspace, alternating, with a smaller batch second:
    no state carries from one call to the next."""
    m = moe()
    say(f"small path modes on a shared workspace {dtype}")
    big = make_inputs(16, 64, 256, 256, 8, dtype=dtype, routing="zipf", seed=11, device="cuda")
    small = make_inputs(3, 64, 256, 256, 8, dtype=dtype, routing="normal", seed=12, device="cuda")
    code = m.MOE_DTYPE_FP8 if dtype == "fp8" else m.MOE_DTYPE_BF16
    n = m.forward_small_workspace_bytes(16, 64, 256, 256, 8, code)
    ws = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    ref = {id(big): _separate(big)[0], id(small): _separate(small)[0]}
    for inp in (big, small, big, small):
        for mode in ("one_kernel", "split"):
            out, _, _, status = _small(inp, flags=_flags(mode), workspace=ws)
            assert status == 0
            assert torch.equal(out.view(torch.int16), ref[id(inp)].view(torch.int16)), mode


# Beyond the small kernels (more than 16 tokens or 256 slots) the forward runs
# routing, alignment and the FFN launches in its own workspace: the same bits
# as the separate calls, and the one-kernel mode is refused.
LARGE_CASES = [  # T, E, H, I, k, routing
    (17, 64, 256, 256, 8, "zipf"),
    (32, 16, 384, 256, 8, "zipf"),      # hot blocks (more than 8 tokens per expert)
    (64, 128, 512, 256, 8, "zipf"),
    (16, 64, 256, 128, 17, "normal"),   # 272 slots
]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("case", LARGE_CASES, ids=lambda c: "T{}_E{}_H{}_I{}_k{}_{}".format(*c))
def test_small_forward_beyond_small_kernels(case, dtype):
    T, E, H, I, k, routing = case
    say(f"small forward (aligned launches) {dtype} T={T} E={E} H={H} I={I} k={k} {routing}")
    inp = make_inputs(T, E, H, I, k, dtype=dtype, routing=routing, seed=T + E + k,
                      device="cuda")
    _check(inp, "split")
    with pytest.raises(Exception):
        moe().forward_small(inp.logits, inp.x, inp.w1, inp.w2, k, False, inp.w1_scale,
                            inp.w2_scale, moe().FORWARD_ONE_KERNEL)


def test_small_forward_skewed_decode_workload():
    # the 64-token skewed decode workload through the one-call forward, every
    # output row against the oracle and bit-equal to the separate calls
    inp = cfg_inputs(4)
    say(f"small forward config 4 T={inp.T} E={inp.E} H={inp.H} I={inp.I} k={inp.k}")
    out, ids, wts, status = _small(inp)
    ids_o, w_o, ref = oracle_full(4)
    assert np.array_equal(ids.cpu().numpy(), ids_o)
    err = oracle.normwise_rel_err(out_f64(out), ref)
    say(f"  normwise rel err {err:.3e}")
    assert err <= TOL[inp.dtype]
    out_s, ids_s, w_s = _separate(inp)
    assert torch.equal(out.view(torch.int16), out_s.view(torch.int16))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_large_then_small_on_one_workspace(dtype):
    """An aligned-launch batch, then a small-kernel batch, then again, on one
    workspace sized for the first."""
    m = moe()
    say(f"small forward, large then small batch on one workspace {dtype}")
    big = make_inputs(48, 32, 256, 256, 8, dtype=dtype, routing="zipf", seed=21, device="cuda")
    small = make_inputs(5, 32, 256, 256, 8, dtype=dtype, routing="normal", seed=22,
                        device="cuda")
    code = m.MOE_DTYPE_FP8 if dtype == "fp8" else m.MOE_DTYPE_BF16
    n = max(m.forward_small_workspace_bytes(48, 32, 256, 256, 8, code),
            m.forward_small_workspace_bytes(5, 32, 256, 256, 8, code))
    ws = torch.full((n,), 0x5A, dtype=torch.uint8, device="cuda")
    ref = {id(big): _separate(big)[0], id(small): _separate(small)[0]}
    for inp in (big, small, big, small):
        out, _, _, _ = _small(inp, workspace=ws)
        assert torch.equal(out.view(torch.int16), ref[id(inp)].view(torch.int16))


def test_empty_batch():
    m = moe()
    say("small path T=0")
    inp = make_inputs(1, 4, 128, 128, 2, dtype="bf16", seed=0, device="cuda")
    for f in (0, m.FORWARD_ONE_KERNEL):
        out, ids, wts = m.forward_small(inp.logits[:0], inp.x[:0], inp.w1, inp.w2, 2, flags=f)
        assert out.shape == (0, 128) and ids.shape == (0, 2)
