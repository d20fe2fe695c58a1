"""GPU parity of the whole path (route -> align -> FFN) against the CPU oracle
on the five workloads and on small ragged shapes; plus determinism, stage
splitting, the XCD-remap switch, guard bytes and token permutation."""
import numpy as np
import pytest
import torch

import oracle
from synth import config_inputs, make_inputs
from tests.gpu_util import (TOL, bench_block_m, cfg_inputs, check_align, check_finite,
                            check_routing, gpu_forward, moe, oracle_forward, oracle_full, out_f64,
                            say)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_config_parity(n):
    # every output row of every workload against the oracle, in the launch
    # configuration the bench times
    inp = cfg_inputs(n)
    bm = bench_block_m(inp)
    say(f"ffn config {n} ({inp.dtype}) T={inp.T} E={inp.E} H={inp.H} I={inp.I} k={inp.k} "
        f"block_m={bm}")
    ids, w, al, out = gpu_forward(inp, bm)
    check_finite(out)
    ids_o, w_o, ref = oracle_full(n)
    check_routing(ids, w, ids_o, w_o)
    check_align(al, ids_o, inp.E, bm, inp.S)
    got = out_f64(out)
    err = oracle.normwise_rel_err(got, ref)
    # reported, not a gate: elementwise relative error where |ref| >= 1e-3 max|ref|
    big = np.abs(ref) >= 1e-3 * np.max(np.abs(ref))
    elem = float(np.max(np.abs(got - ref)[big] / np.abs(ref)[big])) if big.any() else 0.0
    # the worst token row, so that a wrong tile shows where it is
    row_err = np.max(np.abs(got - ref), axis=1) / max(np.max(np.abs(ref)), 1e-300)
    say(f"  normwise rel err {err:.3e} (tol {TOL[inp.dtype]}); elementwise over "
        f"|ref| >= 1e-3 max: {elem:.3e}; worst row {int(np.argmax(row_err))}")
    if inp.dtype == "fp8":  # reported, not a gate: the format's own error
        master = cfg_inputs(2) if n == 3 else None
        if master is not None:
            r32 = oracle.ffn(oracle.bf16_bits_to_f64(inp.host_x()),
                             lambda e: oracle.bf16_bits_to_f64(master.host_w1(e)),
                             lambda e: oracle.bf16_bits_to_f64(master.host_w2(e)), ids_o, w_o)
            say(f"  vs the unquantised (bf16 master) layer: {oracle.normwise_rel_err(got, r32):.3e}")
    assert err <= TOL[inp.dtype]


TILES = {"dense": 0, "range": 1 << 10}  # default 128-row tiles / RANGE_GEMM 256 x 256 tiles


@pytest.mark.parametrize("tiles", list(TILES))
@pytest.mark.parametrize("block_m", [128, 256])
def test_prefill_workload_block_sizes(block_m, tiles):
    # the prefill workload through both prefill tilings at both block sizes
    # that take them, every output row against the oracle
    inp = cfg_inputs(5)
    say(f"ffn config 5 block_m={block_m} tiles={tiles}")
    ids, w, al, out = gpu_forward(inp, block_m, flags=TILES[tiles])
    check_finite(out)
    ids_o, w_o, ref = oracle_full(5)
    check_routing(ids, w, ids_o, w_o)
    check_align(al, ids_o, inp.E, block_m, inp.S)
    err = oracle.normwise_rel_err(out_f64(out), ref)
    say(f"  normwise rel err {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("block_m", [16, 64])
def test_prefill_workload_decode_kernels(block_m):
    # the 4096-token workload at decode block sizes, so the streaming kernels
    # with LDS-staged hot blocks run it: at 64 nearly every block is hot and
    # the hot-first queue orders ~640 blocks; at 16 there are more blocks
    # (> 2048) than the queue orders, so units go out in list order as quads;
    # every output row against the oracle
    inp = cfg_inputs(5)
    say(f"ffn config 5 block_m={block_m} (decode kernels)")
    ids, w, al, out = gpu_forward(inp, block_m)
    check_finite(out)
    ids_o, w_o, ref = oracle_full(5)
    check_routing(ids, w, ids_o, w_o)
    check_align(al, ids_o, inp.E, block_m, inp.S)
    assert int(al[2][0]) // block_m > (2048 if block_m == 16 else 0)
    err = oracle.normwise_rel_err(out_f64(out), ref)
    say(f"  normwise rel err {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("block_m", [128, 256])
def test_prefill_workload_fp8(block_m):
    # the prefill workload's shapes with e4m3 weights (per-row scales) and
    # per-token / per-slot activation scales: the grouped-GEMM tiles on the
    # fp8 MFMA, every output row against the oracle
    inp = config_inputs(5, device="cuda", dtype="fp8")
    say(f"ffn config 5 shapes fp8 block_m={block_m}")
    ids, w, al, out = gpu_forward(inp, block_m)
    check_finite(out)
    ids_o, w_o, ref = _oracle_prefill_fp8()
    check_routing(ids, w, ids_o, w_o)
    check_align(al, ids_o, inp.E, block_m, inp.S)
    err = oracle.normwise_rel_err(out_f64(out), ref)
    say(f"  normwise rel err {err:.3e} (tol {TOL['fp8']})")
    assert err <= TOL["fp8"]


_PREFILL_FP8 = []


def _oracle_prefill_fp8():
    if not _PREFILL_FP8:  # computed once per process (seconds of fp64 work)
        _PREFILL_FP8.append(oracle_forward(config_inputs(5, device="cuda", dtype="fp8")))
    return _PREFILL_FP8[0]


PREFILL_CASES = [  # T, E, H, I, k, routing: several row tiles, ragged blocks,
    (700, 8, 1024, 384, 2, "normal"),    # FC1 2I = 768: three 256-row tiles, ragged blocks
    (333, 4, 640, 512, 3, "zipf"),       # FC2 H = 640: two full and one half 256-row tile
    (129, 1, 256, 128, 1, "normal"),     # one expert: a full block and a 1-token block
]


@pytest.mark.parametrize("block_m", [128, 256])
@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "T{}_E{}_H{}_I{}_k{}_{}".format(*c))
def test_prefill_tiles_ragged_fp8(case, block_m):
    # fp8 through the grouped-GEMM tiles (H, I >= 256) or, for the one-expert
    # case with I = 128, the streaming kernels
    T, E, H, I, k, routing = case
    say(f"ffn prefill tiles fp8 T={T} E={E} H={H} I={I} k={k} {routing} block_m={block_m}")
    inp = make_inputs(T, E, H, I, k, dtype="fp8", routing=routing, seed=T + block_m + 1,
                      device="cuda")
    ids, w, al, out = gpu_forward(inp, block_m)
    check_finite(out)
    ids_o, w_o, ref = oracle_forward(inp)
    check_routing(ids, w, ids_o, w_o)
    check_align(al, ids_o, E, block_m, inp.S)
    err = oracle.normwise_rel_err(out_f64(out), ref)
    say(f"  normwise rel err {err:.3e}")
    assert err <= TOL["fp8"]


@pytest.mark.parametrize("tiles", list(TILES))
@pytest.mark.parametrize("block_m", [128, 256])
@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "T{}_E{}_H{}_I{}_k{}_{}".format(*c))
def test_prefill_tiles_ragged(case, block_m, tiles):
    T, E, H, I, k, routing = case
    say(f"ffn prefill tiles T={T} E={E} H={H} I={I} k={k} {routing} block_m={block_m} "
        f"tiles={tiles}")
    inp = make_inputs(T, E, H, I, k, dtype="bf16", routing=routing, seed=T + block_m,
                      device="cuda")
    ids, w, al, out = gpu_forward(inp, block_m, flags=TILES[tiles])
    check_finite(out)
    ids_o, w_o, ref = oracle_forward(inp)
    check_routing(ids, w, ids_o, w_o)
    check_align(al, ids_o, E, block_m, inp.S)
    err = oracle.normwise_rel_err(out_f64(out), ref)
    say(f"  normwise rel err {err:.3e}")
    assert err <= TOL["bf16"]


# Per-expert token counts at each block size that leave an expert's last
# block with 1, 16, 17, 32 and 33 tokens, give one expert three blocks (a
# 5-token last block), one expert no token and one a single partial block.
# The bf16 grouped-GEMM FC1 computes a last block of at most 32 tokens
# together with the block before it (one pass over the weights).
TAIL_COUNTS = {256: [257, 272, 273, 288, 289, 517, 0, 100],
               128: [129, 144, 145, 160, 161, 261, 0, 50]}


def _counted_logits(counts, seed):
    """Router logits of a top-2 routing in which expert e gets counts[e]
    slots: the slots sorted by expert are split in halves, token t takes
    entries t and t + T (distinct, since no count exceeds T), tokens shuffled."""
    lst = np.repeat(np.arange(len(counts)), counts)
    T = len(lst) // 2
    assert 2 * T == len(lst) and max(counts) <= T
    rng = np.random.default_rng(seed)
    perm = rng.permutation(T)
    logits = np.zeros((T, len(counts)), np.float32)
    logits[perm, lst[:T]] = 4.0
    logits[perm, lst[T:]] = 3.5
    return logits


@pytest.mark.parametrize("block_m", [128, 256])
def test_prefill_merged_tails(block_m):
    counts = TAIL_COUNTS[block_m]
    logits = _counted_logits(counts, block_m)
    T, E = logits.shape
    say(f"ffn merged tails T={T} E={E} k=2 block_m={block_m} counts={counts}")
    inp = make_inputs(T, E, 384, 256, 2, dtype="bf16", seed=block_m + 7, device="cuda",
                      logits=logits)
    ids, w, al, out = gpu_forward(inp, block_m)
    check_finite(out)
    ids_o, w_o, ref = oracle_forward(inp)
    assert np.array_equal(np.bincount(ids_o.ravel(), minlength=E), counts)
    check_routing(ids, w, ids_o, w_o)
    check_align(al, ids_o, E, block_m, inp.S)
    err = oracle.normwise_rel_err(out_f64(out), ref)
    say(f"  normwise rel err {err:.3e}")
    assert err <= TOL["bf16"]


ODD_CASES = [  # T, E, H, I, k, routing: H or I a multiple of 8 but not of 128
    (37, 6, 200, 136, 2, "normal"),
    (5, 3, 72, 40, 3, "normal"),
    (64, 8, 256, 200, 2, "zipf"),
    (300, 4, 136, 264, 2, "normal"),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("block_m", [16, 128])
@pytest.mark.parametrize("case", ODD_CASES, ids=lambda c: "T{}_E{}_H{}_I{}_k{}_{}".format(*c))
def test_odd_shapes_parity(case, block_m, dtype):
    # shapes past the 128-byte-line kernels run the wave-per-output path;
    # every row against the oracle, and the stages split over three calls on
    # one workspace give the same bits as one call
    T, E, H, I, k, routing = case
    say(f"ffn odd shape {dtype} T={T} E={E} H={H} I={I} k={k} {routing} block_m={block_m}")
    m = moe()
    inp = make_inputs(T, E, H, I, k, dtype=dtype, routing=routing, seed=T + H + block_m,
                      device="cuda")
    ids, w, al, out = gpu_forward(inp, block_m)
    check_finite(out)
    ids_o, w_o, ref = oracle_forward(inp)
    check_routing(ids, w, ids_o, w_o)
    err = oracle.normwise_rel_err(out_f64(out), ref)
    say(f"  normwise rel err {err:.3e}")
    assert err <= TOL[dtype]
    sid, be, npad = al
    call = (lambda **kw: m.ffn_fp8(inp.x, inp.w1, inp.w1_scale, inp.w2, inp.w2_scale, ids, w,
                                   sid, be, npad, block_m, **kw)) if dtype == "fp8" else \
        (lambda **kw: m.ffn_bf16(inp.x, inp.w1, inp.w2, ids, w, sid, be, npad, block_m, **kw))
    ws = m.alloc_workspace(T, E, H, I, k, block_m,
                           m.MOE_DTYPE_FP8 if dtype == "fp8" else m.MOE_DTYPE_BF16, "cuda")
    d = torch.empty_like(out)
    call(flags=m.STAGE_PREP, workspace=ws, out=d)
    call(flags=m.STAGE_FC1 | m.PREPARED, workspace=ws, out=d)
    call(flags=m.STAGE_FC2 | m.STAGE_COMBINE, workspace=ws, out=d)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), d.view(torch.int16))


CASES = [  # T, E, H, I, k, routing
    (37, 16, 256, 384, 3, "normal"),
    (5, 4, 128, 128, 4, "normal"),
    (200, 8, 512, 256, 2, "zipf"),
    (1, 1, 256, 128, 1, "normal"),
    # at most 16 tokens: the launch without LDS-staged passes, here with blocks
    # of 9..16 tokens that it serves in two 8-token passes
    (16, 2, 256, 128, 2, "normal"),
    (12, 3, 384, 256, 2, "zipf"),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32"])
@pytest.mark.parametrize("block_m", [1, 16, 64, 128])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "T{}_E{}_H{}_I{}_k{}_{}".format(*c))
def test_small_ragged_parity(case, block_m, dtype):
    T, E, H, I, k, routing = case
    say(f"ffn small {dtype} T={T} E={E} H={H} I={I} k={k} {routing} block_m={block_m}")
    inp = make_inputs(T, E, H, I, k, dtype=dtype, routing=routing, seed=T + E + block_m,
                      device="cuda")
    ids, w, al, out = gpu_forward(inp, block_m)
    check_finite(out)
    ids_o, w_o, ref = oracle_forward(inp)
    check_routing(ids, w, ids_o, w_o)
    check_align(al, ids_o, E, block_m, inp.S)
    err = oracle.normwise_rel_err(out_f64(out), ref)
    say(f"  normwise rel err {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_renormalized_weights(dtype):
    inp = make_inputs(24, 16, 256, 256, 4, dtype=dtype, routing="normal", seed=3, device="cuda")
    say(f"ffn renormalize {dtype}")
    ids, w, al, out = gpu_forward(inp, 16, renormalize=True)
    ids_o, w_o, ref = oracle_forward(inp, renormalize=True)
    check_routing(ids, w, ids_o, w_o)
    assert oracle.normwise_rel_err(out_f64(out), ref) <= TOL[dtype]


def test_all_tokens_to_one_expert_many_groups():
    # one expert holds every token: blocks of 256 slots, four 64-token groups each
    T, E, H, I, k = 300, 4, 256, 256, 1
    L = np.full((T, E), -1.0, np.float32)
    L[:, 2] = 1.0
    inp = make_inputs(T, E, H, I, k, dtype="bf16", seed=9, device="cuda", logits=L)
    say("ffn one hot expert, block_m=256")
    ids, w, al, out = gpu_forward(inp, 256)
    _, _, ref = oracle_forward(inp)
    assert oracle.normwise_rel_err(out_f64(out), ref) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("M", [16, 128])
def test_determinism_stages_remap_and_guards(dtype, M):
    # M = 16: the streaming kernels with LDS-staged hot blocks (40 tokens, zipf
    # routing); M = 128: the grouped-GEMM tiles; both schedule units from work
    # counters in the workspace
    m = moe()
    inp = make_inputs(40, 16, 512, 256, 4, dtype=dtype, routing="zipf", seed=4, device="cuda")
    say(f"ffn determinism/stages/remap/guards {dtype} block_m={M}")
    ids, w = m.route_topk(inp.logits, inp.k)
    sid, be, npad = m.align_block(ids, inp.E, M)
    call = (lambda **kw: m.ffn_fp8(inp.x, inp.w1, inp.w1_scale, inp.w2, inp.w2_scale, ids, w,
                                   sid, be, npad, M, **kw)) if dtype == "fp8" else \
        (lambda **kw: m.ffn_bf16(inp.x, inp.w1, inp.w2, ids, w, sid, be, npad, M, **kw))
    a = call()
    b = call()
    c = call(flags=m.NO_XCD_REMAP)
    ws = m.alloc_workspace(inp.T, inp.E, inp.H, inp.I, inp.k, M,
                           m.MOE_DTYPE_FP8 if dtype == "fp8" else m.MOE_DTYPE_BF16, "cuda")
    guard = torch.full((inp.T * inp.H + 2 * 64,), 0x7F7F, dtype=torch.int16, device="cuda")
    d = guard[64:64 + inp.T * inp.H].view(torch.bfloat16).view(inp.T, inp.H)
    call(flags=m.STAGE_FC1, workspace=ws, out=d)
    call(flags=m.STAGE_FC2, workspace=ws, out=d)
    call(flags=m.STAGE_COMBINE, workspace=ws, out=d)
    # FC2 alone again, twice: each call continues from the FC1 call's h and
    # work counters (an FC2 launch leaves its counters cleared)
    e = torch.empty_like(d)
    call(flags=m.STAGE_FC2, workspace=ws, out=e)
    call(flags=m.STAGE_FC2 | m.STAGE_COMBINE, workspace=ws, out=e)
    # PREP in a call of its own, FC1 after it without (MOE_FFN_PREPARED)
    f = torch.empty_like(d)
    call(flags=m.STAGE_PREP, workspace=ws, out=f)
    call(flags=m.STAGE_FC1 | m.PREPARED, workspace=ws, out=f)
    call(flags=m.STAGE_FC2 | m.STAGE_COMBINE, workspace=ws, out=f)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    assert torch.equal(a.view(torch.int16), d.view(torch.int16))
    assert torch.equal(a.view(torch.int16), e.view(torch.int16))
    assert torch.equal(a.view(torch.int16), f.view(torch.int16))
    g = guard.cpu().numpy()
    assert np.all(g[:64] == 0x7F7F) and np.all(g[64 + inp.T * inp.H:] == 0x7F7F)


def test_token_permutation():
    inp = make_inputs(48, 16, 256, 256, 4, dtype="bf16", routing="normal", seed=8, device="cuda")
    say("ffn token permutation")
    _, _, _, out = gpu_forward(inp, 16)
    perm = torch.from_numpy(np.random.default_rng(1).permutation(inp.T)).cuda()
    inp_p = make_inputs(48, 16, 256, 256, 4, dtype="bf16", seed=8, device="cuda",
                        logits=inp.host_logits()[perm.cpu().numpy()])
    inp_p.x = inp.x[perm].contiguous()
    inp_p.w1, inp_p.w2 = inp.w1, inp.w2
    _, _, _, out_p = gpu_forward(inp_p, 16)
    err = oracle.normwise_rel_err(out_f64(out_p), out_f64(out)[perm.cpu().numpy()])
    assert err <= 1e-6


def test_empty_batch():
    m = moe()
    say("ffn T=0")
    inp = make_inputs(1, 4, 128, 128, 2, dtype="bf16", seed=0, device="cuda")
    x = inp.x[:0]
    ids = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    sid, be, npad = m.align_block(ids, 4, 16)
    out = m.ffn_bf16(x, inp.w1, inp.w2, ids, w, sid, be, npad, 16)
    torch.cuda.synchronize()
    assert out.shape == (0, 128)
