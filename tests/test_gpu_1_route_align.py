"""GPU parity of routing (softmax + top-k) and alignment against the CPU
oracle: bit-exact ids and index lists, router weights within 1e-5."""
import numpy as np
import pytest
import torch

import oracle
from synth import draw_topk_ids
from tests.gpu_util import check_align, check_routing, moe, say

pytestmark = pytest.mark.gpu


def _logits(T, E, seed, kind="normal"):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":
        L = np.round(L * 2) / 2
        L[:, ::5] = 0.0
        L[:, 1::5] = -0.0
    return L


@pytest.mark.parametrize("n", [1, 2, 4, 5])
@pytest.mark.parametrize("renorm", [False, True])
def test_route_configs(n, renorm):
    from synth import CONFIGS
    from tests.gpu_util import cfg_inputs
    say(f"route config {n} renorm={renorm}")
    inp = cfg_inputs(n)
    ids, w = moe().route_topk(inp.logits, inp.k, renorm)
    torch.cuda.synchronize()
    ids_o, w_o = oracle.route(inp.host_logits(), inp.k, renorm)
    check_routing(ids, w, ids_o, w_o)
    if CONFIGS[n]["routing"] == "balanced":
        assert np.all(np.bincount(ids.cpu().numpy().ravel(), minlength=inp.E) == inp.S // inp.E)


@pytest.mark.parametrize("T,E,k,kind", [
    (1, 1, 1, "normal"), (3, 8, 8, "normal"), (7, 65, 3, "ties"), (33, 128, 8, "ties"),
    (5, 1024, 32, "normal"), (9, 1000, 7, "ties"), (257, 64, 6, "normal"), (5000, 100, 6, "ties"),
    (2, 300, 300, "ties")])
def test_route_edge_cases(T, E, k, kind):
    say(f"route T={T} E={E} k={k} {kind}")
    L = _logits(T, E, T * 31 + E, kind)
    if T > 2:
        L[2, :] = -np.inf
        L[2, E // 2] = 1.0                       # one finite logit, the rest -inf
    for renorm in (False, True):
        ids, w = moe().route_topk(torch.from_numpy(L).cuda(), k, renorm)
        torch.cuda.synchronize()
        check_routing(ids, w, *oracle.route(L, k, renorm))


def test_route_empty_batch():
    say("route T=0")
    ids, w = moe().route_topk(torch.empty((0, 8), device="cuda"), 2)
    torch.cuda.synchronize()
    assert ids.shape == (0, 2) and w.shape == (0, 2)


@pytest.mark.parametrize("block_m", [1, 2, 16, 64, 128, 256])
@pytest.mark.parametrize("T,E,k,kind", [
    (16, 64, 8, "uniform"), (64, 128, 8, "zipf"), (37, 16, 3, "uniform"), (100, 8, 2, "one"),
    (1, 1, 1, "uniform"), (4096, 128, 8, "uniform"), (777, 1024, 5, "zipf"),
    # around the limits of the one-thread-per-slot kernels (256 and 1024 slots), with up
    # to 1024 experts
    (16, 1024, 16, "zipf"), (32, 1024, 8, "uniform"), (257, 8, 1, "uniform"),
    (255, 3, 1, "one"), (128, 1024, 8, "zipf"), (1025, 8, 1, "uniform"), (512, 2, 2, "one")])
def test_align_bit_exact(T, E, k, kind, block_m):
    say(f"align T={T} E={E} k={k} {kind} block_m={block_m}")
    ids = draw_topk_ids(T, E, k, seed=T + E + block_m, kind=kind)
    al = moe().align_block(torch.from_numpy(ids).cuda(), E, block_m)
    torch.cuda.synchronize()
    check_align(al, ids, E, block_m, T * k)
    al2 = moe().align_block(torch.from_numpy(ids).cuda(), E, block_m)
    torch.cuda.synchronize()
    for a, b in zip(al, al2):
        assert torch.equal(a, b)                  # deterministic


def test_align_empty_batch():
    say("align T=0")
    sid, be, npad = moe().align_block(torch.empty((0, 4), dtype=torch.int32, device="cuda"), 8, 16)
    torch.cuda.synchronize()
    assert sid.numel() == 0 and be.numel() == 0 and int(npad.item()) == 0


def test_align_max_slots():
    # the largest batch the ABI accepts at k=8: T*k just below 2^24
    T, E, k, M = (1 << 21) - 1, 256, 8, 128
    say(f"align max T={T} E={E} k={k} M={M}")
    rng = np.random.default_rng(5)
    # slot j of every token draws from experts j, j+k, j+2k, ...: k distinct experts per token
    ids = np.stack([rng.integers(0, E // k, T) * k + j for j in range(k)], 1).astype(np.int32)
    al = moe().align_block(torch.from_numpy(ids).cuda(), E, M)
    torch.cuda.synchronize()
    sid, be, npad = (t.cpu().numpy() for t in al)
    flat = ids.ravel()
    counts = np.bincount(flat, minlength=E)
    n = int(npad[0])
    assert n == int(np.sum(-(-counts // M) * M))
    # property check at full size: stable order by (expert, slot), blocks single-expert
    order = np.argsort(flat, kind="stable")
    real = sid[:n][sid[:n] < T * k]
    assert np.array_equal(real, order)
    assert np.all(np.diff(be[:n // M]) >= 0)


@pytest.mark.parametrize("block_m", [1, 16, 64, 256])
@pytest.mark.parametrize("T,E,k,kind", [
    (1, 1, 1, "normal"), (8, 64, 8, "normal"), (5, 1024, 32, "normal"), (3, 65, 65, "ties"),
    (8, 1024, 512, "ties"),                       # 4096 slots: the largest single-launch batch
    (8, 1024, 64, "ties"), (8, 1024, 65, "ties"),  # 512 and 520 slots: both alignment bodies
    (9, 64, 8, "normal"), (16, 64, 8, "normal"),  # larger batches: the two-kernel path
    (16, 1024, 256, "ties"), (16, 1024, 65, "ties"), (17, 64, 8, "normal"),
    (64, 128, 8, "ties"), (300, 16, 4, "ties")])
def test_route_align_matches_separate_calls(T, E, k, kind, block_m):
    say(f"route_align T={T} E={E} k={k} {kind} block_m={block_m}")
    L = torch.from_numpy(_logits(T, E, T * 7 + E, kind)).cuda()
    for renorm in (False, True):
        fused = moe().route_align(L, k, block_m, renorm)
        ids, w = moe().route_topk(L, k, renorm)
        sep = (ids, w) + tuple(moe().align_block(ids, E, block_m))
        torch.cuda.synchronize()
        for a, b in zip(fused, sep):
            assert torch.equal(a, b)              # the same bits either way
        ids_o, w_o = oracle.route(L.cpu().numpy(), k, renorm)
        check_routing(fused[0], fused[1], ids_o, w_o)
        check_align(fused[2:], ids_o, E, block_m, T * k)


def test_route_align_empty_batch():
    say("route_align T=0")
    out = moe().route_align(torch.empty((0, 8), device="cuda"), 2, 16)
    torch.cuda.synchronize()
    assert out[0].shape == (0, 2) and int(out[4].item()) == 0
