"""Pins of the oracle's routing (softmax + top-k) and alignment against brute
force, hand-worked cases, library softmax and invariants."""
import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs


def brute_topk(L, k):
    """Full lexicographic sort of (-logit, expert) per token, pure Python."""
    out = []
    for row in L:
        keys = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
        out.append(keys[:k])
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (5, 8, 2), (7, 64, 8), (3, 128, 128), (33, 96, 5)])
def test_topk_ids_match_brute_force(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[:, ::7] = np.round(L[:, ::7])          # plenty of exact ties
    ids, _ = oracle.route(L, k)
    assert np.array_equal(ids, brute_topk(L, k))


def test_topk_hand_worked_ties():
    # equal logits -> lower index first; -0.0 ties with +0.0; -inf sorts last
    L = np.array([[1.0, 3.0, 3.0, -0.0, 0.0, 2.0, -np.inf, 2.0]], dtype=np.float32)
    ids, _ = oracle.route(L, 7)
    assert ids.tolist() == [[1, 2, 5, 7, 0, 3, 4]]
    ids, _ = oracle.route(L, 8)
    assert ids.tolist() == [[1, 2, 5, 7, 0, 3, 4, 6]]


def test_softmax_weights_match_torch_softmax():
    rng = np.random.default_rng(3)
    L = (rng.standard_normal((9, 40)) * 4).astype(np.float32)
    ids, w = oracle.route(L, 6)
    p = torch.softmax(torch.from_numpy(L).double(), dim=-1).numpy()
    assert np.allclose(w, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-14, atol=0)
    ids2, w2 = oracle.route(L, 6, renormalize=True)
    assert np.array_equal(ids, ids2)
    assert np.allclose(w2.sum(1), 1.0, rtol=1e-14)
    assert np.allclose(w2, w / w.sum(1, keepdims=True), rtol=1e-14)


def test_softmax_closed_forms():
    # logits (0, ln 3): p = (1/4, 3/4) up to the float32 rounding of ln 3
    L = np.array([[0.0, np.log(3.0)]], dtype=np.float32)
    ids, w = oracle.route(L, 2)
    assert ids.tolist() == [[1, 0]]
    assert w[0, 0] == pytest.approx(0.75, abs=1e-7) and w[0, 1] == pytest.approx(0.25, abs=1e-7)
    # E = 1: the only expert, weight 1
    ids, w = oracle.route(np.array([[5.0], [-3.0]], np.float32), 1)
    assert ids.tolist() == [[0], [0]] and np.all(w == 1.0)
    # k = E: a permutation and the weights sum to 1 without renormalising
    L = np.random.default_rng(4).standard_normal((4, 10)).astype(np.float32)
    ids, w = oracle.route(L, 10)
    assert all(sorted(r) == list(range(10)) for r in ids.tolist())
    assert np.allclose(w.sum(1), 1.0, rtol=1e-14)
    # large logits do not overflow (max subtraction)
    ids, w = oracle.route(np.array([[1000.0, 999.0]], np.float32), 2)
    assert w[0, 0] == pytest.approx(1 / (1 + np.exp(-1.0)), rel=1e-12)


def test_balanced_routing_gives_two_slots_per_expert():
    inp = make_inputs(16, 64, 128, 128, 8, dtype="bf16", routing="balanced", seed=0)
    ids, _ = oracle.route(inp.host_logits(), 8)
    assert np.array_equal(np.bincount(ids.reshape(-1), minlength=64), np.full(64, 2))


def brute_align(ids, E, M):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    S = len(flat)
    order = sorted(range(S), key=lambda s: (flat[s], s))     # stable sort by expert
    sorted_ids, blocks = [], []
    i = 0
    while i < S:
        e = flat[order[i]]
        run = []
        while i < S and flat[order[i]] == e:
            run.append(order[i])
            i += 1
        padded = len(run) + (-len(run)) % M
        sorted_ids += run + [S] * (padded - len(run))
        blocks += [e] * (padded // M)
    return sorted_ids, blocks, len(sorted_ids)


@pytest.mark.parametrize("M", [1, 2, 16, 64, 128])
@pytest.mark.parametrize("T,E,k", [(1, 4, 1), (4, 8, 2), (16, 64, 8), (37, 16, 3)])
def test_align_matches_brute_force(T, E, k, M):
    rng = np.random.default_rng(T + E + k + M)
    L = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = oracle.route(L, k)
    s, b, n = oracle.align(ids, E, M)
    bs, bb, bn = brute_align(ids, E, M)
    assert s.tolist() == bs and b.tolist() == bb and n == bn
    assert n <= oracle.align_capacity(T * k, E, M)


def test_align_hand_worked():
    # ids (T=3, k=2): slots 0..5 -> experts 2,0 | 2,1 | 0,2 ; E=4, M=2
    ids = np.array([[2, 0], [2, 1], [0, 2]], dtype=np.int32)
    s, b, n = oracle.align(ids, 4, 2)
    # expert 0: slots 1,4 ; expert 1: slot 3 + pad ; expert 2: slots 0,2,5 + pad ; expert 3: none
    assert s.tolist() == [1, 4, 3, 6, 0, 2, 5, 6]
    assert b.tolist() == [0, 1, 2, 2]
    assert n == 8
    s, b, n = oracle.align(ids, 4, 1)
    assert s.tolist() == [1, 4, 3, 0, 2, 5] and b.tolist() == [0, 0, 1, 2, 2, 2] and n == 6


def test_align_invariants_large():
    rng = np.random.default_rng(9)
    T, E, k, M = 512, 128, 8, 64
    ids, _ = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    s, b, n = oracle.align(ids, E, M)
    S = T * k
    counts = np.bincount(ids.reshape(-1), minlength=E)
    real = s[s < S]
    assert np.array_equal(np.sort(real), np.arange(S))              # a permutation of slots
    assert n == int(np.sum(-(-counts // M) * M))                     # padded total
    assert np.all(np.diff(b) >= 0)                                   # block experts ascending
    for blk in range(n // M):                                        # each block single-expert
        rows = s[blk * M:(blk + 1) * M]
        valid = rows[rows < S]
        assert np.all(ids.reshape(-1)[valid] == b[blk])
        # padding only after an expert's run: valid entries form a prefix
        assert np.all(rows[:valid.size] < S)


# align_capacity: the length the caller allocates for sorted_ids. Worked by
# hand from its definition (every active expert, of which there are at most
# min(E, S), pads its run by fewer than block_m entries; the total is rounded
# up to a whole block), one case per branch of that definition.
@pytest.mark.parametrize("S,E,M,want", [
    (4, 8, 16, 64),     # S < E: 4 active at most -> 4 + 4*15 = 64, already a multiple of 16
    (128, 64, 64, 4160),  # S >= E: 128 + 64*63 = 4160 = 65*64
    (7, 3, 1, 7),       # M = 1: no padding at all
    (5, 2, 4, 12),      # 5 + 2*3 = 11, rounded up to 12
    (6, 2, 4, 12),      # 6 + 2*3 = 12: an exact multiple stays as it is
    (0, 8, 16, 0),      # no slot, no block
    (1, 1024, 256, 256),  # one slot: one block
])
def test_align_capacity_hand_worked(S, E, M, want):
    assert oracle.align_capacity(S, E, M) == want


def _compositions(S, E):
    """Every way of giving S slots to E experts (count vectors)."""
    if E == 1:
        yield (S,)
        return
    for c in range(S + 1):
        for rest in _compositions(S - c, E - 1):
            yield (c,) + rest


@pytest.mark.parametrize("S,E,M", [(5, 2, 4), (6, 3, 4), (7, 4, 2), (3, 5, 8), (8, 3, 3)])
def test_align_capacity_bounds_every_routing(S, E, M):
    # brute force over all expert-count vectors: the padded length of any
    # routing fits, and the capacity is a whole number of blocks
    cap = oracle.align_capacity(S, E, M)
    assert cap % M == 0
    worst = max(sum(-(-c // M) * M for c in cnt) for cnt in _compositions(S, E))
    assert worst <= cap
    # the bound is not loose by a whole block per expert
    assert cap - worst < min(E, S) * M
