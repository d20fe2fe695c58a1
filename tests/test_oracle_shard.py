"""Pins of the oracle's per-shard results (expert and tensor parallel shares of
the Vera Rubin page's "Locality domain" per-rank comparison): the shards'
partial outputs add up to the whole layer, and alignment leaves out slots of
experts served elsewhere."""
import numpy as np
import pytest

import oracle


def _layer(T=6, E=8, H=20, I=12, k=3, seed=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((E, 2 * I, H)) / 4
    w2 = rng.standard_normal((E, H, I)) / 4
    ids, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    return x, w1, w2, ids, w


@pytest.mark.parametrize("G", [2, 4])
def test_expert_shards_sum_to_the_layer(G):
    x, w1, w2, ids, w = _layer()
    E = w1.shape[0]
    full = oracle.ffn(x, lambda e: w1[e], lambda e: w2[e], ids, w)
    El = E // G
    parts = []
    for r in range(G):
        loc = ids - r * El                       # remote experts fall outside [0, El)
        parts.append(oracle.ffn(x, lambda e: w1[r * El + e], lambda e: w2[r * El + e], loc, w,
                                num_experts=El))
    assert np.allclose(sum(parts), full, rtol=1e-12, atol=1e-12)
    # a shard with no local slot contributes exactly zero
    assert not np.any(oracle.ffn(x, lambda e: w1[e], lambda e: w2[e], ids + E, w,
                                 num_experts=E))


@pytest.mark.parametrize("G", [2, 4])
def test_tensor_shards_sum_to_the_layer(G):
    x, w1, w2, ids, w = _layer(I=16)
    I = w2.shape[2]
    full = oracle.ffn(x, lambda e: w1[e], lambda e: w2[e], ids, w)
    c = I // G
    parts = []
    for r in range(G):
        sl = slice(r * c, (r + 1) * c)
        g1 = lambda e: np.concatenate([w1[e, :I][sl], w1[e, I:][sl]])   # gate|up rows of the slice
        g2 = lambda e: w2[e][:, sl]
        parts.append(oracle.ffn(x, g1, g2, ids, w))
    assert np.allclose(sum(parts), full, rtol=1e-12, atol=1e-12)


def test_fp8_expert_shards_sum_to_the_layer():
    # per-slot quantisation of h does not depend on which shard holds the expert
    rng = np.random.default_rng(4)
    T, E, H, I, k = 5, 4, 32, 16, 2
    xb = (rng.standard_normal((T, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w1q = rng.integers(0, 0x7f, (E, 2 * I, H)).astype(np.uint8)
    w2q = rng.integers(0, 0x7f, (E, H, I)).astype(np.uint8)
    s1 = rng.uniform(0.001, 0.01, (E, 2 * I)).astype(np.float32)
    s2 = rng.uniform(0.001, 0.01, (E, H)).astype(np.float32)
    ids, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    full = oracle.ffn_fp8(xb, lambda e: w1q[e], s1, lambda e: w2q[e], s2, ids, w)
    half = E // 2
    parts = [oracle.ffn_fp8(xb, lambda e: w1q[r * half + e], s1[r * half:], lambda e: w2q[r * half + e],
                            s2[r * half:], ids - r * half, w, num_experts=half) for r in range(2)]
    assert np.allclose(parts[0] + parts[1], full, rtol=1e-12, atol=1e-12)


def test_align_leaves_out_remote_slots_brute_force():
    rng = np.random.default_rng(7)
    T, k, E, M = 9, 3, 5, 4
    ids = rng.integers(-3, E + 3, (T, k)).astype(np.int32)     # about half remote
    sid, be, n = oracle.align(ids, E, M)
    flat = ids.ravel()
    local = sorted((int(flat[s]), s) for s in range(flat.size) if 0 <= flat[s] < E)
    expect, blocks = [], []
    for e in range(E):
        run = [s for (ee, s) in local if ee == e]
        if not run:
            continue
        pad = (-len(run)) % M
        expect += run + [flat.size] * pad
        blocks += [e] * ((len(run) + pad) // M)
    assert n == len(expect) and sid.tolist() == expect and be.tolist() == blocks
