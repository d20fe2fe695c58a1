"""Pins of the oracle's block-scaled FP8 variant: the group quantiser's closed
forms and its reduction to the per-row quantiser, and the whole FFN against a
loop-by-loop evaluation in the other order the method allows (each 128-block's
partial sum of codes, scaled by weight-block x activation-group scale), with
torch's e4m3fn cast as the quantiser and decoder."""
import numpy as np
import pytest
import torch

import oracle

B = 128


def test_quant_groups_closed_forms():
    v = np.zeros((2, 256), np.float32)
    v[0, :128] = np.linspace(-1.0, 4.0, 128, dtype=np.float32)   # absmax 4 in group 0
    v[0, 200] = -0.5                                               # absmax 0.5 in group 1
    v[1, 130] = 3e4                                                # group 0 of row 1 is zero
    q, s = oracle.quant_groups_e4m3(v)
    assert s.shape == (2, 2)
    assert s[0, 0] == np.float32(4.0) / np.float32(448.0) and q[0, 127] == 0x7E
    assert s[0, 1] == np.float32(0.5) / np.float32(448.0) and q[0, 200] == 0xFE
    assert s[1, 0] == 1.0 and np.all(q[1, :128] == 0)
    assert s[1, 1] == np.float32(3e4) / np.float32(448.0) and q[1, 130] == 0x7E
    # a group's codes do not depend on the other groups of the row
    w = v.copy()
    w[0, 5] = 1000.0
    q2, s2 = oracle.quant_groups_e4m3(w)
    assert np.array_equal(q2[0, 128:], q[0, 128:]) and s2[0, 1] == s[0, 1]


def test_quant_groups_of_whole_rows_is_the_row_quantiser():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((5, 384)) * rng.uniform(0.01, 100, (5, 1))).astype(np.float32)
    qg, sg = oracle.quant_groups_e4m3(v, group=384)
    qr, sr = oracle.quant_rows_e4m3(v)
    assert np.array_equal(qg, qr) and np.array_equal(sg[:, 0], sr)


def _torch_quant_groups(v32):
    """Independent group quantiser: torch float32 ops and torch's e4m3fn cast."""
    t = torch.from_numpy(np.ascontiguousarray(v32, np.float32))
    R, C = t.shape
    g = t.view(R, C // B, B)
    amax = g.abs().amax(dim=2)
    sc = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
    q = (g / sc[..., None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(R, C).to(torch.float64).numpy(), sc.to(torch.float64).numpy()


def _dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def _block_mm(wq, ws, aq, as_):
    """y[n] = sum_b ws[n//B, b] * as_[b] * sum_{c in b} wq[n, c] * aq[c] (decoded)."""
    N, K = wq.shape
    y = np.zeros(N)
    for n in range(N):
        acc = 0.0
        for b in range(K // B):
            part = float(np.dot(wq[n, b * B:(b + 1) * B], aq[b * B:(b + 1) * B]))
            acc += float(ws[n // B, b]) * float(as_[b]) * part
        y[n] = acc
    return y


def _block_case(seed, T=2, E=2, H=256, I=256):
    rng = np.random.default_rng(seed)
    w1q = rng.integers(0, 256, size=(E, 2 * I, H)).astype(np.uint8)
    w2q = rng.integers(0, 256, size=(E, H, I)).astype(np.uint8)
    w1q[(w1q & 0x7F) == 0x7F] = 0x3B
    w2q[(w2q & 0x7F) == 0x7F] = 0xBB
    w1q = np.where(np.abs(oracle.e4m3fn_decode(w1q)) > 16, 0x44, w1q).astype(np.uint8)
    w2q = np.where(np.abs(oracle.e4m3fn_decode(w2q)) > 16, 0xC4, w2q).astype(np.uint8)
    s1 = rng.uniform(0.002, 0.02, size=(E, 2 * I // B, H // B)).astype(np.float32)
    s2 = rng.uniform(0.002, 0.02, size=(E, H // B, I // B)).astype(np.float32)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[:, :B] *= 8.0                                  # groups of different absmax
    x_bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return x_bits, w1q, s1, w2q, s2


@pytest.mark.parametrize("seed,k", [(1, 1), (2, 2)])
def test_ffn_fp8_block_matches_blockwise_loops(seed, k):
    T, E, H, I = 2, 2, 256, 256
    x_bits, w1q, s1, w2q, s2 = _block_case(seed, T, E, H, I)
    rng = np.random.default_rng(seed + 10)
    ids, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    got = oracle.ffn_fp8_block(x_bits, lambda e: w1q[e], s1, lambda e: w2q[e], s2, ids, w)
    x32 = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    xq, xs = _torch_quant_groups(x32)
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            W1, W2 = _dec(w1q[e]), _dec(w2q[e])
            gu = _block_mm(W1, s1[e], xq[t], xs[t])
            g, u = gu[:I], gu[I:]
            h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
            hq, hs = _torch_quant_groups(h[None, :])
            ref[t] += float(w[t, j]) * _block_mm(W2, s2[e], hq[0], hs[0])
    assert np.allclose(got, ref, rtol=1e-9, atol=1e-12 * np.abs(ref).max())


def test_ffn_fp8_block_uniform_scales_equal_per_row_fp8():
    # weight block scales constant along K (= a per-row scale), every x group
    # with the same absmax as its row and I = 128 (one h group per slot): the
    # block-scaled layer is then the per-row W8A8 layer, value for value
    T, E, H, I, k = 3, 2, 256, 128, 2
    rng = np.random.default_rng(4)
    x_bits, w1q, _, w2q, _ = _block_case(4, T, E, H, I)
    x32 = rng.standard_normal((T, H)).astype(np.float32)
    x32[:, 7] = 9.0
    x32[:, 7 + B] = -9.0                              # equal absmax in both groups
    x_bits = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    r1 = rng.uniform(0.002, 0.02, size=(E, 2 * I // B)).astype(np.float32)
    r2 = rng.uniform(0.002, 0.02, size=(E, H // B)).astype(np.float32)
    s1 = np.repeat(r1[:, :, None], H // B, axis=2)
    s2 = np.repeat(r2[:, :, None], I // B, axis=2)
    ids, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    got = oracle.ffn_fp8_block(x_bits, lambda e: w1q[e], s1, lambda e: w2q[e], s2, ids, w)
    ref = oracle.ffn_fp8(x_bits, lambda e: w1q[e], np.repeat(r1, B, axis=1),
                         lambda e: w2q[e], np.repeat(r2, B, axis=1), ids, w)
    assert np.allclose(got, ref, rtol=1e-12, atol=0)
