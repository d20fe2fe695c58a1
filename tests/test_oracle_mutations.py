"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin catches each: evidence that the pins constrain every step."""
import numpy as np
import pytest

import oracle
import oracle.moe_oracle as om
from tests import test_oracle_block as B
from tests import test_oracle_ffn as F
from tests import test_oracle_formats as FM
from tests import test_oracle_route_align as R


def _fails(fn, *a):
    try:
        fn(*a)
    except Exception:
        return True
    return False


def _route_ascending(logits, k, renormalize=False):
    L = np.asarray(logits, np.float32)
    ids = np.argsort(L, axis=1, kind="stable")[:, :k].astype(np.int32)
    p = np.exp(L - L.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
    return ids, np.take_along_axis(p, ids.astype(np.int64), 1)


def _route_ties_high(logits, k, renormalize=False):
    L = np.asarray(logits, np.float32).astype(np.float64)
    E = L.shape[1]
    ids = np.array([(E - 1 - np.argsort(-r[::-1], kind="stable"))[:k] for r in L], np.int32)
    p = np.exp(L - L.max(1, keepdims=True)); p /= p.sum(1, keepdims=True)
    return ids, np.take_along_axis(p, ids.astype(np.int64), 1)


def _route_always_renorm(logits, k, renormalize=False):
    return MUT_ORIG_ROUTE(logits, k, True)


def _swiglu_swapped(w1e, w2e, xs):
    I = w2e.shape[1]
    return MUT_ORIG_SWIGLU(np.concatenate([w1e[I:], w1e[:I]]), w2e, xs)


def _swiglu_no_gate_factor(w1e, w2e, xs):
    I = w2e.shape[1]
    g, u = xs @ w1e[:I].T, xs @ w1e[I:].T
    return (1.0 / (1.0 + np.exp(-g)) * u) @ w2e.T


def _swiglu_w2_untransposed(w1e, w2e, xs):
    I = w2e.shape[1]
    g, u = xs @ w1e[:I].T, xs @ w1e[I:].T
    return (g / (1.0 + np.exp(-g)) * u) @ w2e.reshape(w2e.shape[1], w2e.shape[0])


def _align_pad_first(ids, E, block_m):
    s, b, n = MUT_ORIG_ALIGN(ids, E, block_m)
    S = np.asarray(ids).size
    out, i = [], 0
    while i < n:
        blk = list(s[i:i + block_m])
        real = [v for v in blk if v < S]
        out += [S] * (len(blk) - len(real)) + real
        i += block_m
    return np.array(out, np.int32), b, n


def _quant_447(v):
    v = np.asarray(v, np.float32)
    amax = np.max(np.abs(v), 1)
    scale = np.where(amax == 0, 1, amax / np.float32(447)).astype(np.float32)
    return om.e4m3fn_encode((v / scale[:, None]).astype(np.float32)), scale


def _encode_ties_away(v):
    c = MUT_ORIG_ENC(v)
    a = np.abs(np.asarray(v, np.float64))
    pos = oracle.E4M3FN_VALUES[:127]
    mids = (pos[:-1] + pos[1:]) / 2
    hit = np.isin(a, mids)
    idx = np.searchsorted(mids, a)
    up = np.minimum(idx + 1, 126).astype(np.uint8) | (c & 0x80)
    return np.where(hit, up, c).astype(np.uint8)


def _ffn_fp8_no_h_quant(x_bits, g1, s1, g2, s2, ids, w, tokens=None):
    orig = om.quant_rows_e4m3
    calls = {"n": 0}

    def q(v):
        calls["n"] += 1
        if calls["n"] == 1:
            return orig(v)
        v = np.asarray(v, np.float32)
        # identity "quantisation": scale 1 and exact values (decoded through a fake table)
        return v, np.ones(v.shape[0], np.float32)
    dec = om.e4m3fn_decode
    om.quant_rows_e4m3 = q
    om.e4m3fn_decode = lambda c: np.asarray(c, np.float64) if np.asarray(c).dtype != np.uint8 else dec(c)
    try:
        return MUT_ORIG_FFN_FP8(x_bits, g1, s1, g2, s2, ids, w, tokens)
    finally:
        om.quant_rows_e4m3 = orig
        om.e4m3fn_decode = dec


def _ffn_fp8_no_x_quant(x_bits, g1, s1, g2, s2, ids, w, tokens=None):
    orig = om.quant_rows_e4m3
    calls = {"n": 0}

    def q(v):
        calls["n"] += 1
        if calls["n"] == 1:
            v = np.asarray(v, np.float32)
            return v, np.ones(v.shape[0], np.float32)
        return orig(v)
    dec = om.e4m3fn_decode
    om.quant_rows_e4m3 = q
    om.e4m3fn_decode = lambda c: np.asarray(c, np.float64) if np.asarray(c).dtype != np.uint8 else dec(c)
    try:
        return MUT_ORIG_FFN_FP8(x_bits, g1, s1, g2, s2, ids, w, tokens)
    finally:
        om.quant_rows_e4m3 = orig
        om.e4m3fn_decode = dec


def _dequant_unscaled(codes, scale):
    return om.e4m3fn_decode(codes)


def _dequant_column_scale(codes, scale):
    c = om.e4m3fn_decode(codes)
    s = np.resize(np.asarray(scale, np.float64), c.shape[1])
    return c * s[None, :]


def _ffn_w8a16_quantises_x(x_bits, g1, s1, g2, s2, ids, w, tokens=None, num_experts=None):
    x = om.bf16_bits_to_f64(x_bits).astype(np.float32)
    q, a = om.quant_rows_e4m3(x)
    xq = (om.e4m3fn_decode(q) * a[:, None]).astype(np.float32)
    return MUT_ORIG_FFN_W8A16((xq.view(np.uint32) >> 16).astype(np.uint16), g1, s1, g2, s2, ids,
                              w, tokens, num_experts)


def _dequant_blocks_transposed(codes, scale, block=128):
    s = np.asarray(scale, np.float64).T
    return om.e4m3fn_decode(codes) * np.repeat(np.repeat(s, block, 0), block, 1)


def _quant_groups_whole_row(v, group=128):
    q, s = om.quant_rows_e4m3(v)
    return q, np.repeat(s[:, None], np.asarray(v).shape[1] // group, axis=1)


def _ffn_fp8_block_no_h_quant(x_bits, g1, s1, g2, s2, ids, w, tokens=None, num_experts=None):
    orig = om.quant_groups_e4m3
    calls = {"n": 0}

    def q(v, group=128):
        calls["n"] += 1
        if calls["n"] == 1:
            return orig(v, group)
        v = np.asarray(v, np.float32)
        return v, np.ones((v.shape[0], v.shape[1] // group), np.float32)
    dec = om.e4m3fn_decode
    om.quant_groups_e4m3 = q
    om.e4m3fn_decode = lambda c: np.asarray(c, np.float64) if np.asarray(c).dtype != np.uint8 else dec(c)
    try:
        return MUT_ORIG_FFN_FP8_BLOCK(x_bits, g1, s1, g2, s2, ids, w, tokens, num_experts)
    finally:
        om.quant_groups_e4m3 = orig
        om.e4m3fn_decode = dec


MUT_ORIG_ROUTE = om.route
MUT_ORIG_SWIGLU = om.swiglu_expert
MUT_ORIG_ALIGN = om.align
MUT_ORIG_ENC = om.e4m3fn_encode
MUT_ORIG_FFN_FP8 = om.ffn_fp8
MUT_ORIG_FFN_W8A16 = om.ffn_w8a16
MUT_ORIG_FFN_FP8_BLOCK = om.ffn_fp8_block

def _capacity_all_experts(S, E, block_m):
    cap = S + E * (block_m - 1)
    return -(-cap // block_m) * block_m


def _capacity_not_rounded(S, E, block_m):
    return S + min(E, S) * (block_m - 1)


MUTATIONS = [
    ("route", _route_ascending, [lambda: R.test_topk_ids_match_brute_force(7, 64, 8)]),
    ("route", _route_ties_high, [R.test_topk_hand_worked_ties]),
    ("route", _route_always_renorm, [R.test_softmax_weights_match_torch_softmax]),
    ("swiglu_expert", _swiglu_swapped, [lambda: F.test_ffn_matches_pure_python_brute_force(3, 4, 5, 7, 2)]),
    ("swiglu_expert", _swiglu_no_gate_factor, [F.test_ffn_closed_form_scalar]),
    ("swiglu_expert", _swiglu_w2_untransposed, [lambda: F.test_ffn_matches_pure_python_brute_force(3, 4, 5, 7, 2)]),
    ("align", _align_pad_first, [R.test_align_hand_worked]),
    ("quant_rows_e4m3", _quant_447, [F.test_quant_rows_closed_forms]),
    ("e4m3fn_encode", _encode_ties_away, [FM.test_e4m3fn_encode_midpoints_go_to_even_code]),
    ("ffn_fp8", _ffn_fp8_no_h_quant, [F.test_ffn_fp8_quantises_h_per_slot_on_grid]),
    ("ffn_fp8", _ffn_fp8_no_x_quant, [F.test_ffn_fp8_quantises_x_per_token]),
    ("dequant_rows", _dequant_unscaled,
     [lambda: F.test_ffn_w8a16_matches_brute_force_with_library_decode(2, 3, 5, 3, 2)]),
    ("dequant_rows", _dequant_column_scale,
     [lambda: F.test_ffn_w8a16_matches_brute_force_with_library_decode(3, 2, 4, 6, 1)]),
    ("dequant_blocks", _dequant_blocks_transposed,
     [lambda: B.test_ffn_fp8_block_matches_blockwise_loops(2, 2)]),
    ("quant_groups_e4m3", _quant_groups_whole_row,
     [B.test_quant_groups_closed_forms, lambda: B.test_ffn_fp8_block_matches_blockwise_loops(1, 1)]),
    ("ffn_fp8_block", _ffn_fp8_block_no_h_quant,
     [lambda: B.test_ffn_fp8_block_matches_blockwise_loops(1, 1)]),
    ("ffn_w8a16", _ffn_w8a16_quantises_x,
     [lambda: F.test_ffn_w8a16_matches_brute_force_with_library_decode(2, 3, 5, 3, 2)]),
    ("align_capacity", _capacity_all_experts,
     [lambda: R.test_align_capacity_hand_worked(4, 8, 16, 64)]),
    ("align_capacity", _capacity_not_rounded,
     [lambda: R.test_align_capacity_hand_worked(5, 2, 4, 12),
      lambda: R.test_align_capacity_bounds_every_routing(5, 2, 4)]),
]


@pytest.mark.parametrize("name,mut,pins", MUTATIONS, ids=[m[1].__name__ for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, mut, pins):
    # every pin passes on the real oracle ...
    for p in pins:
        p()
    # ... and at least one fails once the mistake is planted
    monkeypatch.setattr(om, name, mut)
    monkeypatch.setattr(oracle, name, mut)
    assert any(_fails(p) for p in pins)
