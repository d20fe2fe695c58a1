"""GPU parity of one rank's share of the layer on one GPU (the per-rank FC1+FC2
of the Vera Rubin page's "Locality domain" comparison at EP2/EP4/TP2/TP4):
expert-parallel shards hold E/G local experts and see the other experts'
slots as ids outside [0, E/G); tensor-parallel shards hold an I/G slice of
every expert. Each shard is checked against the oracle's partial sum, and the
shards' sum against the whole layer."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import (TOL, cfg_inputs, check_finite, check_routing, moe, oracle_full,
                            out_f64, say)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,G", [(2, 2), (2, 4), (3, 2), (3, 4), (4, 2), (4, 4), (5, 2)])
def test_expert_parallel_shards(n, G):
    inp = cfg_inputs(n)
    m = moe()
    E, k = inp.E, inp.k
    El = E // G
    bm = m.default_block_m(inp.T, El, k)
    say(f"EP{G} workload {n} ({inp.dtype}) E_local={El} block_m={bm}")
    ids, w = m.route_topk(inp.logits, k)
    torch.cuda.synchronize()
    ids_o, w_o = oracle.route(inp.host_logits(), k)
    check_routing(ids, w, ids_o, w_o)
    total = 0.0
    for r in range(G):
        lo = r * El
        loc = (ids - lo).contiguous()            # remote experts fall outside [0, El)
        sid, be, npad = m.align_block(loc, El, bm)
        w1, w2 = inp.w1[lo:lo + El], inp.w2[lo:lo + El]
        if inp.dtype == "fp8":
            s1, s2 = inp.w1_scale[lo:lo + El], inp.w2_scale[lo:lo + El]
            out = m.ffn_fp8(inp.x, w1, s1, w2, s2, loc, w, sid, be, npad, bm)
            ref = oracle.ffn_fp8(inp.host_x(), lambda e: inp.host_w1(lo + e),
                                 inp.host_w1_scale()[lo:], lambda e: inp.host_w2(lo + e),
                                 inp.host_w2_scale()[lo:], ids_o - lo, w_o,
                                 num_experts=El)
        else:
            out = m.ffn_bf16(inp.x, w1, w2, loc, w, sid, be, npad, bm)
            ref = oracle.ffn(oracle.bf16_bits_to_f64(inp.host_x()),
                             lambda e: oracle.bf16_bits_to_f64(inp.host_w1(lo + e)),
                             lambda e: oracle.bf16_bits_to_f64(inp.host_w2(lo + e)),
                             ids_o - lo, w_o, num_experts=El)
        torch.cuda.synchronize()
        check_finite(out)
        got = out_f64(out)
        err = oracle.normwise_rel_err(got, ref)
        say(f"  rank {r}: normwise rel err {err:.3e}")
        assert err <= TOL[inp.dtype]
        total = total + got
    full = oracle_full(n)[2]
    err = oracle.normwise_rel_err(total, full)
    say(f"  sum of shards vs layer: {err:.3e}")
    assert err <= TOL[inp.dtype]


@pytest.mark.parametrize("n,G", [(2, 2), (2, 4), (4, 2), (5, 2)])
def test_tensor_parallel_shards(n, G):
    # bf16 only: an fp8 shard would quantise h per slice of its row, which is
    # a different quantisation of the layer, not a share of it
    inp = cfg_inputs(n)
    m = moe()
    I, k = inp.I, inp.k
    c = I // G
    bm = m.default_block_m(inp.T, inp.E, k)
    say(f"TP{G} workload {n} I_local={c} block_m={bm}")
    ids, w, sid, be, npad = m.route_align(inp.logits, k, bm)
    ids_o, w_o = oracle.route(inp.host_logits(), k)
    x64 = oracle.bf16_bits_to_f64(inp.host_x())
    total = 0.0
    for r in range(G):
        sl = slice(r * c, (r + 1) * c)
        w1 = torch.cat([inp.w1[:, sl], inp.w1[:, I + r * c:I + (r + 1) * c]], 1).contiguous()
        w2 = inp.w2[:, :, sl].contiguous()
        out = m.ffn_bf16(inp.x, w1, w2, ids, w, sid, be, npad, bm)

        def g1(e, sl=sl):
            a = oracle.bf16_bits_to_f64(inp.host_w1(e))
            return np.concatenate([a[:I][sl], a[I:][sl]])

        def g2(e, sl=sl):
            return oracle.bf16_bits_to_f64(inp.host_w2(e))[:, sl]

        ref = oracle.ffn(x64, g1, g2, ids_o, w_o)
        torch.cuda.synchronize()
        check_finite(out)
        got = out_f64(out)
        err = oracle.normwise_rel_err(got, ref)
        say(f"  rank {r}: normwise rel err {err:.3e}")
        assert err <= TOL["bf16"]
        total = total + got
        del w1, w2
    full = oracle_full(n)[2]
    err = oracle.normwise_rel_err(total, full)
    say(f"  sum of shards vs layer: {err:.3e}")
    assert err <= TOL["bf16"]
