"""Shared helpers of the GPU parity tests: run the HIP path through the
binding, run the CPU oracle on the same seeded inputs, compare."""
import functools
import sys

import numpy as np
import torch

import oracle
from synth import config_inputs, make_inputs  # noqa: F401

TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 5e-2}   # normwise max relative error of the output
WEIGHT_ATOL = 1e-5                               # router weights, absolute


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def moe():
    import moe_expert_ffn_router_amd as m
    return m


@functools.lru_cache(maxsize=None)
def cfg_inputs(n: int):
    return config_inputs(n, device="cuda")


def oracle_forward(inp, tokens=None, renormalize=False):
    """Oracle routing and output rows for ``tokens`` (all by default)."""
    ids, w = oracle.route(inp.host_logits(), inp.k, renormalize)
    if inp.dtype == "fp8":
        out = oracle.ffn_fp8(inp.host_x(), inp.host_w1, inp.host_w1_scale(), inp.host_w2,
                             inp.host_w2_scale(), ids, w, tokens)
    elif inp.dtype == "bf16":
        out = oracle.ffn(oracle.bf16_bits_to_f64(inp.host_x()),
                         lambda e: oracle.bf16_bits_to_f64(inp.host_w1(e)),
                         lambda e: oracle.bf16_bits_to_f64(inp.host_w2(e)), ids, w, tokens)
    else:
        out = oracle.ffn(inp.host_x().astype(np.float64),
                         lambda e: inp.host_w1(e).astype(np.float64),
                         lambda e: inp.host_w2(e).astype(np.float64), ids, w, tokens)
    return ids, w, out


@functools.lru_cache(maxsize=None)
def oracle_full(n: int):
    """Oracle routing and every output row of workload n (cached: the two
    largest workloads take seconds of fp64 work, and several tests compare
    against the same layer)."""
    return oracle_forward(cfg_inputs(n))


def check_finite(out: torch.Tensor) -> None:
    """Every element of the GPU output is finite (checked on all rows, also
    where only a subset is compared)."""
    assert bool(torch.isfinite(out.float()).all()), "non-finite values in the GPU output"


def bench_block_m(inp) -> int:
    """The block size bench.py times for this workload."""
    return moe().default_block_m(inp.T, inp.E, inp.k)


def gpu_forward(inp, block_m=None, renormalize=False, flags=0):
    m = moe()
    if block_m is None:
        block_m = bench_block_m(inp)
    ids, w, sid, be, npad = m.route_align(inp.logits, inp.k, block_m, renormalize)
    if inp.dtype == "fp8":
        out = m.ffn_fp8(inp.x, inp.w1, inp.w1_scale, inp.w2, inp.w2_scale, ids, w, sid, be, npad,
                        block_m, flags)
    elif inp.dtype == "bf16":
        out = m.ffn_bf16(inp.x, inp.w1, inp.w2, ids, w, sid, be, npad, block_m, flags)
    else:
        out = m.ffn_f32(inp.x, inp.w1, inp.w2, ids, w, sid, be, npad, block_m, flags)
    torch.cuda.synchronize()
    return ids, w, (sid, be, npad), out


def out_f64(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64)


def check_routing(ids_g, w_g, ids_o, w_o):
    assert np.array_equal(ids_g.cpu().numpy(), ids_o), "topk_ids differ"
    err = float(np.max(np.abs(w_g.cpu().numpy().astype(np.float64) - w_o))) if w_o.size else 0.0
    assert err <= WEIGHT_ATOL, f"topk_weights max abs err {err}"


def check_align(al, ids_host, E, block_m, S):
    sid, be, npad = (t.cpu().numpy() for t in al)
    s_o, b_o, n_o = oracle.align(ids_host, E, block_m)
    n = int(npad[0])
    assert n == n_o, f"num_padded {n} != {n_o}"
    assert np.array_equal(sid[:n], s_o), "sorted_ids differ"
    assert np.array_equal(be[:n // block_m], b_o), "block_expert differ"
    assert np.all(sid[n:] == S), "sorted_ids tail is not the sentinel"
    assert np.all(be[n // block_m:] == -1), "block_expert tail is not -1"
