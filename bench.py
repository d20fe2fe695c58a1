"""Benchmark of the fused MoE expert FFN hot path on one MI355X.

One step = one pass of the whole path over one batch: router softmax + top-k
and token-to-expert alignment (moe_route_align), FC1 (gate|up) + SiLU*up, FC2, top-k weighted
combine, all in libmoe.so's HIP kernels on torch's current stream. Inputs and
weights are resident in HBM before the timed region; outputs and workspace are
allocated once, outside it.

Default workload: decode, bf16, T=16 tokens, E=64 experts, H=4096, I=1536,
top-8, balanced routing (every expert gets 2 slots), seed 0.

Prints one JSON line: tokens/s of the whole step, the HBM roofline of the
dominant kernel (FC1, timed live with HIP events on the same stream), and the
CPU oracle timed on a bounded sample of the same workload.

Warm-up: the --warmup steps, then more untimed steps until at least
MIN_WARMUP_S of warm-up have run. MI355X needs that long under load to reach
its steady clocks: 20 timed decode steps after 5 warm-up steps (2 ms) measured
0.400 ms per step and FC1 at 0.258 ms, after 100 (38 ms) 0.375 and 0.239 ms,
the rate of long runs. The line reports both counts.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE FC1+FC2 layer tokens/s; expert-weight HBM GB/s (% of peak) at decode"
MIN_WARMUP_S = 0.05
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2516.6
MFMA_FP8_PEAK_TFLOPS = 5033.2  # dense (no 2:1 sparsity)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload number 1..5 (default 2)")
    ap.add_argument("--block-m", type=int, default=0,
                    help="block size; 0 = moe_default_block_m for the workload")
    ap.add_argument("--flags", type=int, default=0, help="extra moe_ffn flags (e.g. 256 = no XCD remap)")
    ap.add_argument("--ep", type=int, default=1,
                    help="time one expert-parallel rank's share: rank 0 of G holds experts "
                         "[0, E/G); slots of the other experts are remote")
    ap.add_argument("--tp", type=int, default=1,
                    help="time one tensor-parallel rank's share: rank 0 of G holds the "
                         "first I/G columns of every expert (FC2 gives a partial sum)")
    ap.add_argument("--weight-only", action="store_true",
                    help="FP8 workloads: run the weight-only (W8A16) FFN on the same codes "
                         "and scales, activations kept in bf16")
    ap.add_argument("--block-fp8", action="store_true",
                    help="FP8 workloads: weights quantised per 128x128 block (same master "
                         "weights), activations per 128-element group")
    ap.add_argument("--fp8", action="store_true",
                    help="bf16 workloads: the same shapes and master weights quantised to e4m3 "
                         "(per-row scales), activations per token / per slot (moe_ffn_fp8)")
    ap.add_argument("--single-launch", action="store_true",
                    help="T <= 16: the whole layer as one cooperative launch (moe_forward_small "
                         "with FORWARD_ONE_KERNEL)")
    ap.add_argument("--small-path", action="store_true",
                    help="T <= 64: the whole layer through one moe_forward_small call "
                         "(separate launches; no alignment step up to 16 tokens)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-stride", type=int, default=0,
                    help="bracket FC1 with timing events on every N-th timed step "
                         "(0: max(1, steps // 10), so every run has ten samples or more)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed region, copy a buffer of this many MiB 3 times "
                         "(a plain copy kernel of known size, to calibrate HBM counters)")
    return ap.parse_args()


def source_digest() -> str:
    """Hash of the sources the FFN kernels are compiled from (moe_ffn.hip and the
    headers), so that measured counters stay tied to the kernels they measured."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "moe_expert_ffn_router_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f == "moe_ffn.hip" or f.endswith(".h"):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    with open(os.path.join(ROOT, "include", "moe.h"), "rb") as fh:
        h.update(b"moe.h" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f).get(f"{kernel}@{workload}")
    if not rec or rec.get("source_digest") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, target_s: float, weight_only: bool = False):
    # inp.dtype "fp8_block" selects the block-scaled oracle
    """The CPU oracle as it stands, on the first n tokens of the same workload;
    n grows until about target_s seconds of oracle work have been timed."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas_threads = 1
    logits = inp.host_logits()
    x_bits = inp.host_x()
    # host copies of the weights of the experts the sample can touch (not timed)
    ids_all, _ = oracle.route(logits, inp.k)
    w1h, w2h = {}, {}
    t_spent, n, per_tok = 0.0, 0, []
    sample_out = None
    reps, t_full = 0, 0.0  # whole-batch evaluations, once n reaches T
    while (n < inp.T and t_spent < target_s) or (n == inp.T and t_full < target_s):
        n_next = min(inp.T, max(n + 1, 2 * n))
        for e in np.unique(ids_all[:n_next]):
            e = int(e)
            if e not in w1h:
                w1h[e], w2h[e] = inp.host_w1(e), inp.host_w2(e)
        toks = list(range(n_next))
        t0 = time.perf_counter()
        ids, w = oracle.route(logits[:n_next], inp.k)
        if inp.dtype == "fp8_block":
            sample_out = oracle.ffn_fp8_block(x_bits[:n_next], w1h.__getitem__,
                                              inp.host_w1_scale(), w2h.__getitem__,
                                              inp.host_w2_scale(), ids, w, toks)
        elif inp.dtype == "fp8" and weight_only:
            sample_out = oracle.ffn_w8a16(x_bits[:n_next], w1h.__getitem__,
                                          inp.host_w1_scale(), w2h.__getitem__,
                                          inp.host_w2_scale(), ids, w, toks)
        elif inp.dtype == "fp8":
            sample_out = oracle.ffn_fp8(x_bits[:n_next], w1h.__getitem__, inp.host_w1_scale(),
                                        w2h.__getitem__, inp.host_w2_scale(), ids, w, toks)
        elif inp.dtype == "bf16":
            sample_out = oracle.ffn(oracle.bf16_bits_to_f64(x_bits[:n_next]),
                                    lambda e: oracle.bf16_bits_to_f64(w1h[e]),
                                    lambda e: oracle.bf16_bits_to_f64(w2h[e]), ids, w, toks)
        else:
            sample_out = oracle.ffn(x_bits[:n_next].astype(np.float64),
                                    lambda e: w1h[e].astype(np.float64),
                                    lambda e: w2h[e].astype(np.float64), ids, w, toks)
        dt = time.perf_counter() - t0
        t_spent += dt
        per_tok.append((n_next, dt))
        if n_next == inp.T:
            # a batch too small for target_s is evaluated again until it is reached
            reps, t_full = reps + 1, t_full + dt
        n = n_next
    if reps:
        value = reps * inp.T / t_full
        sample = (f"all {inp.T} tokens of the same workload, evaluated {reps} time(s) "
                  f"(oracle route + fp64 FFN incl. bf16/e4m3 decode), {t_full:.2f} s")
    else:
        n_last, dt_last = per_tok[-1]
        value = n_last / dt_last
        sample = (f"first {n_last} of {inp.T} tokens of the same workload "
                  f"(oracle route + fp64 FFN incl. bf16/e4m3 decode), {dt_last:.2f} s")
    return {"value": value, "unit": "tokens/s", "cores": blas_threads, "kind": "oracle",
            "sample": sample, "host_cpus": len(os.sched_getaffinity(0))}, sample_out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: one GPU only (the library has no multi-GPU path); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_expert_ffn_router_amd as moe
    from synth import CONFIGS, config_inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    cfg = CONFIGS[args.config]
    if (args.weight_only or args.block_fp8) and CONFIGS[args.config]["dtype"] != "fp8":
        sys.exit("bench.py: --weight-only / --block-fp8 need an FP8 workload (config 3)")
    if args.weight_only and args.block_fp8:
        sys.exit("bench.py: --weight-only and --block-fp8 are separate measurements")
    if args.fp8 and CONFIGS[args.config]["dtype"] != "bf16":
        sys.exit("bench.py: --fp8 takes a bf16 workload (configs 2, 4, 5)")
    inp = config_inputs(args.config, device="cuda",
                        dtype="fp8_block" if args.block_fp8 else ("fp8" if args.fp8 else None))
    T, E, H, I, k = inp.T, inp.E, inp.H, inp.I, inp.k
    Eg = E                                   # experts of the whole layer (routing)
    w1, w2, s1, s2 = inp.w1, inp.w2, inp.w1_scale, inp.w2_scale
    if args.ep > 1 and args.tp > 1:
        sys.exit("bench.py: --ep and --tp are separate measurements")
    if args.ep > 1:                          # rank 0 holds experts [0, E/G): local id = global id
        E = Eg // args.ep
        w1, w2 = w1[:E], w2[:E]
        s1, s2 = (None, None) if s1 is None else (s1[:E], s2[:E])
    if args.tp > 1:                          # rank 0 holds columns [0, I/G) of every expert
        c = I // args.tp
        w1 = torch.cat([w1[:, :c], w1[:, I:I + c]], 1).contiguous()
        w2 = w2[:, :, :c].contiguous()
        I = c
    M = args.block_m or moe.default_block_m(T, E, k)
    S = T * k
    dev = inp.x.device
    wo = args.weight_only
    blk = args.block_fp8
    dt_code = {"f32": moe.MOE_DTYPE_F32, "bf16": moe.MOE_DTYPE_BF16, "fp8": moe.MOE_DTYPE_FP8,
               "fp8_block": moe.MOE_DTYPE_FP8_BLOCK}[inp.dtype]
    if wo:
        dt_code = moe.MOE_DTYPE_W8A16

    # everything the step writes, allocated once
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    cap = moe.align_capacity(T, k, E, M)
    sid = torch.empty(cap, dtype=torch.int32, device=dev)
    be = torch.empty(cap // M, dtype=torch.int32, device=dev)
    npad = torch.empty(1, dtype=torch.int32, device=dev)
    ws = moe.alloc_workspace(T, E, H, I, k, M, dt_code, dev)
    out = torch.empty((T, H), dtype=torch.float32 if inp.dtype == "f32" else torch.bfloat16,
                      device=dev)

    stream = torch.cuda.current_stream()

    # the library calls of a step, checked and marshalled once (moe's prepare=True):
    # each launch in the timed loop is then one C call, so the host stays ahead of
    # the GPU even in short runs and no launch gap lands between an event and its
    # kernel
    def prepared_ffn(flags):
        f = flags | args.flags
        if blk:
            return moe.ffn_fp8_block(inp.x, w1, s1, w2, s2, ids, wts, sid, be, npad, M, f, ws,
                                     out, stream, prepare=True)
        if wo:
            return moe.ffn_w8a16(inp.x, w1, s1, w2, s2, ids, wts, sid, be, npad, M, f, ws, out,
                                 stream, prepare=True)
        if inp.dtype == "fp8":
            return moe.ffn_fp8(inp.x, w1, s1, w2, s2, ids, wts, sid, be, npad, M, f, ws, out,
                               stream, prepare=True)
        if inp.dtype == "bf16":
            return moe.ffn_bf16(inp.x, w1, w2, ids, wts, sid, be, npad, M, f, ws, out, stream,
                                prepare=True)
        return moe.ffn_f32(inp.x, w1, w2, ids, wts, sid, be, npad, M, f, ws, out, stream,
                           prepare=True)

    # a step runs the FFN as three calls: PREP (the counter clearing and x
    # quantisers FC1 needs first), FC1 alone between events, then FC2 and the
    # combine; the FFN-only loop runs it as one call
    ffn_calls = {f: prepared_ffn(f) for f in
                 (moe.STAGE_PREP, moe.STAGE_FC1 | moe.PREPARED,
                  moe.STAGE_FC2 | moe.STAGE_COMBINE, 0)}

    def ffn(flags):
        ffn_calls[flags]()
    # FC1 is bracketed by events on every EVENT_STRIDE-th timed step: a pair of
    # event records costs ~6 us of stream time on MI355X, which on every step
    # would slow the timed steps themselves by ~3 % at decode
    stride = args.event_stride if args.event_stride > 0 else max(1, args.steps // 10)
    n_ev = (args.steps + stride - 1) // stride
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]

    small = args.single_launch or args.small_path
    small_flags = args.flags | (moe.FORWARD_ONE_KERNEL if args.single_launch else 0)
    if small:
        if wo or blk or args.ep > 1 or args.tp > 1 or T > moe.small_max_tokens():
            sys.exit("bench.py: --single-launch/--small-path take an unsharded bf16/fp8 workload of at "
                     f"most {moe.small_max_tokens()} tokens")
        if args.single_launch and (T > 16 or T * k > 256):
            sys.exit("bench.py: --single-launch takes at most 16 tokens and 256 slots")
        ws_small = torch.empty(moe.forward_small_workspace_bytes(T, E, H, I, k, dt_code),
                               dtype=torch.uint8, device=dev)
        small_call = moe.forward_small(inp.logits, inp.x, w1, w2, k, False, s1, s2, small_flags,
                                       out, ids, wts, ws_small, stream, prepare=True)

    def step_small(i=None):
        if i is not None:
            ev_a[i].record(stream)
        small_call()
        if i is not None:
            ev_b[i].record(stream)

    route_call = moe.route_align(inp.logits, k, M, out=(ids, wts, sid, be, npad), stream=stream,
                                 prepare=True) if E == Eg else None

    def step(i=None):
        if small:
            return step_small(i)
        if E == Eg:
            route_call()
        else:  # the rank routes over all experts and aligns its local ones
            moe.route_topk(inp.logits, k, out=(ids, wts), stream=stream)
            moe.align_block(ids, E, M, out=(sid, be, npad), stream=stream)
        ffn(moe.STAGE_PREP)
        if i is not None:
            ev_a[i].record(stream)
        ffn(moe.STAGE_FC1 | moe.PREPARED)
        if i is not None:
            ev_b[i].record(stream)
        ffn(moe.STAGE_FC2 | moe.STAGE_COMBINE)

    tw = time.perf_counter()
    warm = 0
    for _ in range(args.warmup):
        step()
        warm += 1
    torch.cuda.synchronize()
    while time.perf_counter() - tw < MIN_WARMUP_S and warm < 5000:
        for _ in range(8):
            step()
        warm += 8
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i // stride if i % stride == 0 else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    fc1_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(ev_a, ev_b)]))
    # per-step durations from the same events: FC1 start of sampled step i to that
    # of the next sampled step, over the steps between them
    step_ev = np.array([ev_a[i].elapsed_time(ev_a[i + 1]) / stride for i in range(n_ev - 1)]
                       or [0.0])

    # after the timed region: the FFN launches alone (FC1 + FC2 + combine, routing and
    # alignment already in place), each bracketed by its own events
    ffn_ev = None
    if not small:
        n_f = min(50, args.steps)
        fa = [torch.cuda.Event(enable_timing=True) for _ in range(n_f)]
        fb = [torch.cuda.Event(enable_timing=True) for _ in range(n_f)]
        for i in range(n_f):
            fa[i].record(stream)
            ffn(0)
            fb[i].record(stream)
        torch.cuda.synchronize()
        ffn_ev = np.array([a.elapsed_time(b) for a, b in zip(fa, fb)])

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # algorithmic work (active experts from this run's routing)
    ids_h = ids.cpu().numpy()
    A = int(np.unique(ids_h[ids_h < E]).size)       # active local experts
    bw = {"f32": 4, "bf16": 2, "fp8": 1, "fp8_block": 1}[inp.dtype]
    bx = {"f32": 4, "bf16": 2, "fp8": 2, "fp8_block": 2}[inp.dtype]
    S_loc = int((ids_h < E).sum())                   # slots this GPU computes
    # weight scales per expert: per row (fp8) or per 128x128 block (fp8_block)
    sc1 = {"fp8": 2 * I, "fp8_block": (2 * I // 128) * (H // 128)}.get(inp.dtype, 0) * 4
    sc2 = {"fp8": H, "fp8_block": (H // 128) * (I // 128)}.get(inp.dtype, 0) * 4
    w_bytes = A * 3 * I * H * bw + A * (sc1 + sc2)
    layer_bytes = w_bytes + T * H * bx + T * H * (4 if inp.dtype == "f32" else 2) + T * Eg * 4 + S * 8
    flops = S_loc * 6 * H * I
    fc1_bytes = A * 2 * I * H * bw + A * sc1 \
        + T * H * bx + S_loc * I * (2 if inp.dtype == "bf16" or wo else 4)
    fc1_gbs = fc1_bytes / (fc1_ms * 1e-3) / 1e9
    step_s = ms_per_step * 1e-3
    wl = (cfg["name"].replace("_bf16_", "_fp8_") if args.fp8 else cfg["name"]) \
        + ("_w8a16" if wo else "") + ("_block128" if blk else "") \
        + ("_single_launch" if args.single_launch else "") \
        + ("_small_path" if args.small_path else "") + (f"_ep{args.ep}_rank0" if args.ep > 1 else "") \
        + (f"_tp{args.tp}_rank0" if args.tp > 1 else "") \
        + ("_range_gemm" if args.flags & moe.RANGE_GEMM else "") \
        + ("_no_xcd_remap" if args.flags & moe.NO_XCD_REMAP else "")
    if args.single_launch:  # one kernel for the whole layer: its bytes over its duration
        gbs = layer_bytes / (fc1_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic("small_forward", wl),
                    "kernel": "small_forward (whole layer, one launch)",
                    "kernel_ms": round(fc1_ms, 4), "alg_bytes_per_launch": layer_bytes}
    elif args.small_path:  # events bracket the whole call: its bytes over the call's time
        gbs = layer_bytes / (fc1_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "traffic": None,
                    "kernel": "moe_forward_small (whole layer: route, FC1, FC2, combine)",
                    "kernel_ms": round(fc1_ms, 4), "alg_bytes_per_launch": layer_bytes}
    elif M >= 128:  # grouped-GEMM tiles (prefill-sized blocks)
        # the roofline bound is whichever of the two times is longer: the FLOPs at the
        # matrix-core peak or the algorithmic bytes at the HBM peak (at ~256 tokens per
        # expert the weights make it the bytes: 256 FLOP per weight byte in bf16
        # against the chip's 2516.6 TFLOP/s / 8 TB/s = 315); both fractions are given
        fc1_flops = S_loc * 2 * I * H * 2
        fc1_tfs = fc1_flops / (fc1_ms * 1e-3) / 1e12
        peak = MFMA_FP8_PEAK_TFLOPS if inp.dtype == "fp8" else MFMA_BF16_PEAK_TFLOPS
        mfma = {"achieved": round(fc1_tfs, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(fc1_tfs / peak, 4)}
        hbm = {"achieved": round(fc1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(fc1_gbs / HBM_PEAK_GBS, 4)}
        t_mfma_ms = fc1_flops / (peak * 1e12) * 1e3
        t_hbm_ms = fc1_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
        if t_hbm_ms >= t_mfma_ms:
            roofline = {"bound": "hbm", **hbm, "mfma": mfma}
        else:
            roofline = {"bound": "mfma", **mfma, "hbm": hbm}
        roofline.update({"traffic": measured_traffic("fc1", wl),
                         "kernel": "fc1 (FC1 gate|up + SiLU*up)", "kernel_ms": round(fc1_ms, 4),
                         "alg_flops_per_launch": fc1_flops, "alg_bytes_per_launch": fc1_bytes,
                         "bound_ms": {"mfma": round(t_mfma_ms, 4), "hbm": round(t_hbm_ms, 4)}})
    else:
        roofline = {"bound": "hbm", "achieved": round(fc1_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(fc1_gbs / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic("fc1", wl), "kernel": "fc1 (FC1 gate|up + SiLU*up)",
                    "kernel_ms": round(fc1_ms, 4), "alg_bytes_per_launch": fc1_bytes}
    # the FFN launches alone (FC1 + FC2 + combine, p50 of their own events after the
    # timed region): the layer's algorithmic bytes (weights, x, output, routing
    # results; no intermediates) against HBM; at prefill also its FLOPs against the
    # matrix cores, the longer of the two times naming the bound
    ffn_roofline = None
    if ffn_ev is not None:
        ffn_ms = float(np.percentile(ffn_ev, 50))
        ffn_bytes = w_bytes + T * H * bx + T * H * 2 + S * 8
        gbs = ffn_bytes / (ffn_ms * 1e-3) / 1e9
        hbm = {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(gbs / HBM_PEAK_GBS, 4)}
        if M >= 128:  # as for FC1: the longer of the MFMA and the HBM time bounds it
            peak = MFMA_FP8_PEAK_TFLOPS if inp.dtype == "fp8" else MFMA_BF16_PEAK_TFLOPS
            tfs = flops / (ffn_ms * 1e-3) / 1e12
            mfma = {"achieved": round(tfs, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(tfs / peak, 4)}
            if ffn_bytes / (HBM_PEAK_GBS * 1e9) >= flops / (peak * 1e12):
                ffn_roofline = {"bound": "hbm", **hbm, "mfma": mfma}
            else:
                ffn_roofline = {"bound": "mfma", **mfma, "hbm": hbm}
            ffn_roofline.update({"ffn_ms": round(ffn_ms, 4), "alg_flops": flops,
                                 "alg_bytes": ffn_bytes})
        else:
            ffn_roofline = {"bound": "hbm", **hbm, "ffn_ms": round(ffn_ms, 4),
                            "alg_bytes": ffn_bytes}
    roofline["samples"] = n_ev
    rec = {
        "metric": METRIC, "value": round(T / step_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": warm,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms_p10_p50_p90": [round(float(np.percentile(step_ev, q)), 4) for q in (10, 50, 90)],
        "ffn_only_ms_p10_p50_p90": None if ffn_ev is None else
        [round(float(np.percentile(ffn_ev, q)), 4) for q in (10, 50, 90)],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "w8a16" if wo else inp.dtype,
        "data": "synthetic",
        "config": {"workload": wl, "T": T, "E": E, "H": H, "I": I, "k": k, "block_m": M,
                   "routing": cfg["routing"], "active_experts": A, "seed": 0},
        "expert_weight_gbps": round(w_bytes / step_s / 1e9, 1),
        "expert_weight_hbm_frac": round(w_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "layer_alg_bytes": layer_bytes,
        "tflops": round(flops / step_s / 1e12, 2),
        "mfma_bf16_frac": round(flops / step_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": roofline,
        "ffn_roofline": ffn_roofline,
        "samples": {"step_intervals": int(len(step_ev)), "fc1_events": n_ev,
                    "ffn_only": 0 if ffn_ev is None else int(len(ffn_ev))},
        "source_digest": source_digest(),
    }
    if not args.no_cpu_baseline and args.ep == 1 and args.tp == 1:
        cb, _ = cpu_baseline(inp, args.cpu_seconds, wo)
        rec["cpu_baseline"] = cb
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
