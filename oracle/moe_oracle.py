"""Plain, slow, obviously-correct CPU oracle for the fused MoE expert FFN.

TEST INFRASTRUCTURE ONLY: imported by the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path. It
shares no code with the HIP library (no kernels, headers, helpers, tables or
pre/post-processing); only the seeded draws of ``synth`` feed both.

Sources, cited by page title and section (the pages are the text of three web
pages about vLLM's per-architecture kernel selection, vLLM on Vera Rubin, and a
V100 vLLM fork):

* "vLLM support for NVIDIA Vera Rubin NVL72" (Chinese summary), section
  "Locality domain: put the operator next to its weights": in small-token MoE
  decode the forward pass is dominated by reading the FC1 and FC2 expert weight
  matrices; FC1 and FC2 are the two expert projections.
* "vLLM SM architecture adaptation" (Chinese), section 4.3 (Blackwell MoE) and
  the runtime selection-flow figure of section 9: one fused kernel runs the MoE
  layer over all experts, with block-wise FP8 dequantisation inside the GEMM
  loop; section 3.1 (``cutlass_scaled_mm``): scales are applied around an fp32
  accumulator; section 1: FP8 is E4M3.
* The V100 fork article (Japanese), "wall 2": ``silu_and_mul`` is the fused
  activation between FC1 and FC2; "wall 5": MoE routing kernels and an FP8
  activation quantisation kernel exist.

The pages print no formula, tensor shape or value for this path. Where they are
silent the oracle takes the plainest reading, listed in the design notes:
top-k of softmax(router logits) without renormalisation unless asked; ties go
to the lower expert index; FC1 rows [0, I) are the gate (SiLU applied) and rows
[I, 2I) the up projection; SiLU(g) = g * sigmoid(g); the combine is the sum over
the k slots of weight x expert output; e4m3 is OCP e4m3fn (bias 7, max 448, no
infinities) with round-to-nearest-even and saturation; per-row FP8 activation
scales are absmax/448 decided in float32 (the kernel's precision).

Parity of every function here is pinned by the CPU tests against brute force,
closed forms, invariants and library routines; the pages themselves pin no
value ("parity unpinned by the pages" for all outputs).
"""
from __future__ import annotations

from typing import Callable, Iterable, Optional, Tuple

import numpy as np

__all__ = [
    "bf16_bits_to_f64", "e4m3fn_decode", "e4m3fn_encode", "E4M3FN_VALUES",
    "route", "align", "align_capacity", "swiglu_expert", "ffn", "quant_rows_e4m3",
    "ffn_fp8", "dequant_rows", "ffn_w8a16", "quant_groups_e4m3", "dequant_blocks",
    "ffn_fp8_block", "normwise_rel_err",
]

# ---------------------------------------------------------------- formats ---

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact): the 16 stored bits are the
    high half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _e4m3fn_value(code: int) -> float:
    """Value of one OCP FP8 E4M3 ("fn") code from the format definition:
    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
    is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there are no infinities.
    (FP8 E4M3 is the 8-bit float of "vLLM SM architecture adaptation",
    section 1.)"""
    sign = -1.0 if code & 0x80 else 1.0
    ex = (code >> 3) & 0xF
    man = code & 0x7
    if ex == 0xF and man == 0x7:
        return float("nan")
    if ex == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (ex - 7)


E4M3FN_VALUES = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)
_E4M3_POS = E4M3FN_VALUES[:127]          # codes 0x00..0x7E: 0 .. 448, ascending


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """e4m3fn codes (uint8) -> float64, exact."""
    return E4M3FN_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3fn_encode(v: np.ndarray) -> np.ndarray:
    """float32 values -> nearest e4m3fn code, ties to the even code (even
    mantissa), magnitudes above 448 saturate to 448, sign kept (a negative value
    that rounds to zero gives 0x80). NaN is outside the contract."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    a = np.minimum(np.abs(v), 448.0)
    hi = np.searchsorted(_E4M3_POS, a, side="left")     # first grid point >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _E4M3_POS[hi], hi, code)        # exact grid points
    code = code.astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


# ---------------------------------------------------------------- routing ---

def route(logits: np.ndarray, k: int, renormalize: bool = False
          ) -> Tuple[np.ndarray, np.ndarray]:
    """Router softmax and top-k.

    The Vera Rubin page ("hardware growth vs bottlenecks") ties FP32 exp
    throughput to softmax; the V100 article ("wall 5") names the MoE routing
    kernels. Reading: for each token, experts are ordered by the float32 logit
    descending, ties by the lower expert index (-0.0 equals +0.0); the first k
    are the token's slots 0..k-1. p = exp(L - max L) / sum exp(L - max L) in
    float64; slot weight w[t, j] = p[t, ids[t, j]], divided by sum_j w[t, j]
    when ``renormalize``. Selection uses the logits, never rounded
    probabilities (softmax is strictly increasing).
    """
    L = np.asarray(logits, dtype=np.float32)
    T, E = L.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        row = L[t].astype(np.float64)
        order = np.argsort(-row, kind="stable")       # stable: equal logits keep index order
        ids[t] = order[:k]
        z = np.exp(row - row.max())
        p = z / z.sum()
        w[t] = p[ids[t]]
        if renormalize:
            w[t] = w[t] / w[t].sum()
    return ids, w


# -------------------------------------------------------------- alignment ---

def align_capacity(S: int, E: int, block_m: int) -> int:
    """Upper bound on the padded length: every active expert (at most min(E, S)
    of them) adds fewer than block_m padding entries; rounded up to block_m."""
    cap = S + min(E, S) * (block_m - 1)
    return -(-cap // block_m) * block_m


def align(ids: np.ndarray, E: int, block_m: int
          ) -> Tuple[np.ndarray, np.ndarray, int]:
    """Token-to-expert alignment for one fused kernel over all experts.

    The selection-flow figure of "vLLM SM architecture adaptation" (section 9)
    and its section 4.3 run the whole MoE layer as one kernel over all experts;
    the pages do not describe the index structure that needs. Reading: flat slot
    s = t*k + j; for e = 0..E-1 in order, append the slots routed to e in
    ascending s, then pad the run to a multiple of block_m with the sentinel S.
    block_expert[b] is the expert owning block b; num_padded the total length.
    Experts with no slot contribute nothing. A slot whose id lies outside
    [0, E) belongs to an expert served elsewhere (expert parallelism: this
    shard holds experts 0..E-1 of its local numbering) and is left out.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    S = flat.size
    out, blocks = [], []
    for e in range(E):
        slots = np.nonzero(flat == e)[0]                 # ascending s
        c = slots.size
        if c == 0:
            continue
        pad = (-c) % block_m
        out.extend(int(s) for s in slots)
        out.extend([S] * pad)
        blocks.extend([e] * ((c + pad) // block_m))
    return (np.array(out, dtype=np.int32), np.array(blocks, dtype=np.int32), len(out))


# ---------------------------------------------------------------- the FFN ---

def swiglu_expert(w1e: np.ndarray, w2e: np.ndarray, xs: np.ndarray) -> np.ndarray:
    """One expert on a batch of rows ``xs [n, H]`` (float64):
    FC1 gate|up, SiLU-and-mul, FC2.

    FC1/FC2 are the expert projections of the Vera Rubin page ("Locality
    domain"); ``silu_and_mul`` (V100 article, "wall 2") multiplies SiLU of the
    first half of FC1's output by its second half. w1e [2I, H]: rows [0, I) gate,
    [I, 2I) up; w2e [H, I]. SiLU(g) = g / (1 + exp(-g)).
    """
    I = w2e.shape[1]
    g = xs @ w1e[:I].T
    u = xs @ w1e[I:].T
    h = g / (1.0 + np.exp(-g)) * u
    return h @ w2e.T


def ffn(x: np.ndarray, get_w1: Callable[[int], np.ndarray],
        get_w2: Callable[[int], np.ndarray], ids: np.ndarray, weights: np.ndarray,
        tokens: Optional[Iterable[int]] = None, num_experts: Optional[int] = None
        ) -> np.ndarray:
    """out[t] = sum_j weights[t, j] * expert_{ids[t, j]}(x[t]) for each token t in
    ``tokens`` (all by default), float64. ``get_w1(e)``/``get_w2(e)`` return the
    expert's float64 weights. Rows of the result follow ``tokens``. With
    ``num_experts``, slots whose id lies outside [0, num_experts) belong to
    experts served elsewhere and add nothing: the result is this shard's
    partial sum (expert parallelism, the per-rank share of the Vera Rubin
    page's "Locality domain" comparison)."""
    x = np.asarray(x, dtype=np.float64)
    tok = np.arange(x.shape[0]) if tokens is None else np.asarray(list(tokens))
    k = ids.shape[1]
    Y = np.zeros((tok.size, k, x.shape[1]), dtype=np.float64)
    sub = ids[tok]
    for e in np.unique(sub):
        if num_experts is not None and not 0 <= e < num_experts:
            continue
        rows, js = np.nonzero(sub == e)
        Y[rows, js] = swiglu_expert(get_w1(int(e)), get_w2(int(e)), x[tok[rows]])
    w = np.asarray(weights, dtype=np.float64)[tok]
    out = np.zeros((tok.size, x.shape[1]), dtype=np.float64)
    for j in range(k):                                   # combine, slot order
        out += w[:, j:j + 1] * Y[:, j]
    return out


# -------------------------------------------------------------------- FP8 ---

def quant_rows_e4m3(v: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row dynamic FP8 quantisation (the activation quantiser named in
    "wall 5" of the V100 article; scales kept outside the accumulator as in
    ``cutlass_scaled_mm``, section 3.1 of the SM-adaptation page).

    Decisions in float32, the kernel's precision: scale = absmax(row)/448
    (float32 division; 1 for an all-zero row), code = e4m3fn(row / scale) with a
    float32 division. Returns (codes uint8, scale float32)."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.max(np.abs(v), axis=1)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    ratio = (v / scale[:, None]).astype(np.float32)
    return e4m3fn_encode(ratio), scale


def ffn_fp8(x_bits: np.ndarray, get_w1q: Callable[[int], np.ndarray], w1_scale: np.ndarray,
            get_w2q: Callable[[int], np.ndarray], w2_scale: np.ndarray, ids: np.ndarray,
            weights: np.ndarray, tokens: Optional[Iterable[int]] = None,
            num_experts: Optional[int] = None) -> np.ndarray:
    """W8A8 FP8 variant, format-exact: the same codes and scales the GPU gets.

    W^[e, n, :] = dec(Wq[e, n, :]) * scale[e, n] (per output channel);
    x^_t = a_t * dec(q(x_t)) per token; h is computed in float64 from x^ and
    W1^, rounded to float32, then quantised per (token, expert) slot row the
    same way before FC2; combine as in ``ffn`` (``num_experts`` as there).
    ``x_bits`` are bfloat16 bits.
    """
    x32 = bf16_bits_to_f64(x_bits).astype(np.float32)
    tok = np.arange(x32.shape[0]) if tokens is None else np.asarray(list(tokens))
    xq, xs = quant_rows_e4m3(x32[tok])
    xhat = e4m3fn_decode(xq) * xs.astype(np.float64)[:, None]
    k = ids.shape[1]
    H = x32.shape[1]
    Y = np.zeros((tok.size, k, H), dtype=np.float64)
    sub = ids[tok]
    for e in np.unique(sub):
        e = int(e)
        if num_experts is not None and not 0 <= e < num_experts:
            continue
        w1 = e4m3fn_decode(get_w1q(e)) * np.asarray(w1_scale[e], np.float64)[:, None]
        w2 = e4m3fn_decode(get_w2q(e)) * np.asarray(w2_scale[e], np.float64)[:, None]
        I = w2.shape[1]
        rows, js = np.nonzero(sub == e)
        xr = xhat[rows]
        g = xr @ w1[:I].T
        u = xr @ w1[I:].T
        h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
        hq, hs = quant_rows_e4m3(h)
        hhat = e4m3fn_decode(hq) * hs.astype(np.float64)[:, None]
        Y[rows, js] = hhat @ w2.T
    w = np.asarray(weights, dtype=np.float64)[tok]
    out = np.zeros((tok.size, H), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * Y[:, j]
    return out


# ------------------------------------------------------- weight-only FP8 ---

def dequant_rows(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """W^[n, c] = dec(codes[n, c]) * scale[n], float64: one FP8 weight format
    with a per-output-channel scale, widened for 16-bit matrix units
    ("vLLM SM architecture adaptation", section 5.2)."""
    return e4m3fn_decode(codes) * np.asarray(scale, dtype=np.float64)[:, None]


def ffn_w8a16(x_bits: np.ndarray, get_w1q: Callable[[int], np.ndarray], w1_scale: np.ndarray,
              get_w2q: Callable[[int], np.ndarray], w2_scale: np.ndarray, ids: np.ndarray,
              weights: np.ndarray, tokens: Optional[Iterable[int]] = None,
              num_experts: Optional[int] = None) -> np.ndarray:
    """Weight-only FP8 (W8A16) variant: the weight-only fallback MoE backend of
    "vLLM SM architecture adaptation" (sections 4.2 and 5.2). The FFN of ``ffn``
    on the bfloat16 activations (``x_bits``) with each expert's weights
    dequantised by ``dequant_rows``; no activation is quantised."""
    x = bf16_bits_to_f64(x_bits)
    return ffn(x, lambda e: dequant_rows(get_w1q(e), w1_scale[e]),
               lambda e: dequant_rows(get_w2q(e), w2_scale[e]), ids, weights, tokens,
               num_experts)


# ------------------------------------------------------ block-wise FP8 ---
# Block-wise FP8 MoE ("vLLM SM architecture adaptation": section 4.1's
# block_fp8 backends, section 4.2's block-wise FP8 grouped GEMM, the section-9
# figure's block-wise FP8 dequantisation inside the GEMM loop). The pages fix
# no block size; the oracle takes 128 (the 128-wide tiles of that figure):
# weight scales per 128 x 128 block, activation scales per 128 consecutive
# elements of a row.

BLOCK = 128


def quant_groups_e4m3(v: np.ndarray, group: int = BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """``quant_rows_e4m3`` applied to every run of ``group`` consecutive
    elements of each row (the row length is a multiple of ``group``).
    Returns (codes uint8 [R, C], scales float32 [R, C/group])."""
    v = np.asarray(v, dtype=np.float32)
    R, C = v.shape
    q, s = quant_rows_e4m3(v.reshape(R * (C // group), group))
    return q.reshape(R, C), s.reshape(R, C // group)


def dequant_blocks(codes: np.ndarray, scale: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """W^[n, c] = dec(codes[n, c]) * scale[n // block, c // block], float64."""
    s = np.asarray(scale, dtype=np.float64)
    return e4m3fn_decode(codes) * np.repeat(np.repeat(s, block, axis=0), block, axis=1)


def ffn_fp8_block(x_bits: np.ndarray, get_w1q: Callable[[int], np.ndarray],
                  w1_scale: np.ndarray, get_w2q: Callable[[int], np.ndarray],
                  w2_scale: np.ndarray, ids: np.ndarray, weights: np.ndarray,
                  tokens: Optional[Iterable[int]] = None,
                  num_experts: Optional[int] = None) -> np.ndarray:
    """Block-scaled FP8 variant, format-exact. ``w1_scale`` [E, 2I/128, H/128],
    ``w2_scale`` [E, H/128, I/128]. x^ = group-dequantised x (groups of 128
    per token); h is computed in float64 from x^ and W1^, rounded to float32,
    and group-quantised per slot row before FC2; combine as in ``ffn``. Since
    sum_c W^[n,c] x^[c] = sum_b w_s[n/128, b] a[b] sum_{c in b} dec(Wq) dec(xq),
    dequantise-then-multiply is the same number as scaling each block's
    partial sum."""
    x32 = bf16_bits_to_f64(x_bits).astype(np.float32)
    tok = np.arange(x32.shape[0]) if tokens is None else np.asarray(list(tokens))
    xq, xs = quant_groups_e4m3(x32[tok])
    xhat = e4m3fn_decode(xq) * np.repeat(xs.astype(np.float64), BLOCK, axis=1)
    k = ids.shape[1]
    H = x32.shape[1]
    Y = np.zeros((tok.size, k, H), dtype=np.float64)
    sub = ids[tok]
    for e in np.unique(sub):
        e = int(e)
        if num_experts is not None and not 0 <= e < num_experts:
            continue
        w1 = dequant_blocks(get_w1q(e), w1_scale[e])
        w2 = dequant_blocks(get_w2q(e), w2_scale[e])
        I = w2.shape[1]
        rows, js = np.nonzero(sub == e)
        xr = xhat[rows]
        g = xr @ w1[:I].T
        u = xr @ w1[I:].T
        h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
        hq, hs = quant_groups_e4m3(h)
        hhat = e4m3fn_decode(hq) * np.repeat(hs.astype(np.float64), BLOCK, axis=1)
        Y[rows, js] = hhat @ w2.T
    w = np.asarray(weights, dtype=np.float64)[tok]
    out = np.zeros((tok.size, H), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * Y[:, j]
    return out


# ------------------------------------------------------------- comparison ---

def normwise_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max_i |got_i - ref_i| / max_i |ref_i| (0 if ref is all zero and got equal)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
