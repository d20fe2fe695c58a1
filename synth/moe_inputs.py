"""Seeded synthetic inputs for the fused MoE expert FFN workloads.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic: no softmax, no top-k, no alignment, no projection, no
activation, no combine and no activation quantisation. Both the CPU oracle and
the HIP path consume what it returns, and neither is imported here.

Recipe (the pages give no tensor shapes and no data; these draws stand in for
the per-rank MoE FC1+FC2 timing of the Vera Rubin page, section "Locality
domain", which used balanced routing on shapes it does not print):

* ``x`` ~ N(0, 1) drawn as float32 by numpy PCG64, rounded to bfloat16 (RNE)
  for the bf16/fp8 workloads, kept float32 for the f32 workload.
* Expert weights: FC1 ``w1 [E, 2I, H]`` (rows [0, I) gate, rows [I, 2I) up)
  and FC2 ``w2 [E, H, I]``, fp32 master values ~ N(0, std) with
  std = 1/sqrt(fan_in) (fan_in = H for FC1, I for FC2) unless a workload fixes
  std. They are drawn by torch's generator on the device that will hold them,
  one generator per (tensor, expert) seeded from the workload seed, so big
  weight sets are made on the GPU in milliseconds. Masters are rounded to
  bfloat16 (RNE), or quantised per output channel to OCP e4m3fn with an fp32
  scale = absmax(row)/448 (scale 1 for an all-zero row) using torch's own
  float8 cast after clamping to +-448. This quantisation is weight preparation
  done once before serving; it is not on the hot path.
* Router logits ``[T, E]`` float32, by routing kind:
  - ``router``: logits = x @ Wr^T evaluated in float64 and rounded to float32,
    Wr ~ N(0, 1) of shape [E, H] (the router GEMM sits before the hot path).
  - ``balanced``: every expert receives exactly T*k/E slots. For round r of
    T*k/E rounds a permutation pi_r of the experts is drawn; token r*(E/k)+q
    takes experts pi_r[q*k:(q+1)*k] with logits ~ U(1, 2), all other logits
    ~ U(-2, 0), so the top-k set is exact by a margin of 1.
  - ``zipf``: popularity p_e proportional to (pi(e)+1)^-s for a seeded
    permutation pi, logits = ln p_e + N(0, sigma) with sigma = 0.5.
  - ``normal``: logits ~ N(0, 1) (near-uniform load).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional

import numpy as np
import torch

# The five workloads. Sizes follow the workload list this repository is
# measured on; "fan_in" scaling and routing kinds are described above.
CONFIGS: Dict[int, dict] = {
    1: dict(name="tiny_f32_T4_E8_H256_I512_k2", T=4, E=8, H=256, I=512, k=2,
            dtype="f32", routing="router", wstd=0.02),
    2: dict(name="decode_bf16_T16_E64_H4096_I1536_k8_balanced", T=16, E=64, H=4096,
            I=1536, k=8, dtype="bf16", routing="balanced"),
    3: dict(name="decode_fp8_T16_E64_H4096_I1536_k8_balanced", T=16, E=64, H=4096,
            I=1536, k=8, dtype="fp8", routing="balanced"),
    4: dict(name="skewed_decode_bf16_T64_E128_H7168_I2048_k8_zipf1.2", T=64, E=128,
            H=7168, I=2048, k=8, dtype="bf16", routing="zipf", zipf_s=1.2, zipf_sigma=0.5),
    5: dict(name="prefill_bf16_T4096_E128_H4096_I1536_k8", T=4096, E=128, H=4096,
            I=1536, k=8, dtype="bf16", routing="normal"),
}


@dataclasses.dataclass
class MoEInputs:
    """One workload instance. Device tensors feed the HIP path; the oracle
    takes host copies (``host_*`` helpers) of exactly the same bits."""
    T: int
    E: int
    H: int
    I: int
    k: int
    dtype: str                      # "f32" | "bf16" | "fp8" | "fp8_block"
    routing: str
    seed: int
    x: torch.Tensor                 # [T, H] float32 (f32) or bfloat16 (bf16, fp8)
    logits: torch.Tensor            # [T, E] float32
    w1: torch.Tensor                # [E, 2I, H] float32 | bfloat16 | uint8 (e4m3fn codes)
    w2: torch.Tensor                # [E, H, I]
    w1_scale: Optional[torch.Tensor] = None  # [E, 2I] (fp8) | [E, 2I/128, H/128] (fp8_block)
    w2_scale: Optional[torch.Tensor] = None  # [E, H] (fp8) | [E, H/128, I/128] (fp8_block)

    @property
    def S(self) -> int:
        return self.T * self.k

    @property
    def device(self) -> torch.device:
        return self.x.device

    # Host views (exact bit copies) used by the oracle.
    def host_x(self) -> np.ndarray:
        """x as float32 (f32) or as raw bfloat16 bits uint16 (bf16/fp8)."""
        return _bits(self.x)

    def host_logits(self) -> np.ndarray:
        return self.logits.detach().cpu().numpy()

    def host_w1(self, e: int) -> np.ndarray:
        return _bits(self.w1[e])

    def host_w2(self, e: int) -> np.ndarray:
        return _bits(self.w2[e])

    def host_w1_scale(self) -> Optional[np.ndarray]:
        return None if self.w1_scale is None else self.w1_scale.detach().cpu().numpy()

    def host_w2_scale(self) -> Optional[np.ndarray]:
        return None if self.w2_scale is None else self.w2_scale.detach().cpu().numpy()


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.numpy()
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(f"unexpected dtype {t.dtype}")


def _sub_seed(seed: int, *tags) -> int:
    h = hashlib.sha256(repr((seed,) + tags).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _router_logits(rng: np.random.Generator, routing: str, T: int, E: int, k: int,
                   x32: np.ndarray, H: int, zipf_s: float, zipf_sigma: float) -> np.ndarray:
    if routing == "router":
        wr = rng.standard_normal((E, H))
        return (x32.astype(np.float64) @ wr.T).astype(np.float32)
    if routing == "balanced":
        S = T * k
        if S % E != 0 or E % k != 0 or T % (E // k) != 0:
            raise ValueError("balanced routing needs E | T*k and k | E")
        rounds, per_round = S // E, E // k
        logits = rng.uniform(-2.0, 0.0, size=(T, E))
        for r in range(rounds):
            perm = rng.permutation(E)
            for q in range(per_round):
                t = r * per_round + q
                chosen = perm[q * k:(q + 1) * k]
                logits[t, chosen] = rng.uniform(1.0, 2.0, size=k)
        return logits.astype(np.float32)
    if routing == "zipf":
        perm = rng.permutation(E)
        pop = (perm + 1.0) ** (-zipf_s)
        pop /= pop.sum()
        noise = rng.normal(0.0, zipf_sigma, size=(T, E))
        return (np.log(pop)[None, :] + noise).astype(np.float32)
    if routing == "normal":
        return rng.standard_normal((T, E)).astype(np.float32)
    raise ValueError(f"unknown routing kind {routing!r}")


def _expert_master(seed: int, which: str, e: int, rows: int, cols: int, std: float,
                   device: torch.device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(_sub_seed(seed, which, e))
    return torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32) * std


def _quant_rows_e4m3(m: torch.Tensor):
    """Per-output-channel weight preparation: fp32 scale = absmax/448 per row,
    codes by torch's float8_e4m3fn cast of the clamped ratio."""
    amax = m.abs().amax(dim=1)
    scale = amax / 448.0
    scale = torch.where(amax == 0, torch.ones_like(scale), scale)
    q = (m / scale[:, None]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale


def _quant_blocks_e4m3(m: torch.Tensor, b: int = 128):
    """Block-wise weight preparation: fp32 scale = absmax/448 per b x b block,
    codes by torch's float8_e4m3fn cast of the clamped ratio."""
    R, C = m.shape
    blk = m.view(R // b, b, C // b, b)
    amax = blk.abs().amax(dim=(1, 3))
    scale = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
    q = (blk / scale[:, None, :, None]).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(R, C).view(torch.uint8), scale


def make_inputs(T: int, E: int, H: int, I: int, k: int, dtype: str = "bf16",
                routing: str = "normal", seed: int = 0, device="cpu",
                wstd: Optional[float] = None, zipf_s: float = 1.2,
                zipf_sigma: float = 0.5, logits: Optional[np.ndarray] = None) -> MoEInputs:
    """Draw one workload. ``logits`` overrides the routing draw (test fixtures)."""
    device = torch.device(device)
    rng = np.random.default_rng(seed)
    x32 = rng.standard_normal((T, H), dtype=np.float32)
    if logits is None:
        lg = _router_logits(rng, routing, T, E, k, x32, H, zipf_s, zipf_sigma)
    else:
        lg = np.ascontiguousarray(logits, dtype=np.float32)
        assert lg.shape == (T, E)
    xt = torch.from_numpy(x32)
    if dtype in ("bf16", "fp8", "fp8_block"):
        xt = xt.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(dtype)
    x_dev = xt.to(device)
    lg_dev = torch.from_numpy(lg).to(device)

    wdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8,
           "fp8_block": torch.uint8}[dtype]
    w1 = torch.empty((E, 2 * I, H), dtype=wdt, device=device)
    w2 = torch.empty((E, H, I), dtype=wdt, device=device)
    s1 = s2 = None
    if dtype == "fp8":
        s1 = torch.empty((E, 2 * I), dtype=torch.float32, device=device)
        s2 = torch.empty((E, H), dtype=torch.float32, device=device)
    elif dtype == "fp8_block":
        s1 = torch.empty((E, 2 * I // 128, H // 128), dtype=torch.float32, device=device)
        s2 = torch.empty((E, H // 128, I // 128), dtype=torch.float32, device=device)
    std1 = wstd if wstd is not None else 1.0 / np.sqrt(H)
    std2 = wstd if wstd is not None else 1.0 / np.sqrt(I)
    for e in range(E):
        m1 = _expert_master(seed, "w1", e, 2 * I, H, std1, device)
        m2 = _expert_master(seed, "w2", e, H, I, std2, device)
        if dtype == "fp8":
            w1[e], s1[e] = _quant_rows_e4m3(m1)
            w2[e], s2[e] = _quant_rows_e4m3(m2)
        elif dtype == "fp8_block":
            w1[e], s1[e] = _quant_blocks_e4m3(m1)
            w2[e], s2[e] = _quant_blocks_e4m3(m2)
        else:
            w1[e] = m1.to(wdt)
            w2[e] = m2.to(wdt)
        del m1, m2
    return MoEInputs(T=T, E=E, H=H, I=I, k=k, dtype=dtype, routing=routing, seed=seed,
                     x=x_dev, logits=lg_dev, w1=w1, w2=w2, w1_scale=s1, w2_scale=s2)


def config_inputs(n: int, device="cpu", seed: int = 0, dtype: Optional[str] = None) -> MoEInputs:
    """Workload n; ``dtype`` overrides its weight format (same master weights)."""
    c = CONFIGS[n]
    return make_inputs(c["T"], c["E"], c["H"], c["I"], c["k"], dtype=dtype or c["dtype"],
                       routing=c["routing"], seed=seed, device=device,
                       wstd=c.get("wstd"), zipf_s=c.get("zipf_s", 1.2),
                       zipf_sigma=c.get("zipf_sigma", 0.5))


def fingerprint(inp: MoEInputs) -> str:
    """SHA-256 over the host-side draws (x and logits) of a workload."""
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(inp.host_x()).tobytes())
    h.update(np.ascontiguousarray(inp.host_logits()).tobytes())
    return h.hexdigest()


def draw_topk_ids(T: int, E: int, k: int, seed: int = 0, kind: str = "uniform",
                  zipf_s: float = 1.2) -> np.ndarray:
    """Random expert ids [T, k] int32, k distinct experts per token, for tests
    of the alignment step in isolation. ``kind``: "uniform" (each token a
    uniformly random k-subset in random order), "zipf" (subset drawn by
    popularity (rank+1)^-s), "one" (every token's slot 0 is expert 0: one
    expert holds T slots)."""
    rng = np.random.default_rng(seed)
    ids = np.empty((T, k), dtype=np.int32)
    if kind == "zipf":
        perm = rng.permutation(E)
        p = (perm + 1.0) ** (-zipf_s)
        p /= p.sum()
    for t in range(T):
        if kind == "zipf":
            ids[t] = rng.choice(E, size=k, replace=False, p=p)
        else:
            ids[t] = rng.permutation(E)[:k]
            if kind == "one" and 0 not in ids[t, :1]:
                pos = np.nonzero(ids[t] == 0)[0]
                if pos.size:
                    ids[t, pos[0]] = ids[t, 0]
                ids[t, 0] = 0
    return ids
