"""Thin Python binding of libmoe.so (fused MoE expert FFN on MI355X / gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of
libmoe.so; torch supplies device memory and the current stream. Importing the
package loads the library and raises if it has not been built; nothing here
computes a result on the CPU.

The names mirror the C ABI in include/moe.h:

    route_topk(logits, k, renormalize=False)           -> (topk_ids, topk_weights)
    align_block(topk_ids, E, block_m)                   -> (sorted_ids, block_expert, num_padded)
    ffn_bf16(x, w1, w2, ids, wts, sorted_ids, block_expert, num_padded, block_m, ...) -> out
    ffn_fp8(x, w1, w1_scale, w2, w2_scale, ids, wts, ..., block_m, ...)              -> out
    ffn_w8a16(x, w1, w1_scale, w2, w2_scale, ids, wts, ..., block_m, ...)            -> out
    ffn_fp8_block(x, w1, w1_scale, w2, w2_scale, ids, wts, ..., block_m, ...)        -> out
    ffn_f32(x, w1, w2, ids, wts, ..., block_m, ...)                                 -> out
    forward(x, logits, w1, w2, k, ...)   convenience chaining of the three calls
    forward_small(logits, x, w1, w2, k, ...) -> (out, topk_ids, topk_weights)   one launch, T <= 16
    forward_small_static(logits, x, w1, w2, k, ...)   the same without a workspace (allocates nothing)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch  # loads torch's HIP runtime first; libmoe.so then binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_DTYPE_F32, MOE_DTYPE_BF16, MOE_DTYPE_FP8, MOE_DTYPE_W8A16, MOE_DTYPE_FP8_BLOCK = 0, 1, 2, 3, 4
STAGE_FC1, STAGE_FC2, STAGE_COMBINE, STAGE_PREP = 1 << 0, 1 << 1, 1 << 2, 1 << 3
PREPARED = 1 << 11  # with STAGE_FC1: an earlier call ran STAGE_PREP (see include/moe.h)
NO_XCD_REMAP = 1 << 8
FORWARD_ONE_KERNEL = 1 << 9  # forward_small: the whole layer as one cooperative launch
RANGE_GEMM = 1 << 10  # bf16 prefill blocks: 256 x 256 tiles over per-expert token ranges
ABI_VERSION = 1

EXPORTS = ("moe_status_str", "moe_abi_version", "moe_route_topk", "moe_align_capacity",
           "moe_align_block", "moe_route_align", "moe_default_block_m",
           "moe_ffn_workspace_bytes", "moe_ffn_bf16", "moe_ffn_fp8", "moe_ffn_w8a16",
           "moe_ffn_fp8_block", "moe_ffn_f32", "moe_small_max_tokens",
           "moe_forward_small_workspace_bytes", "moe_forward_small", "moe_forward_small_static")
STATIC_SCRATCH_BYTES = 32 << 20  # MOE_STATIC_SCRATCH_BYTES


class MoEError(RuntimeError):
    """A libmoe call returned a non-OK status."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(or python moe_expert_ffn_router_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, U, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_status_str.argtypes = [I]
    lib.moe_abi_version.restype = I
    lib.moe_abi_version.argtypes = []
    lib.moe_route_topk.restype = I
    lib.moe_route_topk.argtypes = [P, I, I, I, I, P, P, P]
    lib.moe_align_capacity.restype = Z
    lib.moe_align_capacity.argtypes = [I, I, I, I]
    lib.moe_align_block.restype = I
    lib.moe_align_block.argtypes = [P, I, I, I, I, P, P, P, P]
    lib.moe_route_align.restype = I
    lib.moe_route_align.argtypes = [P, I, I, I, I, I, P, P, P, P, P, P]
    lib.moe_default_block_m.restype = I
    lib.moe_default_block_m.argtypes = [I, I, I]
    lib.moe_ffn_workspace_bytes.restype = Z
    lib.moe_ffn_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
    ffn_tail = [P, P, P, P, P, I, I, I, I, I, I, U, P, Z, P, P]
    lib.moe_ffn_bf16.restype = I
    lib.moe_ffn_bf16.argtypes = [P, P, P] + ffn_tail
    lib.moe_ffn_f32.restype = I
    lib.moe_ffn_f32.argtypes = [P, P, P] + ffn_tail
    lib.moe_ffn_fp8.restype = I
    lib.moe_ffn_fp8.argtypes = [P, P, P, P, P] + ffn_tail
    lib.moe_ffn_w8a16.restype = I
    lib.moe_ffn_w8a16.argtypes = [P, P, P, P, P] + ffn_tail
    lib.moe_ffn_fp8_block.restype = I
    lib.moe_ffn_fp8_block.argtypes = [P, P, P, P, P] + ffn_tail
    lib.moe_small_max_tokens.restype = I
    lib.moe_small_max_tokens.argtypes = []
    lib.moe_forward_small_workspace_bytes.restype = Z
    lib.moe_forward_small_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.moe_forward_small.restype = I
    lib.moe_forward_small.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, U, P, P, P, Z, P, P]
    lib.moe_forward_small_static.restype = I
    lib.moe_forward_small_static.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, U, P, P, P, P]
    if lib.moe_abi_version() != ABI_VERSION:
        raise ImportError(f"libmoe ABI {lib.moe_abi_version()} != binding ABI {ABI_VERSION}")
    return lib


lib = _load()


def status_str(s: int) -> str:
    return lib.moe_status_str(s).decode()


def _check(s: int) -> None:
    if s != MOE_OK:
        raise MoEError(s, status_str(s))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream: Optional[torch.cuda.Stream]) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t: torch.Tensor, name: str, dtypes, device=None, shape=None,
          min_numel: Optional[int] = None) -> None:
    """Check one tensor argument before its pointer reaches the library (the C
    ABI sees only addresses, so a wrong shape, dtype or device would be read or
    written out of bounds on the GPU): a contiguous device tensor of one of
    ``dtypes``, on ``device``, of exactly ``shape`` and/or at least
    ``min_numel`` elements."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (cuda/hip) tensor, got {t.device}")
    if device is not None and t.device != torch.device(device):
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {min_numel}")


def _dims(t: torch.Tensor, name: str, ndim: int) -> tuple:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


_FP8 = (torch.uint8, torch.float8_e4m3fn)


# ------------------------------------------------------------- routing ---

def _routing_outputs(out, T, k, dev):
    if out is None:
        return (torch.empty((T, k), dtype=torch.int32, device=dev),
                torch.empty((T, k), dtype=torch.float32, device=dev))
    ids, wts = out
    _need(ids, "topk_ids", (torch.int32,), dev, (T, k))
    _need(wts, "topk_weights", (torch.float32,), dev, (T, k))
    return ids, wts


def _align_outputs(out, T, k, E, block_m, dev):
    cap = align_capacity(T, k, E, block_m)
    nblk = cap // block_m if block_m > 0 else 0
    if out is None:
        return (torch.empty(cap, dtype=torch.int32, device=dev),
                torch.empty(nblk, dtype=torch.int32, device=dev),
                torch.empty(1, dtype=torch.int32, device=dev))
    sorted_ids, block_expert, num_padded = out
    _need(sorted_ids, "sorted_ids", (torch.int32,), dev, min_numel=cap)
    _need(block_expert, "block_expert", (torch.int32,), dev, min_numel=nblk)
    _need(num_padded, "num_padded", (torch.int32,), dev, min_numel=1)
    return sorted_ids, block_expert, num_padded


def route_topk(logits: torch.Tensor, k: int, renormalize: bool = False, out=None,
               stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Router softmax + top-k (moe_route_topk). logits [T, E] float32; ``out``
    = (topk_ids [T, k] int32, topk_weights [T, k] float32) to write into."""
    T, E = _dims(logits, "logits", 2)
    _need(logits, "logits", (torch.float32,))
    ids, wts = _routing_outputs(out, T, k, logits.device)
    _check(lib.moe_route_topk(_ptr(logits), T, E, k, int(bool(renormalize)), _ptr(ids),
                              _ptr(wts), _stream(stream)))
    return ids, wts


def align_capacity(T: int, k: int, E: int, block_m: int) -> int:
    return int(lib.moe_align_capacity(T, k, E, block_m))


def default_block_m(T: int, E: int, k: int) -> int:
    """moe_default_block_m: the block size of the fast regime for this batch."""
    return int(lib.moe_default_block_m(T, E, k))


def align_block(topk_ids: torch.Tensor, E: int, block_m: int, out=None, stream=None):
    """Token-to-expert alignment (moe_align_block). Returns device tensors
    (sorted_ids [cap], block_expert [cap/block_m], num_padded [1]); ``out`` may
    supply them (at least that many elements each)."""
    T, k = _dims(topk_ids, "topk_ids", 2)
    _need(topk_ids, "topk_ids", (torch.int32,))
    sorted_ids, block_expert, num_padded = _align_outputs(out, T, k, E, block_m,
                                                          topk_ids.device)
    _check(lib.moe_align_block(_ptr(topk_ids), T, k, E, block_m, _ptr(sorted_ids),
                               _ptr(block_expert), _ptr(num_padded), _stream(stream)))
    return sorted_ids, block_expert, num_padded


align = align_block  # the alignment step under its short name


def route_align(logits: torch.Tensor, k: int, block_m: int, renormalize: bool = False,
                out=None, stream=None, prepare: bool = False):
    """Routing and alignment in one call (moe_route_align). logits [T, E] float32.
    Returns (topk_ids, topk_weights, sorted_ids, block_expert, num_padded), or
    fills `out`, a tuple of those five tensors."""
    T, E = _dims(logits, "logits", 2)
    _need(logits, "logits", (torch.float32,))
    dev = logits.device
    if out is None:
        ids, wts = _routing_outputs(None, T, k, dev)
        sorted_ids, block_expert, num_padded = _align_outputs(None, T, k, E, block_m, dev)
    else:
        ids, wts = _routing_outputs(out[:2], T, k, dev)
        sorted_ids, block_expert, num_padded = _align_outputs(out[2:], T, k, E, block_m, dev)
    keep = (logits, ids, wts, sorted_ids, block_expert, num_padded)
    args = (_ptr(logits), T, E, k, int(bool(renormalize)), block_m, _ptr(ids), _ptr(wts),
            _ptr(sorted_ids), _ptr(block_expert), _ptr(num_padded), _stream(stream))
    return _run(lib.moe_route_align, args, keep, prepare,
                (ids, wts, sorted_ids, block_expert, num_padded))


# ------------------------------------------------------- prepared calls ---

class Prepared:
    """A library call whose arguments were checked and marshalled once (pass
    ``prepare=True`` to route_align, the ffn_* calls or forward_small): calling
    it makes only the C call, which validates its arguments again on the host,
    and checks the status. For loops that launch the same call many times; it
    keeps its tensors alive, and they must not be resized or reallocated."""
    __slots__ = ("_fn", "_args", "_keep")

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self):
        _check(self._fn(*self._args))


def _run(fn, args, keep, prepare, result):
    if prepare:
        return Prepared(fn, args, keep)
    _check(fn(*args))
    return result


# ----------------------------------------------------------------- FFN ---

def workspace_bytes(T: int, E: int, H: int, I: int, k: int, block_m: int, dtype: int) -> int:
    return int(lib.moe_ffn_workspace_bytes(T, E, H, I, k, block_m, dtype))


def alloc_workspace(T, E, H, I, k, block_m, dtype, device) -> torch.Tensor:
    n = workspace_bytes(T, E, H, I, k, block_m, dtype)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _ffn_args(x, w1, w2, wdtypes, xdtypes, topk_ids, topk_weights, sorted_ids, block_expert,
              num_padded, block_m):
    """Shapes of an FFN call, checked against each other: x [T, H], w1 [E, 2I, H],
    w2 [E, H, I], routing [T, k], alignment buffers that hold the capacity of
    ``block_m``. Returns (T, E, H, I, k)."""
    T, H = _dims(x, "x", 2)
    _need(x, "x", xdtypes)
    dev = x.device
    E, I2, H1 = _dims(w1, "w1", 3)
    if H1 != H or I2 % 2:
        raise ValueError(f"w1 has shape {tuple(w1.shape)}, expected [E, 2I, H={H}]")
    I = I2 // 2
    _need(w1, "w1", wdtypes, dev)
    _need(w2, "w2", wdtypes, dev, (E, H, I))
    Tk = _dims(topk_ids, "topk_ids", 2)
    if Tk[0] != T:
        raise ValueError(f"topk_ids has {Tk[0]} rows, x has {T}")
    k = Tk[1]
    _need(topk_ids, "topk_ids", (torch.int32,), dev, (T, k))
    _need(topk_weights, "topk_weights", (torch.float32,), dev, (T, k))
    _align_outputs((sorted_ids, block_expert, num_padded), T, k, E, block_m, dev)
    return T, E, H, I, k


def _ffn_buffers(x, T, E, H, I, k, block_m, dtype, out_dtype, workspace, out):
    dev = x.device
    if workspace is None:
        workspace = alloc_workspace(T, E, H, I, k, block_m, dtype, dev)
    else:
        _need(workspace, "workspace", (torch.uint8,), dev,
              min_numel=workspace_bytes(T, E, H, I, k, block_m, dtype))
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=dev)
    else:
        _need(out, "out", (out_dtype,), dev, (T, H))
    return workspace, out


def ffn_bf16(x, w1, w2, topk_ids, topk_weights, sorted_ids, block_expert, num_padded,
             block_m: int, flags: int = 0, workspace=None, out=None, stream=None,
             prepare: bool = False):
    """moe_ffn_bf16: x [T,H], w1 [E,2I,H], w2 [E,H,I] bfloat16 -> out [T,H] bfloat16."""
    T, E, H, I, k = _ffn_args(x, w1, w2, (torch.bfloat16,), (torch.bfloat16,), topk_ids,
                              topk_weights, sorted_ids, block_expert, num_padded, block_m)
    workspace, out = _ffn_buffers(x, T, E, H, I, k, block_m, MOE_DTYPE_BF16, torch.bfloat16,
                                  workspace, out)
    keep = (x, w1, w2, topk_ids, topk_weights, sorted_ids, block_expert, num_padded, workspace,
            out)
    args = (_ptr(x), _ptr(w1), _ptr(w2), _ptr(topk_ids), _ptr(topk_weights), _ptr(sorted_ids),
            _ptr(block_expert), _ptr(num_padded), T, E, H, I, k, block_m, flags,
            _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream))
    return _run(lib.moe_ffn_bf16, args, keep, prepare, out)


def _scale_shapes(dtype, E, H, I):
    if dtype == MOE_DTYPE_FP8_BLOCK:
        return (E, 2 * I // 128, H // 128), (E, H // 128, I // 128)
    return (E, 2 * I), (E, H)


def _ffn_scaled(fn, dtype, x, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, sorted_ids,
                block_m, flags, workspace, out, stream, block_expert, num_padded,
                prepare=False):
    T, E, H, I, k = _ffn_args(x, w1, w2, _FP8, (torch.bfloat16,), topk_ids, topk_weights,
                              sorted_ids, block_expert, num_padded, block_m)
    s1, s2 = _scale_shapes(dtype, E, H, I)
    _need(w1_scale, "w1_scale", (torch.float32,), x.device, s1)
    _need(w2_scale, "w2_scale", (torch.float32,), x.device, s2)
    workspace, out = _ffn_buffers(x, T, E, H, I, k, block_m, dtype, torch.bfloat16,
                                  workspace, out)
    keep = (x, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, sorted_ids, block_expert,
            num_padded, workspace, out)
    args = (_ptr(x), _ptr(w1), _ptr(w1_scale), _ptr(w2), _ptr(w2_scale), _ptr(topk_ids),
            _ptr(topk_weights), _ptr(sorted_ids), _ptr(block_expert), _ptr(num_padded), T, E,
            H, I, k, block_m, flags, _ptr(workspace), workspace.numel(), _ptr(out),
            _stream(stream))
    return _run(fn, args, keep, prepare, out)


def ffn_fp8(x, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, sorted_ids, block_expert,
            num_padded, block_m: int, flags: int = 0, workspace=None, out=None, stream=None,
            prepare: bool = False):
    """moe_ffn_fp8: x [T,H] bfloat16; w1 [E,2I,H], w2 [E,H,I] e4m3fn codes (uint8 or
    float8_e4m3fn) with float32 per-output-row scales -> out [T,H] bfloat16."""
    return _ffn_scaled(lib.moe_ffn_fp8, MOE_DTYPE_FP8, x, w1, w1_scale, w2, w2_scale, topk_ids,
                       topk_weights, sorted_ids, block_m, flags, workspace, out, stream,
                       block_expert, num_padded, prepare)


def ffn_w8a16(x, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, sorted_ids, block_expert,
              num_padded, block_m: int, flags: int = 0, workspace=None, out=None, stream=None,
              prepare: bool = False):
    """moe_ffn_w8a16: weight-only fp8. Arguments as ffn_fp8; activations stay
    bfloat16 -> out [T,H] bfloat16."""
    return _ffn_scaled(lib.moe_ffn_w8a16, MOE_DTYPE_W8A16, x, w1, w1_scale, w2, w2_scale,
                       topk_ids, topk_weights, sorted_ids, block_m, flags, workspace, out,
                       stream, block_expert, num_padded, prepare)


def ffn_fp8_block(x, w1, w1_scale, w2, w2_scale, topk_ids, topk_weights, sorted_ids,
                  block_expert, num_padded, block_m: int, flags: int = 0, workspace=None,
                  out=None, stream=None, prepare: bool = False):
    """moe_ffn_fp8_block: x [T,H] bfloat16; w1 [E,2I,H], w2 [E,H,I] e4m3fn codes with
    float32 scales per 128x128 block (w1_scale [E,2I/128,H/128], w2_scale [E,H/128,I/128])
    -> out [T,H] bfloat16."""
    return _ffn_scaled(lib.moe_ffn_fp8_block, MOE_DTYPE_FP8_BLOCK, x, w1, w1_scale, w2,
                       w2_scale, topk_ids, topk_weights, sorted_ids, block_m, flags, workspace,
                       out, stream, block_expert, num_padded, prepare)


def ffn_f32(x, w1, w2, topk_ids, topk_weights, sorted_ids, block_expert, num_padded,
            block_m: int, flags: int = 0, workspace=None, out=None, stream=None,
            prepare: bool = False):
    """moe_ffn_f32: float32 throughout."""
    T, E, H, I, k = _ffn_args(x, w1, w2, (torch.float32,), (torch.float32,), topk_ids,
                              topk_weights, sorted_ids, block_expert, num_padded, block_m)
    workspace, out = _ffn_buffers(x, T, E, H, I, k, block_m, MOE_DTYPE_F32, torch.float32,
                                  workspace, out)
    keep = (x, w1, w2, topk_ids, topk_weights, sorted_ids, block_expert, num_padded, workspace,
            out)
    args = (_ptr(x), _ptr(w1), _ptr(w2), _ptr(topk_ids), _ptr(topk_weights), _ptr(sorted_ids),
            _ptr(block_expert), _ptr(num_padded), T, E, H, I, k, block_m, flags,
            _ptr(workspace), workspace.numel(), _ptr(out), _stream(stream))
    return _run(lib.moe_ffn_f32, args, keep, prepare, out)


def forward(x, logits, w1, w2, k: int, block_m: Optional[int] = None, renormalize: bool = False,
            w1_scale=None, w2_scale=None, flags: int = 0, weight_only: bool = False,
            stream=None):
    """route_align -> ffn_{f32,bf16,fp8,w8a16,fp8_block}, dtype taken from w1 (fp8
    codes with 3-d block scales run ffn_fp8_block; with per-row scales ffn_w8a16
    if ``weight_only``, else ffn_fp8); block_m defaults to moe_default_block_m."""
    E = _dims(w1, "w1", 3)[0]
    if block_m is None:
        block_m = default_block_m(x.shape[0], E, k)
    ids, wts, sorted_ids, block_expert, num_padded = route_align(logits, k, block_m, renormalize,
                                                                 stream=stream)
    if w1.dtype in _FP8:
        if w1_scale is not None and w1_scale.dim() == 3:
            return ffn_fp8_block(x, w1, w1_scale, w2, w2_scale, ids, wts, sorted_ids,
                                 block_expert, num_padded, block_m, flags, stream=stream)
        return (ffn_w8a16 if weight_only else ffn_fp8)(x, w1, w1_scale, w2, w2_scale, ids, wts,
                                                       sorted_ids, block_expert, num_padded,
                                                       block_m, flags, stream=stream)
    if w1.dtype == torch.bfloat16:
        return ffn_bf16(x, w1, w2, ids, wts, sorted_ids, block_expert, num_padded, block_m,
                        flags, stream=stream)
    return ffn_f32(x, w1, w2, ids, wts, sorted_ids, block_expert, num_padded, block_m, flags,
                   stream=stream)


# ----------------------------------------------------- small-batch path ---

def small_max_tokens() -> int:
    return int(lib.moe_small_max_tokens())


def forward_small_workspace_bytes(T, E, H, I, k, dtype) -> int:
    return int(lib.moe_forward_small_workspace_bytes(T, E, H, I, k, dtype))


def _small_args(logits, x, w1, w2, k, fp8, w1_scale, w2_scale):
    """Shapes of a small-batch forward, checked against each other: logits
    [T, E], x [T, H], w1 [E, 2I, H], w2 [E, H, I], fp8 scales [E, 2I] and
    [E, H]. Returns (T, H, E, I, dtype)."""
    T, H = _dims(x, "x", 2)
    _need(x, "x", (torch.bfloat16,))
    dev = x.device
    E, I2, H1 = _dims(w1, "w1", 3)
    if H1 != H or I2 % 2:
        raise ValueError(f"w1 has shape {tuple(w1.shape)}, expected [E, 2I, H={H}]")
    I = I2 // 2
    _need(logits, "logits", (torch.float32,), dev, (T, E))
    wdt = _FP8 if fp8 else (torch.bfloat16,)
    _need(w1, "w1", wdt, dev)
    _need(w2, "w2", wdt, dev, (E, H, I))
    if fp8:
        _need(w1_scale, "w1_scale", (torch.float32,), dev, (E, 2 * I))
        _need(w2_scale, "w2_scale", (torch.float32,), dev, (E, H))
    return T, H, E, I, MOE_DTYPE_FP8 if fp8 else MOE_DTYPE_BF16


def _small_outputs(x, T, H, k, out, topk_ids, topk_weights):
    dev = x.device
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    else:
        _need(topk_ids, "topk_ids", (torch.int32,), dev, (T, k))
    if topk_weights is None:
        topk_weights = torch.empty((T, k), dtype=torch.float32, device=dev)
    else:
        _need(topk_weights, "topk_weights", (torch.float32,), dev, (T, k))
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", (torch.bfloat16,), dev, (T, H))
    return out, topk_ids, topk_weights


def forward_small(logits, x, w1, w2, k: int, renormalize: bool = False, w1_scale=None,
                  w2_scale=None, flags: int = 0, out=None, topk_ids=None, topk_weights=None,
                  workspace=None, stream=None, prepare: bool = False):
    """moe_forward_small: the whole layer in one call for T <= small_max_tokens():
    up to 16 tokens (and 256 slots) without an alignment step (separate
    launches; one cooperative launch with flags | FORWARD_ONE_KERNEL), beyond
    that routing, alignment and the FFN launches in its workspace. bf16 weights,
    or e4m3fn codes with per-row float32 scales (W8A8). Returns
    (out [T,H] bfloat16, topk_ids [T,k] int32, topk_weights [T,k] float32)."""
    fp8 = w1.dtype in _FP8
    T, H, E, I, dtype = _small_args(logits, x, w1, w2, k, fp8, w1_scale, w2_scale)
    out, topk_ids, topk_weights = _small_outputs(x, T, H, k, out, topk_ids, topk_weights)
    n = forward_small_workspace_bytes(T, E, H, I, k, dtype)
    if workspace is None:
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
    else:
        _need(workspace, "workspace", (torch.uint8,), x.device, min_numel=n)
    keep = (logits, x, w1, w2, w1_scale, w2_scale, topk_ids, topk_weights, workspace, out)
    args = (_ptr(logits), _ptr(x), _ptr(w1), _ptr(w1_scale) if fp8 else None, _ptr(w2),
            _ptr(w2_scale) if fp8 else None, T, E, H, I, k, 1 if renormalize else 0, dtype,
            flags, _ptr(topk_ids), _ptr(topk_weights), _ptr(workspace), workspace.numel(),
            _ptr(out), _stream(stream))
    return _run(lib.moe_forward_small, args, keep, prepare, (out, topk_ids, topk_weights))


def forward_small_static(logits, x, w1, w2, k: int, renormalize: bool = False, w1_scale=None,
                         w2_scale=None, flags: int = 0, out=None, topk_ids=None,
                         topk_weights=None, stream=None):
    """moe_forward_small_static: forward_small with the intermediates in the
    library's static per-GPU scratch (STATIC_SCRATCH_BYTES) instead of a
    workspace; the library call allocates nothing (pass ``out``, ``topk_ids``
    and ``topk_weights`` to allocate nothing here either). Calls that overlap
    in time on one GPU race. Returns (out, topk_ids, topk_weights)."""
    fp8 = w1.dtype in (torch.uint8, torch.float8_e4m3fn)
    T, H, E, I, dtype = _small_args(logits, x, w1, w2, k, fp8, w1_scale, w2_scale)
    out, topk_ids, topk_weights = _small_outputs(x, T, H, k, out, topk_ids, topk_weights)
    _check(lib.moe_forward_small_static(
        _ptr(logits), _ptr(x), _ptr(w1), _ptr(w1_scale) if fp8 else None, _ptr(w2),
        _ptr(w2_scale) if fp8 else None, T, E, H, I, k, 1 if renormalize else 0, dtype, flags,
        _ptr(topk_ids), _ptr(topk_weights), _ptr(out), _stream(stream)))
    return out, topk_ids, topk_weights
