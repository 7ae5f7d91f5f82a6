"""Python binding of libfalqon.so, the gfx950 HIP library of FALQON's melded
FP8 LoRA linear step.

Argument marshalling only: every function takes device tensors, checks
dtype/shape/contiguity, passes their device pointers and sizes to the C
function of the same name (include/falqon.h) and raises FalqError on a
non-zero status.  All computation runs in the library's HIP kernels on the
stream given (default: torch's current stream).  There is no fallback: if
the library is missing, load() raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["load", "FalqError", "fp8_quantize", "fp8_quantize_workspace_bytes",
           "melded_linear_fwd", "melded_linear_bwd", "melded_linear_bwd_workspace_bytes",
           "adapter_step", "adapter_step_adamw", "adamw_state", "ADAMW_STATE_BYTES",
           "rowwise_proxy_update", "rowwise_proxy_update_topk_rank",
           "rowwise_proxy_update_topk_rank_workspace_bytes",
           "fp8_dequantize", "melded_linear_fwd_frozen_a", "fp8_quantize_fmt",
           "melded_linear_bwd_fmt", "melded_linear_bwd_frozen_a_fmt", "FORMATS",
           "melded_linear_fwd_frozen_a_workspace_bytes", "melded_linear_bwd_frozen_a",
           "melded_linear_bwd_frozen_a_workspace_bytes", "rowwise_proxy_update_workspace_bytes",
           "fp4_quantize", "melded_linear_fwd_fp4", "version", "LIB_PATH",
           "fp8_quantize_noalloc", "QUANTIZE_SCRATCH_BYTES", "fp8_quantize_wait_ticks",
           "melded_linear_xa_fused", "melded_linear_fwd_xa", "melded_linear_bwd_xa",
           "melded_linear_bwd_xa_t", "rowwise_proxy_update_t", "fp8_transpose",
           "adapter_pieces_bytes", "adapter_pieces", "adapter_step_pieces",
           "melded_linear_fwd_xa_pieces",
           "melded_linear_fwd_xa_workspace_bytes", "melded_linear_bwd_xa_workspace_bytes",
           "lora_separate_fp8_saved_bytes", "lora_separate_fp8_workspace_bytes",
           "lora_separate_fp8_fwd", "lora_separate_fp8_bwd", "lora_bf16_saved_bytes",
           "lora_bf16_workspace_bytes", "lora_bf16_fwd", "lora_bf16_bwd"]

#: bytes of the per-device scratch array behind fp8_quantize_noalloc
QUANTIZE_SCRATCH_BYTES = 16384

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfalqon.so")
_lib = None

_c_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_f32 = ctypes.c_float
_i32 = ctypes.c_int

_SIGS = {
    "falq_status_string": (ctypes.c_char_p, [_i32]),
    "falq_version": (ctypes.c_char_p, []),
    "fp8_quantize_workspace_bytes": (_sz, [_i64]),
    "fp8_quantize": (_i32, [_c_p, _i32, _i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _sz, _c_p]),
    "melded_linear_fwd": (_i32, [_c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64, _c_p, _c_p]),
    "melded_linear_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "melded_linear_bwd": (_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _i64, _i64,
                                 _i64, _i64, _c_p, _c_p, _c_p, _c_p, _sz, _c_p]),
    "adapter_step": (_i32, [_c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64, _f32, _c_p]),
    "adapter_step_adamw": (_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _i64, _i64,
                                  _i64, _f32, _f32, _f32, _f32, _f32, _c_p, _c_p]),
    "fp8_dequantize": (_i32, [_c_p, _c_p, _i64, _c_p, _c_p]),
    "fp8_transpose": (_i32, [_c_p, _i64, _i64, _c_p, _c_p]),
    "fp8_quantize_fmt": (_i32, [_c_p, _i32, _i64, _i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _sz,
                                _c_p]),
    "melded_linear_bwd_fmt": (_i32, [_c_p, _i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _i64,
                                     _i64, _i64, _i64, _c_p, _c_p, _c_p, _c_p, _sz, _c_p]),
    "melded_linear_bwd_frozen_a_fmt": (_i32, [_c_p, _i32, _c_p, _c_p, _c_p, _c_p, _i64, _i64,
                                              _i64, _i64, _c_p, _c_p, _c_p, _sz, _c_p]),
    "melded_linear_fwd_frozen_a_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "melded_linear_fwd_frozen_a": (_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64,
                                          _i64, _c_p, _c_p, _c_p, _sz, _c_p]),
    "melded_linear_bwd_frozen_a_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "melded_linear_bwd_frozen_a": (_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64, _i64,
                                          _c_p, _c_p, _c_p, _sz, _c_p]),
    "rowwise_proxy_update_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "rowwise_proxy_update_topk_rank_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "rowwise_proxy_update_topk_rank": (_i32, [_c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64, _i64,
                                              _f32, _i64, _c_p, _c_p, _c_p, _c_p, _c_p, _sz,
                                              _c_p]),
    "rowwise_proxy_update": (_i32, [_c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64, _f32, _i64, _c_p,
                                    _c_p, _c_p, _c_p, _sz, _c_p]),
    "rowwise_proxy_update_t": (_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64, _f32, _i64,
                                      _c_p, _c_p, _c_p, _c_p, _sz, _c_p]),
    "fp4_quantize": (_i32, [_c_p, _i32, _i64, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _sz, _c_p]),
    "fp8_quantize_wait_ticks": (ctypes.c_uint64, [ctypes.c_uint64]),
    "fp8_quantize_noalloc": (_i32, [_c_p, _i32, _i64, _i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p]),
    "melded_linear_fwd_fp4": (_i32, [_c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64, _c_p, _c_p]),
    "melded_linear_xa_fused": (_i32, [_i64, _i64, _i64, _i64]),
    "adapter_pieces_bytes": (_sz, [_i64, _i64]),
    "adapter_pieces": (_i32, [_c_p, _i64, _i64, _c_p, _sz, _c_p]),
    "adapter_step_pieces": (_i32, [_c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64, _f32, _c_p, _sz,
                                   _c_p]),
    "melded_linear_fwd_xa_pieces": (_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _sz, _i64, _i64, _i64,
                                           _i64, _c_p, _c_p, _c_p]),
    "melded_linear_fwd_xa_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "melded_linear_fwd_xa": (_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64, _i64, _c_p,
                                    _c_p, _c_p, _sz, _c_p]),
    "melded_linear_bwd_xa_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "melded_linear_bwd_xa": (_i32, [_c_p, _i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                    _i64, _i64, _i64, _i64, _c_p, _c_p, _c_p, _c_p, _sz, _c_p]),
    "melded_linear_bwd_xa_t": (_i32, [_c_p, _i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                      _i64, _i64, _i64, _i64, _c_p, _c_p, _c_p, _c_p, _sz, _c_p]),
    "lora_separate_fp8_saved_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "lora_separate_fp8_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "lora_separate_fp8_fwd": (_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64, _i64,
                                     _c_p, _c_p, _sz, _c_p, _sz, _c_p]),
    "lora_separate_fp8_bwd": (_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _sz, _i64, _i64,
                                     _i64, _i64, _c_p, _c_p, _c_p, _c_p, _sz, _c_p]),
    "lora_bf16_saved_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "lora_bf16_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "lora_bf16_fwd": (_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _i64, _i64, _i64, _i64,
                             _c_p, _c_p, _sz, _c_p, _sz, _c_p]),
    "lora_bf16_bwd": (_i32, [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _sz, _i64,
                             _i64, _i64, _i64, _c_p, _c_p, _c_p, _c_p, _sz, _c_p]),
}


class FalqError(RuntimeError):
    pass


#: FP8 code formats (falq_fp8_format): OCP E4M3 and OCP E5M2
FORMATS = {"e4m3": 0, "e5m2": 1}


def _fmt(f) -> int:
    if f not in FORMATS:
        raise FalqError(f"format must be one of {sorted(FORMATS)}, not {f!r}")
    return FORMATS[f]


def load(path: Optional[str] = None):
    """Load libfalqon.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FalqError(f"{p} not found: build it with `python -c 'import __graft_entry__ as g; "
                        f"g.build()'` or `python fp8_quantized_lora_amd/build.py`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def version() -> str:
    return load().falq_version().decode()


def _check(status: int, what: str):
    if status != 0:
        msg = load().falq_status_string(status).decode()
        raise FalqError(f"{what}: {msg}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise FalqError("tensor arguments must live on the GPU")
    if not t.is_contiguous():
        raise FalqError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _req(t: torch.Tensor, dtype, shape, name):
    if t.dtype != dtype:
        raise FalqError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise FalqError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


# ---------------------------------------------------------------------------
def fp8_quantize_workspace_bytes(n: int) -> int:
    return int(load().fp8_quantize_workspace_bytes(n))


def fp8_quantize(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor,
                 scale_in: Optional[torch.Tensor] = None, amax: Optional[torch.Tensor] = None,
                 nonfinite: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                 stream=None, fmt: str = "e4m3") -> None:
    """q = FP8(x * s), s = max / amax(x); fmt "e4m3" (fp8_quantize) or "e5m2"
    (fp8_quantize_fmt)."""
    lib = load()
    if x.dtype == torch.float32:
        dt = 0
    elif x.dtype == torch.bfloat16:
        dt = 1
    else:
        raise FalqError("fp8_quantize: x must be float32 or bfloat16")
    n = x.numel()
    _req(q, torch.uint8, x.shape, "q")
    wsb = fp8_quantize_workspace_bytes(n)
    if ws is None:
        ws = torch.empty(wsb, dtype=torch.uint8, device=x.device)
    f = _fmt(fmt)
    if f == 0:
        _check(lib.fp8_quantize(_ptr(x), dt, n, _ptr(scale_in), _ptr(q), _ptr(scale), _ptr(amax),
                                _ptr(nonfinite), _ptr(ws), ws.numel(), _stream(stream)),
               "fp8_quantize")
    else:
        _check(lib.fp8_quantize_fmt(_ptr(x), dt, n, f, _ptr(scale_in), _ptr(q), _ptr(scale),
                                    _ptr(amax), _ptr(nonfinite), _ptr(ws), ws.numel(),
                                    _stream(stream)), "fp8_quantize_fmt")


def fp8_quantize_fmt(x, q, scale, fmt: str, **kw) -> None:
    fp8_quantize(x, q, scale, fmt=fmt, **kw)


def fp8_quantize_noalloc(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor,
                         scale_in: Optional[torch.Tensor] = None,
                         amax: Optional[torch.Tensor] = None,
                         nonfinite: Optional[torch.Tensor] = None, stream=None,
                         fmt: str = "e4m3") -> None:
    """fp8_quantize with no workspace: the library's per-device scratch array
    holds the amax partials (for callers that cannot allocate).  Calls that
    overlap on one GPU race on that array."""
    if x.dtype == torch.float32:
        dt = 0
    elif x.dtype == torch.bfloat16:
        dt = 1
    else:
        raise FalqError("fp8_quantize_noalloc: x must be float32 or bfloat16")
    _req(q, torch.uint8, x.shape, "q")
    _check(load().fp8_quantize_noalloc(_ptr(x), dt, x.numel(), _fmt(fmt), _ptr(scale_in),
                                       _ptr(q), _ptr(scale), _ptr(amax), _ptr(nonfinite),
                                       _stream(stream)), "fp8_quantize_noalloc")


def fp8_quantize_wait_ticks(ticks: int) -> int:
    """Set how long (100 MHz GPU counter ticks) the one-launch quantize waits
    for the other workgroups' maxima before reading their ranges itself;
    returns the previous setting."""
    if ticks < 0:
        raise FalqError("fp8_quantize_wait_ticks: ticks must be >= 0")
    return int(load().fp8_quantize_wait_ticks(int(ticks)))


def melded_linear_fwd(xq: torch.Tensor, s_x: torch.Tensor, wq: torch.Tensor, s_w: torch.Tensor,
                      y: torch.Tensor, stream=None) -> None:
    T, d_in = xq.shape
    d_out = wq.shape[0]
    _req(wq, torch.uint8, (d_out, d_in), "wq")
    _req(y, torch.float32, (T, d_out), "y")
    _check(load().melded_linear_fwd(_ptr(xq), _ptr(s_x), _ptr(wq), _ptr(s_w), T, d_in, d_out,
                                    _ptr(y), _stream(stream)), "melded_linear_fwd")


def fp4_quantize(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor,
                 scale_in: Optional[torch.Tensor] = None, amax: Optional[torch.Tensor] = None,
                 nonfinite: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                 stream=None) -> None:
    """q = FP4 E2M1(x * s), s = 6 / amax(x), two codes per byte along the last
    axis (q has the shape of x with the last axis halved)."""
    lib = load()
    if x.dtype == torch.float32:
        dt = 0
    elif x.dtype == torch.bfloat16:
        dt = 1
    else:
        raise FalqError("fp4_quantize: x must be float32 or bfloat16")
    if x.dim() == 0 or x.shape[-1] % 2:
        raise FalqError("fp4_quantize: the last axis of x must have even length")
    n = x.numel()
    _req(q, torch.uint8, tuple(x.shape[:-1]) + (x.shape[-1] // 2,), "q")
    wsb = fp8_quantize_workspace_bytes(n)
    if ws is None:
        ws = torch.empty(wsb, dtype=torch.uint8, device=x.device)
    _check(lib.fp4_quantize(_ptr(x), dt, n, _ptr(scale_in), _ptr(q), _ptr(scale), _ptr(amax),
                            _ptr(nonfinite), _ptr(ws), ws.numel(), _stream(stream)),
           "fp4_quantize")


def melded_linear_fwd_fp4(xq: torch.Tensor, s_x: torch.Tensor, wq: torch.Tensor,
                          s_w: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    """y = dec(xq) dec(wq)^T / (s_x s_w) with FP4 E2M1 operands (two codes per
    byte: xq [T x d_in/2], wq [d_out x d_in/2])."""
    T, half = xq.shape
    d_in = 2 * half
    d_out = wq.shape[0]
    _req(wq, torch.uint8, (d_out, half), "wq")
    _req(y, torch.float32, (T, d_out), "y")
    _check(load().melded_linear_fwd_fp4(_ptr(xq), _ptr(s_x), _ptr(wq), _ptr(s_w), T, d_in, d_out,
                                        _ptr(y), _stream(stream)), "melded_linear_fwd_fp4")


def melded_linear_bwd_workspace_bytes(T: int, d_in: int, d_out: int, r: int) -> int:
    return int(load().melded_linear_bwd_workspace_bytes(T, d_in, d_out, r))


def melded_linear_bwd(gq, s_g, xq, s_x, wq, s_w, A, B, dx, dA, dB, ws=None, stream=None,
                      g_fmt: str = "e4m3") -> None:
    T, d_out = gq.shape
    d_in = xq.shape[1]
    r = A.shape[0]
    _req(xq, torch.uint8, (T, d_in), "xq")
    _req(wq, torch.uint8, (d_out, d_in), "wq")
    _req(A, torch.float32, (r, d_in), "A")
    _req(B, torch.float32, (d_out, r), "B")
    _req(dB, torch.float32, (d_out, r), "dB")
    if dx is not None:
        _req(dx, torch.float32, (T, d_in), "dx")
    if dA is not None:
        _req(dA, torch.float32, (r, d_in), "dA")
    wsb = melded_linear_bwd_workspace_bytes(T, d_in, d_out, r)
    if ws is None:
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=gq.device)
    _check(load().melded_linear_bwd_fmt(_ptr(gq), _fmt(g_fmt), _ptr(s_g), _ptr(xq), _ptr(s_x),
                                        _ptr(wq), _ptr(s_w), _ptr(A), _ptr(B), T, d_in, d_out, r,
                                        _ptr(dx), _ptr(dA), _ptr(dB), _ptr(ws), ws.numel(),
                                        _stream(stream)), "melded_linear_bwd")


def melded_linear_bwd_fmt(gq, g_fmt: str, s_g, xq, s_x, wq, s_w, A, B, dx, dA, dB, **kw) -> None:
    melded_linear_bwd(gq, s_g, xq, s_x, wq, s_w, A, B, dx, dA, dB, g_fmt=g_fmt, **kw)


def fp8_dequantize(q: torch.Tensor, scale: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """out = dec(q) / scale (float32), elementwise."""
    _req(q, torch.uint8, tuple(q.shape), "q")
    _req(out, torch.float32, tuple(q.shape), "out")
    _req(scale, torch.float32, (1,), "scale")
    _check(load().fp8_dequantize(_ptr(q), _ptr(scale), q.numel(), _ptr(out), _stream(stream)),
           "fp8_dequantize")


def melded_linear_fwd_frozen_a_workspace_bytes(T: int, d_in: int, r: int) -> int:
    return int(load().melded_linear_fwd_frozen_a_workspace_bytes(T, d_in, r))


def melded_linear_fwd_frozen_a(xq, s_x, wq, s_w, aq, s_a, y, u, ws=None, stream=None) -> None:
    """y = X~ W~^T / (s_x s_w) and u = X~ A~^T / (s_x s_a)."""
    T, d_in = xq.shape
    d_out = wq.shape[0]
    r = aq.shape[0]
    _req(xq, torch.uint8, (T, d_in), "xq")
    _req(wq, torch.uint8, (d_out, d_in), "wq")
    _req(aq, torch.uint8, (r, d_in), "aq")
    _req(y, torch.float32, (T, d_out), "y")
    _req(u, torch.float32, (T, r), "u")
    need = melded_linear_fwd_frozen_a_workspace_bytes(T, d_in, r)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=xq.device)
    _check(load().melded_linear_fwd_frozen_a(_ptr(xq), _ptr(s_x), _ptr(wq), _ptr(s_w), _ptr(aq),
                                             _ptr(s_a), T, d_in, d_out, r, _ptr(y), _ptr(u),
                                             _ptr(ws), ws.numel(), _stream(stream)),
           "melded_linear_fwd_frozen_a")


def melded_linear_bwd_frozen_a_workspace_bytes(T: int, d_in: int, d_out: int, r: int) -> int:
    return int(load().melded_linear_bwd_frozen_a_workspace_bytes(T, d_in, d_out, r))


def melded_linear_bwd_frozen_a(gq, s_g, wq, s_w, u, dx, dB, ws=None, stream=None,
                               g_fmt: str = "e4m3") -> None:
    """dx = G~ W~ / (s_g s_w) (dx may be None) and dB = G^^T u."""
    T, d_out = gq.shape
    d_in = wq.shape[1]
    r = u.shape[1]
    _req(gq, torch.uint8, (T, d_out), "gq")
    _req(wq, torch.uint8, (d_out, d_in), "wq")
    _req(u, torch.float32, (T, r), "u")
    _req(dB, torch.float32, (d_out, r), "dB")
    if dx is not None:
        _req(dx, torch.float32, (T, d_in), "dx")
    need = melded_linear_bwd_frozen_a_workspace_bytes(T, d_in, d_out, r)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=gq.device)
    _check(load().melded_linear_bwd_frozen_a_fmt(_ptr(gq), _fmt(g_fmt), _ptr(s_g), _ptr(wq),
                                                 _ptr(s_w), _ptr(u), T, d_in, d_out, r, _ptr(dx),
                                                 _ptr(dB), _ptr(ws), ws.numel(), _stream(stream)),
           "melded_linear_bwd_frozen_a")


def melded_linear_bwd_frozen_a_fmt(gq, g_fmt: str, s_g, wq, s_w, u, dx, dB, **kw) -> None:
    melded_linear_bwd_frozen_a(gq, s_g, wq, s_w, u, dx, dB, g_fmt=g_fmt, **kw)


def adapter_step(A, B, dA, dB, lr: float, stream=None) -> None:
    r, d_in = A.shape
    d_out = B.shape[0]
    _req(B, torch.float32, (d_out, r), "B")
    _req(dB, torch.float32, (d_out, r), "dB")
    if dA is not None:
        _req(dA, torch.float32, (r, d_in), "dA")
    _check(load().adapter_step(_ptr(A), _ptr(B), _ptr(dA), _ptr(dB), r, d_in, d_out, lr,
                               _stream(stream)), "adapter_step")


#: bytes of the AdamW optimizer state (zero-filled before the first step)
ADAMW_STATE_BYTES = 64


def adamw_state(device="cuda") -> torch.Tensor:
    """A fresh AdamW state: zeros, before step 1 (int64 step count first)."""
    return torch.zeros(ADAMW_STATE_BYTES // 8, dtype=torch.int64, device=device)


def adapter_step_adamw(A, B, dA, dB, mA, vA, mB, vB, state, lr: float, beta1: float = 0.9,
                       beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0,
                       stream=None) -> None:
    """One AdamW step on A and B with moments mA, vA, mB, vB, in place; `state`
    (adamw_state()) carries the step count and is advanced by the call.  dA =
    None freezes A (mA and vA may then be None)."""
    r, d_in = A.shape
    d_out = B.shape[0]
    for t, name in ((B, "B"), (dB, "dB"), (mB, "mB"), (vB, "vB")):
        _req(t, torch.float32, (d_out, r), name)
    if dA is not None:
        for t, name in ((A, "A"), (dA, "dA"), (mA, "mA"), (vA, "vA")):
            _req(t, torch.float32, (r, d_in), name)
    if state.numel() * state.element_size() != ADAMW_STATE_BYTES:
        raise FalqError(f"state must be {ADAMW_STATE_BYTES} bytes (adamw_state())")
    _check(load().adapter_step_adamw(_ptr(A), _ptr(B), _ptr(dA), _ptr(dB), _ptr(mA), _ptr(vA),
                                     _ptr(mB), _ptr(vB), r, d_in, d_out, lr, beta1, beta2, eps,
                                     weight_decay, _ptr(state), _stream(stream)),
           "adapter_step_adamw")


def rowwise_proxy_update_workspace_bytes(d_in: int, d_out: int, r: int) -> int:
    return int(load().rowwise_proxy_update_workspace_bytes(d_in, d_out, r))


def rowwise_proxy_update_t(wq, wqT, s_w, A, B, tau: float, k_max: int, sel_idx, n_sel, rho=None,
                           ws=None, stream=None) -> None:
    """rowwise_proxy_update that also writes wqT = the updated wq, transposed."""
    d_out, d_in = wq.shape
    r = A.shape[0]
    _req(wqT, torch.uint8, (d_in, d_out), "wqT")
    _req(A, torch.float32, (r, d_in), "A")
    _req(B, torch.float32, (d_out, r), "B")
    _req(sel_idx, torch.int32, (d_out,), "sel_idx")
    if rho is not None:
        _req(rho, torch.float32, (d_out,), "rho")
    wsb = rowwise_proxy_update_workspace_bytes(d_in, d_out, r)
    if ws is None:
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=wq.device)
    _check(load().rowwise_proxy_update_t(_ptr(wq), _ptr(wqT), _ptr(s_w), _ptr(A), _ptr(B), d_in,
                                         d_out, r, tau, k_max, _ptr(sel_idx), _ptr(n_sel),
                                         _ptr(rho), _ptr(ws), ws.numel(), _stream(stream)),
           "rowwise_proxy_update_t")


def rowwise_proxy_update(wq, s_w, A, B, tau: float, k_max: int, sel_idx, n_sel, rho=None, ws=None,
                         stream=None) -> None:
    d_out, d_in = wq.shape
    r = A.shape[0]
    _req(A, torch.float32, (r, d_in), "A")
    _req(B, torch.float32, (d_out, r), "B")
    _req(sel_idx, torch.int32, (d_out,), "sel_idx")
    if rho is not None:
        _req(rho, torch.float32, (d_out,), "rho")
    wsb = rowwise_proxy_update_workspace_bytes(d_in, d_out, r)
    if ws is None:
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=wq.device)
    _check(load().rowwise_proxy_update(_ptr(wq), _ptr(s_w), _ptr(A), _ptr(B), d_in, d_out, r, tau,
                                       k_max, _ptr(sel_idx), _ptr(n_sel), _ptr(rho), _ptr(ws),
                                       ws.numel(), _stream(stream)), "rowwise_proxy_update")




def rowwise_proxy_update_topk_rank_workspace_bytes(d_in: int, d_out: int, r: int,
                                                   k_rank: int) -> int:
    return int(load().rowwise_proxy_update_topk_rank_workspace_bytes(d_in, d_out, r, k_rank))


def rowwise_proxy_update_topk_rank(wq, s_w, A, B, k_rank: int, tau: float, k_max: int, sel_idx,
                                   n_sel, comp_idx, rho=None, ws=None, stream=None) -> None:
    """The row-wise proxy update over the k_rank rank components of largest
    score (comp_idx receives them, ascending)."""
    d_out, d_in = wq.shape
    r = A.shape[0]
    _req(A, torch.float32, (r, d_in), "A")
    _req(B, torch.float32, (d_out, r), "B")
    _req(comp_idx, torch.int32, (k_rank,), "comp_idx")
    need = rowwise_proxy_update_topk_rank_workspace_bytes(d_in, d_out, r, k_rank)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=wq.device)
    _check(load().rowwise_proxy_update_topk_rank(
        _ptr(wq), _ptr(s_w), _ptr(A), _ptr(B), d_in, d_out, r, k_rank, tau, k_max, _ptr(sel_idx),
        _ptr(n_sel), _ptr(rho), _ptr(comp_idx), _ptr(ws), ws.numel(), _stream(stream)),
        "rowwise_proxy_update_topk_rank")


# ---------------------------------------------------------------------------
# X^ A^T formed with the forward product, G^ B with the dX product
def melded_linear_xa_fused(T: int, d_in: int, d_out: int, r: int) -> bool:
    """Whether X^ A^T and G^ B ride in the FP8 products for this shape."""
    return bool(load().melded_linear_xa_fused(T, d_in, d_out, r))


def melded_linear_fwd_xa_workspace_bytes(T: int, d_in: int, d_out: int, r: int) -> int:
    return int(load().melded_linear_fwd_xa_workspace_bytes(T, d_in, d_out, r))


def melded_linear_bwd_xa_workspace_bytes(T: int, d_in: int, d_out: int, r: int) -> int:
    return int(load().melded_linear_bwd_xa_workspace_bytes(T, d_in, d_out, r))


def melded_linear_fwd_xa(xq, s_x, wq, s_w, A, y, xa, ws=None, stream=None) -> None:
    """y = X~ W~^T / (s_x s_w) and xa = X^ A^T (the factor dB needs)."""
    T, d_in = xq.shape
    d_out = wq.shape[0]
    r = A.shape[0]
    _req(wq, torch.uint8, (d_out, d_in), "wq")
    _req(A, torch.float32, (r, d_in), "A")
    _req(y, torch.float32, (T, d_out), "y")
    _req(xa, torch.float32, (T, r), "xa")
    ws = _buf(ws, melded_linear_fwd_xa_workspace_bytes(T, d_in, d_out, r), xq.device, "ws")
    _check(load().melded_linear_fwd_xa(_ptr(xq), _ptr(s_x), _ptr(wq), _ptr(s_w), _ptr(A), T, d_in,
                                       d_out, r, _ptr(y), _ptr(xa), _ptr(ws), ws.numel(),
                                       _stream(stream)), "melded_linear_fwd_xa")


def adapter_pieces_bytes(r: int, d_in: int) -> int:
    """Bytes of the buffer that holds A's pieces (0: not available)."""
    return int(load().adapter_pieces_bytes(r, d_in))


def adapter_pieces(A, pieces, stream=None) -> None:
    """A's block-scaled E4M3 pieces into `pieces` (uint8, adapter_pieces_bytes)."""
    r, d_in = A.shape
    _req(A, torch.float32, (r, d_in), "A")
    _check(load().adapter_pieces(_ptr(A), r, d_in, _ptr(pieces), pieces.numel(),
                                 _stream(stream)), "adapter_pieces")


def adapter_step_pieces(A, B, dA, dB, lr: float, pieces, stream=None) -> None:
    """adapter_step (SGD on A and B), and the pieces of the new A into `pieces`."""
    r, d_in = A.shape
    d_out = B.shape[0]
    _req(A, torch.float32, (r, d_in), "A")
    _req(dA, torch.float32, (r, d_in), "dA")
    _req(B, torch.float32, (d_out, r), "B")
    _req(dB, torch.float32, (d_out, r), "dB")
    _check(load().adapter_step_pieces(_ptr(A), _ptr(B), _ptr(dA), _ptr(dB), r, d_in, d_out, lr,
                                      _ptr(pieces), pieces.numel(), _stream(stream)),
           "adapter_step_pieces")


def melded_linear_fwd_xa_pieces(xq, s_x, wq, s_w, pieces, r: int, y, xa, stream=None) -> None:
    """melded_linear_fwd_xa with A given as its pieces (adapter_pieces / adapter_step_pieces)."""
    T, d_in = xq.shape
    d_out = wq.shape[0]
    _req(wq, torch.uint8, (d_out, d_in), "wq")
    _req(y, torch.float32, (T, d_out), "y")
    _req(xa, torch.float32, (T, r), "xa")
    _check(load().melded_linear_fwd_xa_pieces(_ptr(xq), _ptr(s_x), _ptr(wq), _ptr(s_w),
                                              _ptr(pieces), pieces.numel(), T, d_in, d_out, r,
                                              _ptr(y), _ptr(xa), _stream(stream)),
           "melded_linear_fwd_xa_pieces")


def melded_linear_bwd_xa(gq, s_g, xq, s_x, wq, s_w, A, B, xa, dx, dA, dB, ws=None, stream=None,
                         g_fmt: str = "e4m3", wq_t: bool = False) -> None:
    """dx, dA = (G^ B)^T X^ and dB = G^^T xa, with xa from melded_linear_fwd_xa.
    wq_t: wq is the backbone's transpose [d_in x d_out] (melded_linear_bwd_xa_t)."""
    T, d_out = gq.shape
    d_in = xq.shape[1]
    r = A.shape[0]
    _req(wq, torch.uint8, (d_in, d_out) if wq_t else (d_out, d_in), "wqT" if wq_t else "wq")
    _req(A, torch.float32, (r, d_in), "A")
    _req(B, torch.float32, (d_out, r), "B")
    _req(xa, torch.float32, (T, r), "xa")
    _req(dB, torch.float32, (d_out, r), "dB")
    if dx is not None:
        _req(dx, torch.float32, (T, d_in), "dx")
    if dA is not None:
        _req(dA, torch.float32, (r, d_in), "dA")
    ws = _buf(ws, melded_linear_bwd_xa_workspace_bytes(T, d_in, d_out, r), gq.device, "ws")
    name = "melded_linear_bwd_xa_t" if wq_t else "melded_linear_bwd_xa"
    _check(getattr(load(), name)(_ptr(gq), _fmt(g_fmt), _ptr(s_g), _ptr(xq), _ptr(s_x),
                                 _ptr(wq), _ptr(s_w), _ptr(A), _ptr(B), _ptr(xa), T, d_in,
                                 d_out, r, _ptr(dx), _ptr(dA), _ptr(dB), _ptr(ws),
                                 ws.numel(), _stream(stream)), name)


def melded_linear_bwd_xa_t(gq, s_g, xq, s_x, wqT, s_w, A, B, xa, dx, dA, dB, ws=None,
                           stream=None, g_fmt: str = "e4m3") -> None:
    """melded_linear_bwd_xa with the backbone handed in transposed, wqT [d_in x d_out]."""
    melded_linear_bwd_xa(gq, s_g, xq, s_x, wqT, s_w, A, B, xa, dx, dA, dB, ws=ws, stream=stream,
                         g_fmt=g_fmt, wq_t=True)


def fp8_transpose(q: torch.Tensor, qT: torch.Tensor, stream=None) -> None:
    """qT = q^T for a byte matrix (rows and columns multiples of 16)."""
    rows, cols = q.shape
    _req(q, torch.uint8, (rows, cols), "q")
    _req(qT, torch.uint8, (cols, rows), "qT")
    _check(load().fp8_transpose(_ptr(q), rows, cols, _ptr(qT), _stream(stream)), "fp8_transpose")


# ---------------------------------------------------------------------------
# the baselines: LoRA with a separate adapter branch (separate-path FP8, bf16)
def lora_separate_fp8_saved_bytes(T: int, d_in: int, d_out: int, r: int) -> int:
    return int(load().lora_separate_fp8_saved_bytes(T, d_in, d_out, r))


def lora_separate_fp8_workspace_bytes(T: int, d_in: int, d_out: int, r: int) -> int:
    return int(load().lora_separate_fp8_workspace_bytes(T, d_in, d_out, r))


def lora_bf16_saved_bytes(T: int, d_in: int, d_out: int, r: int) -> int:
    return int(load().lora_bf16_saved_bytes(T, d_in, d_out, r))


def lora_bf16_workspace_bytes(T: int, d_in: int, d_out: int, r: int) -> int:
    return int(load().lora_bf16_workspace_bytes(T, d_in, d_out, r))


def _buf(t, nbytes, device, name):
    if t is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if t.numel() * t.element_size() < nbytes:
        raise FalqError(f"{name}: needs {nbytes} bytes")
    return t


def lora_separate_fp8_fwd(xq, s_x, wq, s_w, A, B, y, saved, ws=None, stream=None) -> None:
    """Y = X^ W^^T + Q(X^ Q(A)^T)^ Q(B)^^T: the layer with a separate FP8 LoRA
    branch; `saved` (lora_separate_fp8_saved_bytes, uint8) keeps A~, B~, U~
    and their scales for the backward."""
    T, d_in = xq.shape
    d_out = wq.shape[0]
    r = A.shape[0]
    _req(wq, torch.uint8, (d_out, d_in), "wq")
    _req(A, torch.float32, (r, d_in), "A")
    _req(B, torch.float32, (d_out, r), "B")
    _req(y, torch.float32, (T, d_out), "y")
    ws = _buf(ws, lora_separate_fp8_workspace_bytes(T, d_in, d_out, r), xq.device, "ws")
    _check(load().lora_separate_fp8_fwd(_ptr(xq), _ptr(s_x), _ptr(wq), _ptr(s_w), _ptr(A),
                                        _ptr(B), T, d_in, d_out, r, _ptr(y), _ptr(saved),
                                        saved.numel() * saved.element_size(), _ptr(ws),
                                        ws.numel(), _stream(stream)), "lora_separate_fp8_fwd")


def lora_separate_fp8_bwd(gq, s_g, xq, s_x, wq, s_w, saved, r: int, dx, dA, dB, ws=None,
                          stream=None) -> None:
    """dX, dA, dB of the separate-path FP8 LoRA layer from the forward's `saved`."""
    T, d_out = gq.shape
    d_in = xq.shape[1]
    _req(dx, torch.float32, (T, d_in), "dx")
    _req(dA, torch.float32, (r, d_in), "dA")
    _req(dB, torch.float32, (d_out, r), "dB")
    ws = _buf(ws, lora_separate_fp8_workspace_bytes(T, d_in, d_out, r), gq.device, "ws")
    _check(load().lora_separate_fp8_bwd(_ptr(gq), _ptr(s_g), _ptr(xq), _ptr(s_x), _ptr(wq),
                                        _ptr(s_w), _ptr(saved),
                                        saved.numel() * saved.element_size(), T, d_in, d_out, r,
                                        _ptr(dx), _ptr(dA), _ptr(dB), _ptr(ws), ws.numel(),
                                        _stream(stream)), "lora_separate_fp8_bwd")


def lora_bf16_fwd(x, xq, s_x, wq, s_w, A, B, y, saved, ws=None, stream=None) -> None:
    """Y = X^ W^^T + bf(bf(X) bf(A)^T) bf(B)^T: the FP8 backbone with a bf16
    LoRA branch; `saved` (lora_bf16_saved_bytes) keeps bf(U)."""
    T, d_in = xq.shape
    d_out = wq.shape[0]
    r = A.shape[0]
    _req(x, torch.float32, (T, d_in), "x")
    _req(A, torch.float32, (r, d_in), "A")
    _req(B, torch.float32, (d_out, r), "B")
    _req(y, torch.float32, (T, d_out), "y")
    ws = _buf(ws, lora_bf16_workspace_bytes(T, d_in, d_out, r), xq.device, "ws")
    _check(load().lora_bf16_fwd(_ptr(x), _ptr(xq), _ptr(s_x), _ptr(wq), _ptr(s_w), _ptr(A),
                                _ptr(B), T, d_in, d_out, r, _ptr(y), _ptr(saved),
                                saved.numel() * saved.element_size(), _ptr(ws), ws.numel(),
                                _stream(stream)), "lora_bf16_fwd")


def lora_bf16_bwd(dy, gq, s_g, x, wq, s_w, A, B, saved, dx, dA, dB, ws=None,
                  stream=None) -> None:
    """dX, dA, dB of the bf16 LoRA layer from the forward's `saved`."""
    T, d_out = gq.shape
    d_in = x.shape[1]
    r = A.shape[0]
    _req(dy, torch.float32, (T, d_out), "dy")
    _req(dx, torch.float32, (T, d_in), "dx")
    _req(dA, torch.float32, (r, d_in), "dA")
    _req(dB, torch.float32, (d_out, r), "dB")
    ws = _buf(ws, lora_bf16_workspace_bytes(T, d_in, d_out, r), gq.device, "ws")
    _check(load().lora_bf16_bwd(_ptr(dy), _ptr(gq), _ptr(s_g), _ptr(x), _ptr(wq), _ptr(s_w),
                                _ptr(A), _ptr(B), _ptr(saved),
                                saved.numel() * saved.element_size(), T, d_in, d_out, r,
                                _ptr(dx), _ptr(dA), _ptr(dB), _ptr(ws), ws.numel(),
                                _stream(stream)), "lora_bf16_bwd")


from .step import MeldedLinear  # noqa: E402  (buffers + the step's call sequence)
__all__.append("MeldedLinear")
