"""CPU oracle of the two LoRA layers the melded layer is compared with.

TEST INFRASTRUCTURE ONLY (as the rest of oracle/): imported by tests/ and by
the CPU-baseline leg of bench.py, never by the HIP library.

Pages cited (by address and section):
* [P2] FALQON introduction, luneresearch.com: abstract and method paragraph
  (the melded layer removes the quantization overhead of a separate LoRA
  computational path).
* [P4] FALQON OpenReview rebuttal, paperhub.cn/paper/yPXOfBoQL7: thread 1,
  reply Q2 and Table R1 (LoRA adapter compute in FP16 against FP8; the FP8
  path only pays off near rank 8192), thread 2 reply W2 (per-tensor scaling
  to FP8).

Both layers keep the melded layer's FP8 backbone product and add the LoRA
adapter as its own branch, Y = X W^T + (X A^T) B^T, with the straight-through
backward dX = G W + (G B) A, dB = G^T (X A^T), dA = (G B)^T X.  They differ in
the precision of that branch:

* separate-path FP8 LoRA: every tensor entering a product is quantized per
  tensor to E4M3 (fp8_quantize, the reading of [P4] W2), the factors on
  every step since they train, and the rank-r intermediates U = X A^T and
  V = G B before they are used;
* BF16 LoRA: the branch in bfloat16 with fp32 accumulation from the
  unquantized X and dY; U and V are rounded to bfloat16 before they are used.

Reading: the pages name these comparison points without their arithmetic;
the branch is taken as the plainest LoRA layer at that precision, each
product accumulated exactly (float64) and rounded once to float32, each
quantization or bfloat16 rounding applied where the tensor is produced.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from . import e4m3
from .melded import fp8_quantize, melded_linear_fwd


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values -> the nearest bfloat16 values (ties to the even
    significand), returned as float32.  A bfloat16 is the top half of a
    binary32 pattern, so rounding keeps the top 16 bits and decides on the
    low 16: above half-way rounds up, below rounds down, exactly half-way goes
    to the pattern whose bit 16 is 0.  NaN stays NaN; values that round past
    the largest finite bfloat16 become infinities, as in binary32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    top = u >> 16
    up = (low > 0x8000) | ((low == 0x8000) & ((top & 1) == 1))
    r = ((top + up.astype(np.uint64)) << 16).astype(np.uint32)
    nan = np.isnan(x)
    r[nan] = (u[nan].astype(np.uint32) | 0x00400000) & 0xFFFF0000
    return r.view(np.float32)


def fp8_product(aq: np.ndarray, s_a: float, bq: np.ndarray, s_b: float) -> np.ndarray:
    """(sum_k dec(aq[i,k]) dec(bq[j,k])) / (s_a s_b) rounded once to float32:
    the product of two E4M3 tensors as the FP8 matrix cores form it (decoded
    products are exact and so are their float64 sums at these sizes)."""
    acc = e4m3.decode(aq) @ e4m3.decode(bq).T
    return (acc / (np.float64(np.float32(s_a)) * np.float64(np.float32(s_b)))).astype(np.float32)


def bf16_product(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """sum_k a[i,k] b[j,k] of bfloat16 values, exact in float64 (products of
    two 8-bit significands, sums at these sizes), rounded once to float32."""
    return (np.asarray(a, np.float64) @ np.asarray(b, np.float64).T).astype(np.float32)


def _add32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """a + b for float32 arrays, rounded to float32 (the branch is added onto
    the backbone product)."""
    return (np.asarray(a, np.float64) + np.asarray(b, np.float64)).astype(np.float32)


# ----------------------------------------------------------------------------
# separate-path FP8 LoRA
# ----------------------------------------------------------------------------
def lora_separate_fp8_fwd(xq, s_x, wq, s_w, A, B) -> Tuple[np.ndarray, dict]:
    """Forward of the layer with a separate FP8 LoRA branch ([P2]: the path
    the melded layer removes).
        A~, s_a = Q(A);  B~, s_b = Q(B)
        U = X^ A^^T                       (float32)
        U~, s_u = Q(U)
        Y = X^ W^^T + U^ B^^T              (the branch added onto the backbone)
    Returns (Y, saved) with saved = {aq, s_a, bq, s_b, uq, s_u}."""
    aq, s_a, _, _ = fp8_quantize(A)
    bq, s_b, _, _ = fp8_quantize(B)
    u = fp8_product(xq, s_x, aq, s_a)
    uq, s_u, _, _ = fp8_quantize(u)
    y0 = melded_linear_fwd(xq, s_x, wq, s_w)
    y = _add32(y0, fp8_product(uq, s_u, bq, s_b))
    return y, {"aq": aq, "s_a": s_a, "bq": bq, "s_b": s_b, "uq": uq, "s_u": s_u, "u": u}


def lora_separate_fp8_bwd(gq, s_g, xq, s_x, wq, s_w, saved: dict,
                          vq: Optional[np.ndarray] = None, s_v: Optional[float] = None):
    """Backward of the separate-path FP8 layer (straight-through through every
    quantization):
        V = G^ B^                         (float32);  V~, s_v = Q(V)
        dX = G^ W^ + V^ A^
        dB = G^^T U^,   dA = V^^T X^
    With vq, s_v given, those codes are used instead of Q(V) (to follow a
    computation whose V rounded otherwise near a code boundary).
    Returns (dX, dA, dB, vq, s_v, v)."""
    aq, s_a, bq, s_b = saved["aq"], saved["s_a"], saved["bq"], saved["s_b"]
    uq, s_u = saved["uq"], saved["s_u"]
    v = fp8_product(gq, s_g, np.ascontiguousarray(bq.T), s_b)
    if vq is None:
        vq, s_v, _, _ = fp8_quantize(v)
    dx0 = fp8_product(gq, s_g, np.ascontiguousarray(wq.T), s_w)
    dx = _add32(dx0, fp8_product(vq, s_v, np.ascontiguousarray(aq.T), s_a))
    dB = fp8_product(np.ascontiguousarray(gq.T), s_g, np.ascontiguousarray(uq.T), s_u)
    dA = fp8_product(np.ascontiguousarray(vq.T), s_v, np.ascontiguousarray(xq.T), s_x)
    return dx, dA, dB, vq, np.float32(s_v), v


# ----------------------------------------------------------------------------
# BF16 LoRA
# ----------------------------------------------------------------------------
def lora_bf16_fwd(X, xq, s_x, wq, s_w, A, B) -> Tuple[np.ndarray, np.ndarray]:
    """Forward of the FP8 backbone with a bfloat16 LoRA branch ([P4] thread 1,
    Table R1: the FP16 LoRA adapter the FP8 one is compared with):
        U = bf(X) bf(A)^T (float32), then bf(U)
        Y = X^ W^^T + bf(U) bf(B)^T
    Returns (Y, bf(U))."""
    u = bf16_product(bf16_round(X), bf16_round(A))
    ub = bf16_round(u)
    y0 = melded_linear_fwd(xq, s_x, wq, s_w)
    y = _add32(y0, bf16_product(ub, bf16_round(B)))
    return y, ub


def lora_bf16_bwd(dY, gq, s_g, X, wq, s_w, A, B, ub):
    """Backward of the bfloat16 LoRA layer:
        V = bf(dY) bf(B) (float32), then bf(V)
        dX = G^ W^ + bf(V) bf(A)
        dB = bf(dY)^T bf(U),   dA = bf(V)^T bf(X)
    Returns (dX, dA, dB, bf(V))."""
    gb, ab, bb, xb = (bf16_round(t) for t in (dY, A, B, X))
    vb = bf16_round(bf16_product(gb, np.ascontiguousarray(bb.T)))
    dx0 = fp8_product(gq, s_g, np.ascontiguousarray(wq.T), s_w)
    dx = _add32(dx0, bf16_product(vb, np.ascontiguousarray(ab.T)))
    dB = bf16_product(np.ascontiguousarray(gb.T), np.ascontiguousarray(np.asarray(ub).T))
    dA = bf16_product(np.ascontiguousarray(vb.T), np.ascontiguousarray(xb.T))
    return dx, dA, dB, vb
