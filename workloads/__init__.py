"""Seeded synthetic workloads for the melded FP8 LoRA linear step.

This module only *draws* inputs.  It holds none of the method's arithmetic
(no FP8 encoding, no scaling, no GEMMs): both the CPU oracle and the HIP path
consume the arrays it returns, so it is the one piece they share.

Every tensor is drawn from NumPy's PCG64 seeded with
``SeedSequence([config_id, linear_index, tensor_id, step])``: standard normals
in float64, multiplied by the stated standard deviation, then rounded to
float32 (round to nearest even).  Tensor ids: W=1, X=2, dY=3, A=4, B=5,
outlier-channel choice=6.

Shapes follow the PyTorch ``nn.Linear`` convention: W is [d_out x d_in],
X is [T x d_in], dY is [T x d_out], A is [r x d_in], B is [d_out x r].
Where a workload text gives ``N(0, v)``, v is a standard deviation, except for
the adapter factor A whose ``N(0, 1/r)`` is read as a variance (std 1/sqrt(r)),
so that the accumulated adapter delta reaches the size of one FP8 step on a
fraction of the rows instead of on none of them.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

T_W, T_X, T_DY, T_A, T_B, T_OUTLIER = 1, 2, 3, 4, 5, 6


@dataclasses.dataclass(frozen=True)
class LinearSpec:
    """One melded linear layer of a workload."""
    name: str
    d_out: int
    d_in: int
    tokens: int
    rank: int
    w_std: float = 0.02
    x_std: float = 1.0
    dy_std: float = 1e-3
    b_std: float = 1e-3          # 0.0 -> B starts at zero
    outlier_frac: float = 0.0    # fraction of input channels scaled by outlier_gain
    outlier_gain: float = 20.0
    x_bf16: bool = False         # X drawn in fp32 then rounded to bf16 and passed as bf16
    lr: float = 1e-3
    tau: float = 0.5             # row threshold in units of the row's E4M3 step
    k_max: int = 0               # 0 = no cap on the number of merged rows


@dataclasses.dataclass(frozen=True)
class Workload:
    config_id: int
    name: str
    linears: List[LinearSpec]
    steps: int = 1


def _rng(config_id: int, linear_idx: int, tensor_id: int, step: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([config_id, linear_idx, tensor_id, step])))


def _normal(config_id, linear_idx, tensor_id, step, shape, std) -> np.ndarray:
    g = _rng(config_id, linear_idx, tensor_id, step)
    return (g.standard_normal(shape, dtype=np.float64) * std).astype(np.float32)


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even) and return the 16-bit patterns.

    Used only to *store* a workload's activations in bf16, as the 7B MLP
    workload asks; it is input preparation, not part of the method.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_fp32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_linear(cfg_id: int, li: int, spec: LinearSpec, step: int = 0,
                rank: Optional[int] = None) -> dict:
    """Draw W, X, dY, A, B for one linear.  X and dY depend on `step`;
    W, A and B are the step-0 initial state."""
    r = spec.rank if rank is None else rank
    out = {}
    out["W"] = _normal(cfg_id, li, T_W, 0, (spec.d_out, spec.d_in), spec.w_std)
    x = _normal(cfg_id, li, T_X, step, (spec.tokens, spec.d_in), spec.x_std)
    n_out = int(round(spec.outlier_frac * spec.d_in))
    if n_out > 0:
        cols = _rng(cfg_id, li, T_OUTLIER, 0).choice(spec.d_in, size=n_out, replace=False)
        x[:, np.sort(cols)] *= np.float32(spec.outlier_gain)
        out["outlier_cols"] = np.sort(cols)
    if spec.x_bf16:
        out["X_bf16"] = fp32_to_bf16_bits(x)
        x = bf16_bits_to_fp32(out["X_bf16"])
    out["X"] = x
    out["dY"] = _normal(cfg_id, li, T_DY, step, (spec.tokens, spec.d_out), spec.dy_std)
    out["A"] = _normal(cfg_id, li, T_A, 0, (r, spec.d_in), 1.0 / np.sqrt(r)) if r > 0 \
        else np.zeros((0, spec.d_in), np.float32)
    if spec.b_std > 0 and r > 0:
        out["B"] = _normal(cfg_id, li, T_B, 0, (spec.d_out, r), spec.b_std)
    else:
        out["B"] = np.zeros((spec.d_out, r), np.float32)
    return out


def step_activations(cfg_id: int, li: int, spec: LinearSpec, step: int) -> dict:
    """X (and its bf16 form) and dY for a later step, without redrawing W, A, B."""
    d = {}
    x = _normal(cfg_id, li, T_X, step, (spec.tokens, spec.d_in), spec.x_std)
    n_out = int(round(spec.outlier_frac * spec.d_in))
    if n_out > 0:
        cols = _rng(cfg_id, li, T_OUTLIER, 0).choice(spec.d_in, size=n_out, replace=False)
        x[:, np.sort(cols)] *= np.float32(spec.outlier_gain)
    if spec.x_bf16:
        d["X_bf16"] = fp32_to_bf16_bits(x)
        x = bf16_bits_to_fp32(d["X_bf16"])
    d["X"] = x
    d["dY"] = _normal(cfg_id, li, T_DY, step, (spec.tokens, spec.d_out), spec.dy_std)
    return d


# --------------------------------------------------------------------------
# The five workloads (single linear; 7B attention projection; 7B MLP;
# 13B decoder layer; rank sweep).
# --------------------------------------------------------------------------
WORKLOADS = {
    1: Workload(1, "single_linear_512", [
        LinearSpec("linear", 512, 512, 256, 16, w_std=0.02, x_std=1.0, dy_std=1e-2,
                   b_std=0.0)], steps=1),
    2: Workload(2, "attn_proj_7b_4096", [
        LinearSpec("attn_proj", 4096, 4096, 4096, 64, dy_std=1e-3, b_std=1e-3,
                   outlier_frac=0.01, outlier_gain=20.0)], steps=10),
    3: Workload(3, "mlp_7b", [
        LinearSpec("gate", 11008, 4096, 8192, 64, x_bf16=True),
        LinearSpec("up", 11008, 4096, 8192, 64, x_bf16=True),
        LinearSpec("down", 4096, 11008, 8192, 64, x_bf16=True)], steps=1),
    4: Workload(4, "decoder_layer_13b", [
        LinearSpec("q", 5120, 5120, 4096, 64), LinearSpec("k", 5120, 5120, 4096, 64),
        LinearSpec("v", 5120, 5120, 4096, 64), LinearSpec("o", 5120, 5120, 4096, 64),
        LinearSpec("gate", 13824, 5120, 4096, 64), LinearSpec("up", 13824, 5120, 4096, 64),
        LinearSpec("down", 5120, 13824, 4096, 64)], steps=1),
    5: Workload(5, "rank_sweep_4096", [
        LinearSpec("linear", 4096, 4096, 8192, 64, b_std=1e-3)], steps=1),
}
RANK_SWEEP = (8, 64, 512, 2048, 8192)


def step_flops(T: int, d_in: int, d_out: int, r: int, frozen_a: bool = False) -> int:
    """Algorithmic flops of one melded-linear step: forward and dX FP8 GEMMs,
    the four rank-r adapter contractions (two with A frozen: X A^T and the dB
    product), and the rank-r row delta B.A."""
    adapter = (2 if frozen_a else 4) * T * r * (d_in + d_out)
    return 4 * T * d_in * d_out + adapter + 2 * d_out * d_in * r
