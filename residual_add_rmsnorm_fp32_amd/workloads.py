"""Seeded synthetic inputs for the fused add + RMSNorm epilogue.

This module only draws random numbers and stores them in the storage dtypes. It holds
none of the epilogue's arithmetic, imports neither the HIP binding nor the CPU oracle,
and is the one piece of code both sides of a parity test share.

The five named workloads follow the configurations the pages' method is measured on
(partials, residual and gamma distributions, eps, weight_bias, quantisation). Each
tensor is drawn in float64 from ``numpy.random.Generator(PCG64(seed))`` and then stored
in bf16 or fp16 by a library conversion (numpy for fp16, torch for bf16). Draw order:
partials p = 0..P-1, residual, gamma, then the outlier rows.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

QUANT_MODES = ("none", "static", "dynamic")


@dataclass(frozen=True)
class Workload:
    name: str
    P: int
    T: int
    H: int
    dtype: str                      # "bf16" | "fp16"
    partial_dist: tuple             # ("normal", mu, sigma)
    residual_dist: tuple
    gamma_dist: tuple               # ("normal", mu, sigma) | ("uniform", lo, hi)
    eps: float
    weight_bias: float
    quant: str                      # "none" | "static" | "dynamic"
    seed: int
    static_scale: float | None = None
    outlier_fraction: float = 0.0   # fraction of token rows scaled in every partial
    outlier_factor: float = 1.0
    view_shape: tuple | None = None  # leading dims the caller passes (flattened to T)
    sweep_T: tuple = field(default_factory=tuple)
    description: str = ""

    @property
    def elem_bytes(self) -> int:
        return 2


WORKLOADS = {
    "c1": Workload(
        name="c1", P=2, T=16, H=2048, dtype="bf16",
        partial_dist=("normal", 0.0, 1.0), residual_dist=("normal", 0.0, 1.0),
        gamma_dist=("normal", 1.0, 0.1), eps=1e-6, weight_bias=0.0, quant="none",
        seed=20261201,
        description="P=2 bf16 [16,2048], no quant"),
    "c2": Workload(
        name="c2", P=8, T=80, H=4096, dtype="bf16",
        partial_dist=("normal", 0.0, 0.5), residual_dist=("normal", 0.0, 2.0),
        gamma_dist=("normal", 1.0, 0.1), eps=1e-6, weight_bias=0.0, quant="none",
        seed=20261202, sweep_T=(1, 8, 32),
        description="decode: P=8 bf16 [80,4096], no quant (swept at T=1,8,32)"),
    "c3": Workload(
        name="c3", P=4, T=64, H=8192, dtype="bf16",
        partial_dist=("normal", 0.0, 1.0), residual_dist=("normal", 0.0, 1.0),
        gamma_dist=("normal", 1.0, 0.1), eps=1e-5, weight_bias=0.0, quant="static",
        static_scale=0.05, seed=20261203,
        description="P=4 bf16 [64,8192], static per-tensor fp8, S=0.05"),
    "c4": Workload(
        name="c4", P=2, T=2048, H=5120, dtype="bf16",
        partial_dist=("normal", 0.0, 1.0), residual_dist=("normal", 0.0, 1.0),
        gamma_dist=("uniform", 0.5, 1.5), eps=1e-6, weight_bias=0.0, quant="dynamic",
        outlier_fraction=0.01, outlier_factor=50.0, seed=20261204,
        description="prefill: P=2 bf16 [2048,5120], 1% outlier rows x50, dynamic per-token fp8"),
    "c5": Workload(
        name="c5", P=8, T=16384, H=3584, dtype="fp16",
        partial_dist=("normal", 0.0, 0.25), residual_dist=("normal", 0.0, 1.0),
        gamma_dist=("normal", 0.0, 0.1), eps=1e-6, weight_bias=1.0, quant="none",
        seed=20261205, view_shape=(4, 4096, 3584),
        description="Gemma-style weight_bias=1, fp16 [4,4096,3584] -> [16384,3584], P=8"),
}


def to_codes(values: np.ndarray, dtype: str) -> np.ndarray:
    """Store float64 values in ``dtype``; returns the raw uint16 codes."""
    values = np.ascontiguousarray(values, dtype=np.float64)
    if dtype == "fp16":
        return values.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(values).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def _draw(rng: np.random.Generator, dist: tuple, shape) -> np.ndarray:
    kind = dist[0]
    if kind == "normal":
        return rng.normal(dist[1], dist[2], shape)
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], shape)
    raise ValueError(kind)


def make_inputs(wl: Workload, T: int | None = None, P: int | None = None) -> dict:
    """Draw the workload's inputs. Returns a dict of numpy arrays:

    ``partials`` [P, T, H] codes, ``residual`` [T, H] codes, ``gamma`` [H] codes,
    ``scale`` float32 [1] (static quant only, else None), ``outlier_rows`` (indices).
    ``T`` smaller than the workload's takes the first T rows of the full draw.
    """
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    P_all = wl.P
    partials = np.empty((P_all, wl.T, wl.H), dtype=np.uint16)
    raw = []
    for p in range(P_all):
        raw.append(_draw(rng, wl.partial_dist, (wl.T, wl.H)))
    residual = to_codes(_draw(rng, wl.residual_dist, (wl.T, wl.H)), wl.dtype)
    gamma = to_codes(_draw(rng, wl.gamma_dist, (wl.H,)), wl.dtype)
    outliers = np.array([], dtype=np.int64)
    if wl.outlier_fraction > 0:
        n_out = int(wl.T * wl.outlier_fraction)
        outliers = np.sort(rng.choice(wl.T, n_out, replace=False))
        for p in range(P_all):
            raw[p][outliers, :] *= wl.outlier_factor
    for p in range(P_all):
        partials[p] = to_codes(raw[p], wl.dtype)
        raw[p] = None
    t = wl.T if T is None else T
    p_used = P_all if P is None else P
    scale = None
    if wl.quant == "static":
        scale = np.array([wl.static_scale], dtype=np.float32)
    return {
        "partials": np.ascontiguousarray(partials[:p_used, :t]),
        "residual": np.ascontiguousarray(residual[:t]),
        "gamma": gamma,
        "scale": scale,
        "outlier_rows": outliers[outliers < t],
    }


def random_case(seed: int, P: int, T: int, H: int, dtype: str = "bf16",
                partial_sigma: float = 1.0, residual_sigma: float = 1.0,
                gamma_mu: float = 1.0, gamma_sigma: float = 0.1) -> dict:
    """Small seeded case of arbitrary shape (normal partials, residual and gamma)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    partials = np.stack([to_codes(rng.normal(0.0, partial_sigma, (T, H)), dtype)
                         for _ in range(P)]) if T > 0 else np.zeros((P, 0, H), np.uint16)
    residual = to_codes(rng.normal(0.0, residual_sigma, (T, H)), dtype)
    gamma = to_codes(rng.normal(gamma_mu, gamma_sigma, (H,)), dtype)
    return {"partials": partials, "residual": residual, "gamma": gamma}


def algorithmic_bytes(P: int, T: int, H: int, elem_bytes: int, quant: str,
                      with_norm_out: bool, with_residual: bool = True,
                      with_residual_out: bool = True) -> int:
    """Bytes the method must move per call, each stream once:
    P partials read, residual read, new residual written, norm_out written (if
    requested), fp8 codes written (quant), gamma once, static scale read, dynamic
    scales written (one per token, one per 128-element group, or one per tensor)."""
    per_elem = P * elem_bytes
    per_elem += elem_bytes if with_residual else 0
    per_elem += elem_bytes if with_residual_out else 0
    per_elem += elem_bytes if with_norm_out else 0
    per_elem += 1 if quant != "none" else 0
    b = T * H * per_elem + H * elem_bytes
    if quant == "static":
        b += 4
    elif quant == "dynamic":
        b += 4 * T
    elif quant == "group":
        b += 4 * T * -(-H // 128)
    elif quant == "tensor":
        b += 4
    return b


def with_overrides(wl: Workload, **kw) -> Workload:
    return replace(wl, **kw)
