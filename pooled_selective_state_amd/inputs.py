"""Seeded synthetic inputs for the pooled selective-scan layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Both the GPU tests and the CPU oracle consume what it
returns, so the two sides always see bit-identical inputs.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per workload, draws in
this order):

1. ``x`` ~ N(0, 1), fp32, shape (B, h, w, E) dense or (B, K, E) masked;
2. ``z`` of block 0, same distribution and shape;
3. per block, then per direction (fwd, bwd):
   ``x_proj_w`` = 0.02 * N(0,1) of shape (R + 2N, E);
   ``dt_proj_w`` = 0.02 * N(0,1) of shape (E, R);
   ``dt0`` = exp(U(ln 1e-3, ln 1e-1)) per channel, in fp64, and
   ``dt_proj_b`` = dt0 + log(-expm1(-dt0)) (the inverse of softplus, so that
   the step size starts at dt0), cast to fp32;
   ``A_log[e, n]`` = log(n + 1); ``D`` = 1;
4. ``z`` of every later block (chained workloads);
5. masked workloads: per image, the first K entries of a permutation of h*w,
   int32, unsorted.

bf16 workloads round x and z to the nearest-even bf16 value; the arrays stay
float32 holding exactly representable bf16 values.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np

from .configs import LayerConfig

DIRECTIONS = ("fwd", "bwd")


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def draw_dir_params(rng: np.random.Generator, E: int, N: int, R: int) -> Dict[str, np.ndarray]:
    x_proj_w = (0.02 * rng.standard_normal((R + 2 * N, E), dtype=np.float32)).astype(np.float32)
    dt_proj_w = (0.02 * rng.standard_normal((E, R), dtype=np.float32)).astype(np.float32)
    dt0 = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), E))
    dt_proj_b = (dt0 + np.log(-np.expm1(-dt0))).astype(np.float32)
    A_log = np.tile(np.log(np.arange(1, N + 1, dtype=np.float64)), (E, 1)).astype(np.float32)
    D = np.ones(E, np.float32)
    return {"x_proj_w": x_proj_w, "dt_proj_w": dt_proj_w, "dt_proj_b": dt_proj_b,
            "A_log": A_log, "D": D}


def draw_workload(cfg: LayerConfig, seed: int = 0, batch: int | None = None) -> Dict[str, object]:
    """Draw x, the per-block z and parameters, and (masked) idx for ``cfg``.

    ``batch`` overrides B (the draws for a smaller batch are a different
    stream, not a prefix of the full one)."""
    B = cfg.B if batch is None else batch
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, cfg.K, cfg.E) if cfg.masked else (B, cfg.h, cfg.w, cfg.E)
    x = rng.standard_normal(shape, dtype=np.float32)
    zs: List[np.ndarray] = [rng.standard_normal(shape, dtype=np.float32)]
    blocks = []
    for _ in range(cfg.nblocks):
        blocks.append({d: draw_dir_params(rng, cfg.E, cfg.N, cfg.R) for d in DIRECTIONS})
    for _ in range(1, cfg.nblocks):
        zs.append(rng.standard_normal(shape, dtype=np.float32))
    idx = None
    if cfg.masked:
        idx = np.stack([rng.permutation(cfg.h * cfg.w)[: cfg.K] for _ in range(B)]).astype(np.int32)
    if cfg.io_dtype == "bf16":
        x = round_to_bf16(x)
        zs = [round_to_bf16(z) for z in zs]
    return {"x": x, "z": zs, "params": blocks, "idx": idx, "cfg": cfg, "B": B}


def zero_D(params: Dict[str, Dict[str, np.ndarray]]) -> Dict[str, Dict[str, np.ndarray]]:
    """Copy of one block's parameters with D_fwd = D_bwd = 0 (the skip-free twin)."""
    out = {}
    for d, p in params.items():
        q = dict(p)
        q["D"] = np.zeros_like(p["D"])
        out[d] = q
    return out


def random_mask(rng: np.random.Generator, B: int, h: int, w: int, K: int) -> np.ndarray:
    """Per image, K distinct flat indices into the h*w grid, unsorted, int32."""
    return np.stack([rng.permutation(h * w)[:K] for _ in range(B)]).astype(np.int32)
