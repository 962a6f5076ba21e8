"""Seeded synthetic inputs for the routed-attention layer.

Every tensor is drawn in float32 from numpy's PCG64 and, for bf16 workloads,
rounded once to bfloat16 (round to nearest even).  The GPU path and the oracle
then consume the same bits, so the generator itself is not part of any parity
contract.

Draw recipe, per batch element ``b`` with seed ``seeds[b]``:

1. Overlap matrix ``O[b]`` of shape ``[nq, C]`` from a generator seeded with
   ``seeds[b]``: uniform U[0,1], Beta(2,5), or the synthetic camera-frustum
   construction below.
2. Coverage flags: a frustum workload marks a query block uncovered when it
   overlaps no past chunk; then ``round(uncovered_frac * nq)`` query blocks
   chosen without replacement are forced uncovered.
3. Per head ``h`` (generator seeded with ``[seeds[b], h + 1]`` so heads can be
   drawn in parallel): mean offsets ``mu_Q[d]``, ``mu_K[C+1, d]``,
   ``mu_V[C+1, d]`` ~ N(0, sigma^2) (skipped when sigma = 0), then the tokens of
   Q ``[T, d]``, K ``[N, d]``, V ``[N, d]`` ~ N(0, 1) plus the offset of their
   chunk (Q belongs to the current chunk).

Synthetic frustum overlap (the article's per-chunk camera frustum slices with
a depth interval, sns.style "Velox" article, Deep analysis; the article gives
no geometry, so this construction is this project's stand-in): yaw follows a
random walk with 5 degree steps, every past chunk sees a 90 degree horizontal
field of view around its yaw and a depth interval from two U[1,20] m draws;
query block ``i`` is the ``i``-th of ``nq`` equal angular strips of the current
view with its own depth interval; the overlap is the fraction of the strip's
angle covered by the chunk's view times the fraction of the strip's depth
interval covered by the chunk's depth interval.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import Config

FOV_DEG = 90.0
YAW_STEP_STD_DEG = 5.0
DEPTH_RANGE_M = (1.0, 20.0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Inputs:
    cfg: Config
    q: np.ndarray        # [B,H,T,d]  float32, or uint16 bf16 bits
    k: np.ndarray        # [B,H,N,d]
    v: np.ndarray        # [B,H,N,d]
    overlap: np.ndarray  # [B,nq,C] float32
    covered: np.ndarray  # [B,nq] uint8
    geometry: Optional[list] = None  # per batch element FrustumGeometry (frustum workloads)

    def as_f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


def _wrap_deg(x: np.ndarray) -> np.ndarray:
    """Wrap angles to (-180, 180]."""
    y = np.mod(x + 180.0, 360.0) - 180.0
    return np.where(y == -180.0, 180.0, y)


def _interval_overlap(a0, a1, b0, b1):
    return np.clip(np.minimum(a1, b1) - np.maximum(a0, b0), 0.0, None)


@dataclass
class FrustumGeometry:
    """Synthetic camera geometry of one rollout (float32, as handed to a device)."""
    yaw: np.ndarray          # [C+1] degrees; yaw[C] is the current view
    past_depth: np.ndarray   # [C, 2] (near, far) metres of each past chunk's slice
    query_depth: np.ndarray  # [nq, 2] (near, far) metres of each query block's strip
    fov: float = FOV_DEG     # horizontal field of view in degrees


def draw_frustum_geometry(rng: np.random.Generator, nq: int, C: int) -> FrustumGeometry:
    steps = rng.normal(0.0, YAW_STEP_STD_DEG, size=C) if C > 0 else np.zeros(0)
    yaw = np.concatenate([[0.0], np.cumsum(steps)])          # yaw[c], c = 0..C; yaw[C] = current view
    past_depth = np.sort(rng.uniform(*DEPTH_RANGE_M, size=(C, 2)), axis=1)
    q_depth = np.sort(rng.uniform(*DEPTH_RANGE_M, size=(nq, 2)), axis=1)
    return FrustumGeometry(yaw.astype(np.float32), past_depth.astype(np.float32), q_depth.astype(np.float32))


def frustum_overlap(g: FrustumGeometry) -> np.ndarray:
    """Overlap [nq, C] between the current view's angular strips and past chunks' frusta
    (the workload's overlap input, evaluated in float64 from the float32 geometry)."""
    yaw = g.yaw.astype(np.float64)
    past_depth = g.past_depth.astype(np.float64)
    q_depth = g.query_depth.astype(np.float64)
    C, nq = past_depth.shape[0], q_depth.shape[0]
    half = g.fov / 2.0
    # strips of the current view, in angles relative to the current yaw
    edges = -half + g.fov * np.arange(nq + 1) / nq
    s0, s1 = edges[:-1, None], edges[1:, None]                  # [nq,1]
    rel = _wrap_deg(yaw[:C] - yaw[C])[None, :]                  # [1,C]
    ang = _interval_overlap(s0, s1, rel - half, rel + half) / (s1 - s0)
    d0, d1 = q_depth[:, 0:1], q_depth[:, 1:2]
    dep = _interval_overlap(d0, d1, past_depth[None, :, 0], past_depth[None, :, 1])
    dep = dep / np.maximum(d1 - d0, 1e-12)
    return (ang * dep).astype(np.float32)


def _draw_overlap(cfg: Config, rng: np.random.Generator):
    nq, C = cfg.nq, cfg.past_chunks
    if cfg.overlap == "uniform":
        o = rng.random((nq, C), dtype=np.float32)
        cov = np.ones(nq, dtype=np.uint8)
    elif cfg.overlap == "beta25":
        o = rng.beta(2.0, 5.0, size=(nq, C)).astype(np.float32)
        cov = np.ones(nq, dtype=np.uint8)
    elif cfg.overlap == "frustum":
        geom = draw_frustum_geometry(rng, nq, C)
        o = frustum_overlap(geom)
        cov = (o > 0).any(axis=1).astype(np.uint8) if C > 0 else np.zeros(nq, np.uint8)
    else:
        raise ValueError(f"unknown overlap kind {cfg.overlap!r}")
    n_unc = int(round(cfg.uncovered_frac * nq))
    if n_unc > 0:
        cov[rng.choice(nq, n_unc, replace=False)] = 0
    return o, cov, (geom if cfg.overlap == "frustum" else None)


def _draw_head(cfg: Config, seed: int, h: int):
    rng = np.random.Generator(np.random.PCG64([seed, h + 1]))
    T, d, C, N = cfg.chunk_tokens, cfg.head_dim, cfg.past_chunks, cfg.kv_tokens
    sig = cfg.mean_offset_std
    if sig > 0:
        mu_q = rng.normal(0.0, sig, size=d).astype(np.float32)
        mu_k = rng.normal(0.0, sig, size=(C + 1, d)).astype(np.float32)
        mu_v = rng.normal(0.0, sig, size=(C + 1, d)).astype(np.float32)
    q = rng.standard_normal((T, d), dtype=np.float32)
    k = rng.standard_normal((C + 1, T, d), dtype=np.float32)
    v = rng.standard_normal((C + 1, T, d), dtype=np.float32)
    if sig > 0:
        q += mu_q
        k += mu_k[:, None, :]
        v += mu_v[:, None, :]
    k = k.reshape(N, d)
    v = v.reshape(N, d)
    if cfg.dtype == "bf16":
        return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    return q, k, v


def make_inputs(cfg: Config, seeds: Optional[tuple] = None, threads: Optional[int] = None) -> Inputs:
    """Draw the inputs of one layer call for ``cfg`` (seeds default to the config's)."""
    seeds = tuple(seeds if seeds is not None else cfg.seeds)
    if len(seeds) != cfg.batch:
        raise ValueError("need one seed per batch element")
    B, H, T, N, d = cfg.batch, cfg.heads, cfg.chunk_tokens, cfg.kv_tokens, cfg.head_dim
    et = np.uint16 if cfg.dtype == "bf16" else np.float32
    q = np.empty((B, H, T, d), et)
    k = np.empty((B, H, N, d), et)
    v = np.empty((B, H, N, d), et)
    overlap = np.empty((B, cfg.nq, cfg.past_chunks), np.float32)
    covered = np.empty((B, cfg.nq), np.uint8)
    geoms = [None] * B
    for b, seed in enumerate(seeds):
        overlap[b], covered[b], geoms[b] = _draw_overlap(cfg, np.random.Generator(np.random.PCG64(seed)))

    def fill(job):
        b, h = job
        q[b, h], k[b, h], v[b, h] = _draw_head(cfg, seeds[b], h)

    jobs = [(b, h) for b in range(B) for h in range(H)]
    nthreads = threads or min(16, len(os.sched_getaffinity(0)), len(jobs))
    if nthreads <= 1:
        for j in jobs:
            fill(j)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(fill, jobs))
    return Inputs(cfg, q, k, v, overlap, covered, geoms if cfg.overlap == "frustum" else None)
