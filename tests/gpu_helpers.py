"""Shared helpers for the GPU tests: device upload of synthetic inputs and the
query tokens that full-size checks compare."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

from synth import Inputs, make_inputs


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, bf16: bool = False) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if bf16:
        t = t.view(torch.int16).view(torch.bfloat16) if a.dtype == np.uint16 else t.to(torch.bfloat16)
    return t.cuda()


def dev_inputs(x: Inputs):
    bf = x.cfg.dtype == "bf16"
    return dict(q=to_dev(x.q, bf), k=to_dev(x.k, bf), v=to_dev(x.v, bf), overlap=to_dev(x.overlap),
                covered=to_dev(x.covered))


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


@functools.lru_cache(maxsize=2)
def cached_inputs(name: str):
    from synth import get_config
    cfg = get_config(name)
    say(f"generating inputs for {name}: B{cfg.batch} H{cfg.heads} d{cfg.head_dim} T{cfg.chunk_tokens} "
        f"C{cfg.past_chunks} blk{cfg.block} k{cfg.top_k} seeds {cfg.seeds}")
    return make_inputs(cfg)


def every_row_tokens(cfg, per_row: int = 8, seed: int = 0):
    """Flat token indices covering every row: in each query block the first and
    last query of every 32-query MFMA tile (t = 32g and 32g + 31, which includes
    the block's first and last token and both halves of each 64-query wave
    group), topped up with random queries to `per_row` per block."""
    rng = np.random.default_rng(seed)
    blk = cfg.block
    fixed = np.array(sorted({32 * g + e for g in range(blk // 32) for e in (0, 31)}), np.int64)
    rest = np.setdiff1d(np.arange(blk), fixed)
    toks = []
    for r in range(cfg.rows):
        bh, i = divmod(r, cfg.nq)
        base = bh * cfg.chunk_tokens + i * blk
        extra = rng.choice(rest, size=max(0, per_row - fixed.size), replace=False)
        toks.append(base + np.union1d(fixed, extra))
    return np.concatenate(toks).astype(np.int64)
