"""Shared helpers for the GPU tests: device upload of synthetic inputs and
sampling of rows/tokens for full-size checks."""
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


def sample_tokens(cfg, n_rows: int, per_row: int, seed: int = 0):
    """Flat token indices (b*H + h)*T + t over a spread of rows, always including
    the first and last row and the first and last token of a block."""
    rng = np.random.default_rng(seed)
    rows = cfg.rows
    pick = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, size=min(n_rows, rows), replace=False)]))
    toks = []
    for r in pick:
        bh, i = divmod(int(r), cfg.nq)
        base = bh * cfg.chunk_tokens + i * cfg.block
        inner = rng.choice(cfg.block, size=min(per_row, cfg.block), replace=False)
        for t in np.unique(np.concatenate([[0, cfg.block - 1], inner])):
            toks.append(base + int(t))
    return np.array(sorted(toks), np.int64), pick
