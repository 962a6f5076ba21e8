"""Split-KV attention (velox_sparse_attn_split) against the oracle.

Each row's list is cut into segments attended by separate workgroups and
merged through their LSEs.  The merged result must meet the same bars as the
unsplit kernel: max-abs 2e-2 / mean-abs 2e-3 (bf16) or 1e-4 / 1e-5 (float32)
against the fp64 oracle on the same lists; LSE within 1e-4 (float32), and for
bf16 within 1e-3 plus the per-token slack of the fast pass's scaled Q (the
LSE rule in parity_rules).
Cases: split counts from 1 to more segments than listed blocks (empty
segments), automatic split count, lists with invalid entries and empty rows.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import geometry_routed_block_velox_amd as velox
from oracle import velox_oracle as O
from tests.gpu_helpers import cached_inputs, dev_inputs, every_row_tokens, out_to_f64, say, to_dev
from tests.parity_rules import (BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, F32_MEAN_ABS, bf16_fast_lse_slack,
                                check_close, check_lse)

pytestmark = pytest.mark.gpu


def tol(cfg):
    return (BF16_MAX_ABS, BF16_MEAN_ABS) if cfg.dtype == "bf16" else (F32_MAX_ABS, F32_MEAN_ABS)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    velox.lib()


def compare(x, kv_idx, kv_cnt, splits, toks=None, ref_idx=None, ref_cnt=None):
    """GPU split attention on (kv_idx, kv_cnt) against the oracle on (ref_idx, ref_cnt),
    by default the same lists, over the flat query tokens `toks` (default all)."""
    cfg = x.cfg
    d = dev_inputs(x)
    say(f"{cfg.name}: velox_sparse_attn_split, splits={splits}")
    out, lse = velox.sparse_attn(d["q"], d["k"], d["v"], to_dev(kv_idx), to_dev(kv_cnt), cfg.block,
                                 return_lse=True, splits=splits)
    torch.cuda.synchronize()
    out = out_to_f64(out).reshape(-1, cfg.head_dim)
    lse = lse.cpu().numpy().astype(np.float64).reshape(-1)
    if toks is None:
        toks = np.arange(cfg.batch * cfg.heads * cfg.chunk_tokens)
    ref_idx = kv_idx if ref_idx is None else ref_idx
    ref_cnt = kv_cnt if ref_cnt is None else ref_cnt
    ref, ref_lse = O.attn(x.q, x.k, x.v, ref_idx, ref_cnt, cfg.block, tokens=toks)
    mx, mn = check_close(out[toks], ref, *tol(cfg))
    if cfg.dtype == "bf16":
        lmx, _ = check_lse(lse[toks], ref_lse, bf16_fast_lse_slack(x.q, x.k, kv_idx, kv_cnt, cfg.block, toks))
    else:
        lmx, _ = check_close(lse[toks], ref_lse, 1e-4, 1e-3, "lse")
    say(f"{cfg.name}: splits={splits}: out max {mx:.3g} mean {mn:.3g}; lse max excess {lmx:.3g}")
    return out, lse


@pytest.mark.parametrize("name,splits", [("tiny", 1), ("tiny", 5), ("tiny", 16), ("tiny", "auto"),
                                         ("small", 1), ("small", 3), ("small", 8), ("small", "auto"),
                                         ("small", 64), ("mid", 4), ("mid", "auto")])
def test_split_matches_oracle(name, splits):
    x = cached_inputs(name)
    cfg = x.cfg
    r = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    toks = None
    if cfg.rows > 64:
        toks = every_row_tokens(cfg, seed=3)
    compare(x, r["kv_idx"], r["kv_cnt"], splits, toks)


def test_split_headline_every_row():
    x = cached_inputs("headline")
    cfg = x.cfg
    r = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    compare(x, r["kv_idx"], r["kv_cnt"], 2, every_row_tokens(cfg, seed=4))


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_split_with_invalid_entries_and_empty_rows(name):
    """Out-of-range entries are skipped, a row with no valid entry gives zeros and lse = -inf,
    a row whose only valid block is its last entry leaves the other segments empty."""
    x = cached_inputs(name)
    cfg = x.cfg
    r = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    idx = r["kv_idx"].copy().reshape(cfg.rows, -1)
    cnt = r["kv_cnt"].copy().reshape(-1)
    rng = np.random.default_rng(9)
    for rr in rng.choice(np.arange(1, cfg.rows), size=min(3, cfg.rows - 1), replace=False):
        pos = rng.choice(int(cnt[rr]), size=2, replace=False)
        idx[rr, pos[0]] = -1
        idx[rr, pos[1]] = cfg.nk + 5
    idx[0, :-1] = -7                      # only the last entry of row 0 is valid
    cnt[0] = idx.shape[1]
    empty = cfg.rows - 1
    cnt[empty] = 0
    # the oracle gets each row's valid entries only, in list order
    ref_idx = np.full_like(idx, -1)
    ref_cnt = np.zeros_like(cnt)
    for rr in range(cfg.rows):
        valid = [j for j in idx[rr, :cnt[rr]] if 0 <= j < cfg.nk]
        ref_idx[rr, :len(valid)] = valid
        ref_cnt[rr] = len(valid)
    toks = np.array([t for t in range(cfg.batch * cfg.heads * cfg.chunk_tokens) if t // cfg.block != empty])
    shape = r["kv_idx"].shape
    out, lse = compare(x, idx.reshape(shape), cnt.reshape(shape[:3]), 4, toks, ref_idx.reshape(shape),
                       ref_cnt.reshape(shape[:3]))
    et = np.arange(empty * cfg.block, (empty + 1) * cfg.block)
    assert np.all(out[et] == 0) and np.all(np.isneginf(lse[et]))


def test_split_agrees_with_unsplit_kernel():
    x = cached_inputs("small")
    cfg = x.cfg
    d = dev_inputs(x)
    kv_idx, kv_cnt = velox.route(d["q"], d["k"], d["overlap"], d["covered"], cfg.block, cfg.top_k, cfg.alpha)
    a = velox.sparse_attn(d["q"], d["k"], d["v"], kv_idx, kv_cnt, cfg.block)
    b = velox.sparse_attn(d["q"], d["k"], d["v"], kv_idx, kv_cnt, cfg.block, splits="auto")
    torch.cuda.synchronize()
    diff = (a.float() - b.float()).abs()
    say(f"split vs unsplit: max {float(diff.max()):.3g} mean {float(diff.mean()):.3g}")
    assert float(diff.max()) <= BF16_MAX_ABS and float(diff.mean()) <= BF16_MEAN_ABS
