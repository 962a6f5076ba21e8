"""GPU path vs the CPU oracle on the five workloads (called through the C ABI).

* Scores: the GPU's float32 pooled importance against the fp64 oracle.
* Selection: the gap rule (membership must match wherever the oracle's
  modulated score is more than 1e-4 from the row's k-th score; lists must be
  valid everywhere).
* Selection decision alone, in float32 on both sides: bit-exact.
* Attention: GPU kernel and oracle fed the same (oracle) block lists,
  max-abs 2e-2 / mean-abs 2e-3 for bf16, 1e-4 / 1e-5 for float32.
* End to end: the GPU's routing, then the GPU's attention on its own lists
  against the oracle's attention on those same lists.
Full sizes compare every row at 8 queries per block (the first and last query
of each 32-query MFMA tile); small sizes compare everything.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import geometry_routed_block_velox_amd as velox
from oracle import velox_oracle as O
from synth import get_config, make_inputs
from tests.gpu_helpers import cached_inputs, dev_inputs, every_row_tokens, out_to_f64, say, to_dev
from tests.parity_rules import (BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, F32_MEAN_ABS, bf16_fast_lse_slack,
                                check_close, check_lse, check_selection)

pytestmark = pytest.mark.gpu

ALL = ["tiny", "small", "mid", "headline", "stress"]
SCORE_ATOL, SCORE_RTOL = 2e-5, 1e-5


def tol(cfg):
    return (BF16_MAX_ABS, BF16_MEAN_ABS) if cfg.dtype == "bf16" else (F32_MAX_ABS, F32_MEAN_ABS)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    velox.lib()


@pytest.mark.parametrize("name", ALL)
def test_route_matches_oracle(name):
    x = cached_inputs(name)
    cfg = x.cfg
    d = dev_inputs(x)
    say(f"{name}: velox_route")
    kv_idx, kv_cnt, scores = velox.route(d["q"], d["k"], d["overlap"], d["covered"], cfg.block, cfg.top_k,
                                         cfg.alpha, return_scores=True)
    torch.cuda.synchronize()
    say(f"{name}: oracle route")
    r = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    s_gpu = scores.cpu().numpy().astype(np.float64)
    err = np.abs(s_gpu - r["s"])
    bound = SCORE_ATOL + SCORE_RTOL * np.abs(r["s"])
    say(f"{name}: score max err {err.max():.3g}, max err/bound {np.max(err / bound):.3g}")
    assert np.all(err <= bound), f"scores: max err {err.max():.3g}"
    st = check_selection(kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), r["m"], r["kth"], r["kv_idx"], cfg.k_eff,
                         cfg.nk - cfg.ncur)
    say(f"{name}: selection {st}")


@pytest.mark.parametrize("name", ALL)
def test_select_decision_is_bit_exact(name):
    """Same float32 scores on both sides, decision in float32: identical lists."""
    cfg = get_config(name)
    rng = np.random.default_rng(11)
    B, H, nq, nk = cfg.batch, cfg.heads, cfg.nq, cfg.nk
    s = rng.standard_normal((B, H, nq, nk)).astype(np.float32)
    # plant exact ties, signed zeros and repeated values
    s[..., ::7] = 0.25
    s[..., 3::11] = -0.0
    s[..., 5::11] = 0.0
    s[..., 1::13] = np.round(s[..., 1::13], 1)
    x = cached_inputs(name) if name in ("tiny", "small") else None
    ov = x.overlap if x is not None else rng.random((B, nq, cfg.past_chunks)).astype(np.float32)
    cov = x.covered if x is not None else (rng.random((B, nq)) > 0.3).astype(np.uint8)
    say(f"{name}: velox_select")
    kv_idx, kv_cnt = velox.select(to_dev(s), to_dev(ov), to_dev(cov), cfg.block, cfg.top_k, cfg.alpha)
    m = O.modulate(s, ov, cov, cfg.block, cfg.chunk_tokens, cfg.alpha, fp32=True)
    ref_idx, ref_cnt, _ = O.select(m, cfg.top_k)
    assert np.array_equal(kv_idx.cpu().numpy(), ref_idx)
    assert np.array_equal(kv_cnt.cpu().numpy(), ref_cnt)


@pytest.mark.parametrize("name", ALL)
def test_attention_matches_oracle_same_lists(name):
    x = cached_inputs(name)
    cfg = x.cfg
    d = dev_inputs(x)
    r = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    say(f"{name}: velox_sparse_attn on oracle lists")
    out, lse = velox.sparse_attn(d["q"], d["k"], d["v"], to_dev(r["kv_idx"]), to_dev(r["kv_cnt"]), cfg.block,
                                 return_lse=True)
    torch.cuda.synchronize()
    out = out_to_f64(out).reshape(-1, cfg.head_dim)
    lse = lse.cpu().numpy().astype(np.float64).reshape(-1)
    if cfg.rows <= 64:
        toks = np.arange(cfg.batch * cfg.heads * cfg.chunk_tokens)
    else:
        toks = every_row_tokens(cfg)
    say(f"{name}: oracle attention on {toks.size} tokens ({cfg.rows} rows)")
    ref, ref_lse = O.attn(x.q, x.k, x.v, r["kv_idx"], r["kv_cnt"], cfg.block, tokens=toks)
    mx, mn = check_close(out[toks], ref, *tol(cfg))
    if cfg.dtype == "bf16":
        slack = bf16_fast_lse_slack(x.q, x.k, r["kv_idx"], r["kv_cnt"], cfg.block, toks)
        lmx, smx = check_lse(lse[toks], ref_lse, slack)
        say(f"{name}: out max {mx:.3g} mean {mn:.3g}; lse max excess over slack {lmx:.3g} (slack <= {smx:.3g})")
    else:
        lmx, _ = check_close(lse[toks], ref_lse, 1e-4, 1e-3, "lse")
        say(f"{name}: out max {mx:.3g} mean {mn:.3g}; lse max {lmx:.3g}")


@pytest.mark.parametrize("name", ALL)
def test_end_to_end_layer(name):
    """velox_route then velox_sparse_attn on the GPU.  The lists pass the gap rule
    against the oracle's routing, and the attention matches the oracle's
    attention computed on the GPU's own lists (every row)."""
    x = cached_inputs(name)
    cfg = x.cfg
    d = dev_inputs(x)
    say(f"{name}: velox_route + velox_sparse_attn")
    kv_idx, kv_cnt = velox.route(d["q"], d["k"], d["overlap"], d["covered"], cfg.block, cfg.top_k, cfg.alpha)
    out = velox.sparse_attn(d["q"], d["k"], d["v"], kv_idx, kv_cnt, cfg.block)
    torch.cuda.synchronize()
    r = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    gi, gc = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    st = check_selection(gi, gc, r["m"], r["kth"], r["kv_idx"], cfg.k_eff, cfg.nk - cfg.ncur)
    if cfg.rows <= 64:
        toks = np.arange(cfg.batch * cfg.heads * cfg.chunk_tokens)
    else:
        toks = every_row_tokens(cfg, seed=1)
    say(f"{name}: selection {st}; oracle attention on the GPU's lists, {toks.size} tokens")
    ref, _ = O.attn(x.q, x.k, x.v, gi, gc, cfg.block, tokens=toks)
    mx, mn = check_close(out_to_f64(out).reshape(-1, cfg.head_dim)[toks], ref, *tol(cfg))
    say(f"{name}: end-to-end out max {mx:.3g} mean {mn:.3g}")


@pytest.mark.parametrize("name", ALL)
def test_route_sign_safe_mode_matches_oracle(name):
    """Sign-safe modulation (s + log1p(alpha*o)) against the oracle's fp64 mode 1: gap rule."""
    x = cached_inputs(name)
    cfg = x.cfg
    d = dev_inputs(x)
    say(f"{name}: velox_route, log-probability modulation")
    kv_idx, kv_cnt = velox.route(d["q"], d["k"], d["overlap"], d["covered"], cfg.block, cfg.top_k, cfg.alpha,
                                 modulation=velox.MOD_LOG_PROB)
    lit_idx, _ = velox.route(d["q"], d["k"], d["overlap"], d["covered"], cfg.block, cfg.top_k, cfg.alpha)
    torch.cuda.synchronize()
    r = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha, mode=1)
    st = check_selection(kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), r["m"], r["kth"], r["kv_idx"], cfg.k_eff,
                         cfg.nk - cfg.ncur)
    changed = int((kv_idx != lit_idx).any(dim=-1).sum())
    say(f"{name}: selection {st}; rows whose list differs from the literal mode: {changed} of {cfg.rows}")


@pytest.mark.parametrize("name", ["tiny", "small", "headline"])
def test_select_sign_safe_decision_is_bit_exact(name):
    cfg = get_config(name)
    rng = np.random.default_rng(12)
    B, H, nq, nk = cfg.batch, cfg.heads, cfg.nq, cfg.nk
    s = (rng.standard_normal((B, H, nq, nk)) - 0.5).astype(np.float32)
    s[..., ::7] = -0.25
    s[..., 3::11] = -0.0
    ov = rng.random((B, nq, cfg.past_chunks)).astype(np.float32)
    ov[:, :, ::3] = 0.0
    cov = (rng.random((B, nq)) > 0.3).astype(np.uint8)
    say(f"{name}: velox_select, log-probability modulation")
    kv_idx, kv_cnt = velox.select(to_dev(s), to_dev(ov), to_dev(cov), cfg.block, cfg.top_k, cfg.alpha,
                                  modulation=velox.MOD_LOG_PROB)
    m = O.modulate(s, ov, cov, cfg.block, cfg.chunk_tokens, cfg.alpha, fp32=True, mode=1)
    ref_idx, ref_cnt, _ = O.select(m, cfg.top_k)
    assert np.array_equal(kv_idx.cpu().numpy(), ref_idx) and np.array_equal(kv_cnt.cpu().numpy(), ref_cnt)
