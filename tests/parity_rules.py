"""Comparison rules between the GPU path and the oracle (test infrastructure).

Selection rule: the oracle ranks blocks by the fp64 modulated score m; let
m_k be the k_eff-th largest m of a row.  Every block whose m lies more than
GAP away from m_k must have the same membership on both sides; blocks within
GAP of m_k are exempt (their order can flip under fp32 rounding of the pooled
sums), but the GPU list must still be valid: exactly k_eff distinct,
ascending, in-range ids containing every current-chunk block, padded with -1.

Attention rule (bf16 inputs, fp32 accumulation): max |out - ref| <= 2e-2 and
mean |out - ref| <= 2e-3 against the oracle fed the same block lists; float32
inputs: 1e-4 / 1e-5.

LSE rule (bf16): |lse - ref| <= 1e-3 + slack_t per token (mean of the excess
over slack_t <= 1e-3).  slack_t is derived from the kernel's arithmetic: its
fast pass multiplies Q by c = log2(e)/sqrt(d) and rounds the product to bf16,
which moves the base-2 score of key j by r_t . k_j with r_t = bf16(c q_t) -
c q_t; the row's base-2 log-sum-exp moves by at most the largest such shift,
so slack_t = ln 2 * max_j |r_t . k_j| over the token's listed keys.
"""
from __future__ import annotations

import math

import numpy as np

GAP = 1e-4
BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
F32_MAX_ABS, F32_MEAN_ABS = 1e-4, 1e-5


def check_list_valid(kv_idx: np.ndarray, kv_cnt: np.ndarray, nk: int, k_eff: int, cur_first: int):
    """Structural validity of GPU lists: count, range, strict ascent, padding, current blocks kept."""
    kv_idx = kv_idx.reshape(-1, kv_idx.shape[-1])
    kv_cnt = kv_cnt.reshape(-1)
    assert np.all(kv_cnt == k_eff), f"kv_cnt != {k_eff}: {np.unique(kv_cnt)}"
    head = kv_idx[:, :k_eff]
    assert head.min() >= 0 and head.max() < nk, "block id out of range"
    if k_eff > 1:
        assert np.all(np.diff(head, axis=1) > 0), "list not strictly ascending"
    assert np.all(kv_idx[:, k_eff:] == -1), "padding must be -1"
    ncur = nk - cur_first
    if ncur > 0:
        assert np.all(head[:, k_eff - ncur:] == np.arange(cur_first, nk)[None, :]), \
            "current-chunk blocks must all be kept"


def check_selection(gpu_idx: np.ndarray, gpu_cnt: np.ndarray, m: np.ndarray, kth: np.ndarray,
                    oracle_idx: np.ndarray, k_eff: int, cur_first: int, gap: float = GAP) -> dict:
    """Gap rule; returns {'rows': n, 'rows_differing': n_in_band_swaps, 'exempt_blocks': n}."""
    nk = m.shape[-1]
    m = m.reshape(-1, nk)
    kth = kth.reshape(-1)
    gpu_idx = gpu_idx.reshape(m.shape[0], -1)
    oracle_idx = oracle_idx.reshape(m.shape[0], -1)
    check_list_valid(gpu_idx, gpu_cnt, nk, k_eff, cur_first)
    rows = m.shape[0]
    gpu_mask = np.zeros((rows, nk), bool)
    ora_mask = np.zeros((rows, nk), bool)
    r = np.repeat(np.arange(rows), k_eff)
    gpu_mask[r, gpu_idx[:, :k_eff].reshape(-1)] = True
    ora_mask[r, oracle_idx[:, :k_eff].reshape(-1)] = True
    inf_rows = np.isinf(kth) & (kth > 0)
    if inf_rows.any():
        assert np.array_equal(gpu_mask[inf_rows], ora_mask[inf_rows]), "k = ncur rows must match exactly"
    with np.errstate(invalid="ignore"):
        far = np.abs(m - kth[:, None]) > gap
    bad = far & (gpu_mask != ora_mask)
    if bad.any():
        rr, jj = np.nonzero(bad)
        msg = [f"row {a} block {b}: m={m[a, b]!r} kth={kth[a]!r} gpu={gpu_mask[a, b]} oracle={ora_mask[a, b]}"
               for a, b in list(zip(rr, jj))[:8]]
        raise AssertionError(f"{bad.sum()} out-of-band membership mismatches:\n" + "\n".join(msg))
    differing = int(np.any(gpu_mask != ora_mask, axis=1).sum())
    return dict(rows=rows, rows_differing=differing, exempt_blocks=int((~far).sum()))


def check_close(out: np.ndarray, ref: np.ndarray, max_abs: float, mean_abs: float, what: str = "out"):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    assert np.all(np.isfinite(out)), f"{what}: non-finite values"
    err = np.abs(out - ref)
    mx, mn = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    assert mx <= max_abs and mn <= mean_abs, f"{what}: max-abs {mx:.3g} (<= {max_abs}), mean-abs {mn:.3g} (<= {mean_abs})"
    return mx, mn


def bf16_fast_lse_slack(q_bits: np.ndarray, k_bits: np.ndarray, kv_idx: np.ndarray, kv_cnt: np.ndarray, blk: int,
                        tokens: np.ndarray) -> np.ndarray:
    """Per-token LSE slack of the bf16 fast pass (see the module docstring).

    q_bits [B,H,T,d], k_bits [B,H,N,d]: bf16 bit patterns; kv_idx [B,H,nq,top_k], kv_cnt [B,H,nq]; tokens:
    flat indices into B*H*T.  Invalid list entries are skipped.  The products r_t . k_j are taken in
    float32 (relative error ~1e-6, far inside the 1e-3 base tolerance)."""
    from synth.generate import bf16_bits_to_f32, f32_to_bf16_bits
    B, H, T, d = q_bits.shape
    N = k_bits.shape[2]
    nq, nk = T // blk, N // blk
    c32 = np.float32(1.4426950408889634) / np.sqrt(np.float32(d))  # the kernel's float32 scale
    c = math.log2(math.e) / math.sqrt(d)
    tokens = np.asarray(tokens).reshape(-1)
    out = np.zeros(tokens.size)
    q = bf16_bits_to_f32(q_bits).reshape(-1, d)
    heads = tokens // T
    for bh in np.unique(heads):
        sel = np.nonzero(heads == bh)[0]
        b, h = divmod(int(bh), H)
        qt = q[tokens[sel]]
        scaled = bf16_bits_to_f32(f32_to_bf16_bits(qt * c32)).astype(np.float64)
        resid = (scaled - qt.astype(np.float64) * c).astype(np.float32)
        shift = np.abs(resid @ bf16_bits_to_f32(k_bits[b, h]).T).reshape(sel.size, nk, blk).max(axis=2)
        for n, t in enumerate(tokens[sel]):
            i = (int(t) % T) // blk
            lst = kv_idx[b, h, i, :max(int(kv_cnt[b, h, i]), 0)]
            lst = lst[(lst >= 0) & (lst < nk)]
            if lst.size:
                out[sel[n]] = math.log(2.0) * float(shift[n, lst].max())
    return out


def check_lse(lse: np.ndarray, ref: np.ndarray, slack: np.ndarray, max_abs: float = 1e-3, mean_abs: float = 1e-3):
    """LSE rule: |lse - ref| - slack <= max_abs everywhere, and its positive part averages <= mean_abs."""
    lse = np.asarray(lse, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    slack = np.asarray(slack, np.float64).reshape(-1)
    assert lse.shape == ref.shape == slack.shape, (lse.shape, ref.shape, slack.shape)
    same_inf = np.isinf(lse) & np.isinf(ref) & (np.sign(lse) == np.sign(ref))
    assert np.all(np.isfinite(lse) | same_inf), "lse: unexpected non-finite values"
    excess = np.where(same_inf, 0.0, np.abs(np.where(same_inf, 0.0, lse - ref)) - slack)
    mx = float(excess.max()) if excess.size else 0.0
    mn = float(np.maximum(excess, 0.0).mean()) if excess.size else 0.0
    assert mx <= max_abs and mn <= mean_abs, \
        f"lse: max excess over slack {mx:.3g} (<= {max_abs}), mean {mn:.3g} (<= {mean_abs})"
    return mx, float(slack.max()) if slack.size else 0.0
