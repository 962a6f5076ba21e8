"""GPU invariants and edge cases of the routed attention layer, each checked
against the oracle or against a fact that holds at any size."""
import json
import math
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import geometry_routed_block_velox_amd as velox
from oracle import velox_oracle as O
from synth import get_config, make_inputs
from tests.gpu_helpers import cached_inputs, dev_inputs, out_to_f64, say, to_dev
from tests.parity_rules import (BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, F32_MEAN_ABS, bf16_fast_lse_slack,
                                check_close, check_lse, check_selection)

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    velox.lib()


def tol(cfg):
    return (BF16_MAX_ABS, BF16_MEAN_ABS) if cfg.dtype == "bf16" else (F32_MAX_ABS, F32_MEAN_ABS)


def run_layer(x, top_k=None, alpha=None, covered=None):
    cfg = x.cfg
    d = dev_inputs(x)
    cov = d["covered"] if covered is None else to_dev(covered)
    kv_idx, kv_cnt = velox.route(d["q"], d["k"], d["overlap"], cov, cfg.block, top_k or cfg.top_k,
                                 cfg.alpha if alpha is None else alpha)
    out = velox.sparse_attn(d["q"], d["k"], d["v"], kv_idx, kv_cnt, cfg.block)
    torch.cuda.synchronize()
    return kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), out


# shapes spanning several tiles with ragged tails (nk not a multiple of the
# 32-block scoring group), all four (d, blk) builds, both dtypes and B > 1
EDGE = [
    ("bf16-d128-b128-B2", dict(batch=2, heads=3, head_dim=128, chunk_tokens=384, past_chunks=6, block=128,
                               top_k=9, dtype="bf16", seeds=(21, 22))),
    ("bf16-d64-b128", dict(heads=2, head_dim=64, chunk_tokens=256, past_chunks=9, block=128, top_k=7)),
    ("bf16-d128-b64", dict(heads=2, head_dim=128, chunk_tokens=192, past_chunks=5, block=64, top_k=8)),
    ("bf16-d64-b64-C0", dict(heads=2, head_dim=64, chunk_tokens=256, past_chunks=0, block=64, top_k=4)),
    ("f32-d128-b128", dict(heads=2, head_dim=128, chunk_tokens=256, past_chunks=4, block=128, top_k=5,
                           dtype="f32", mean_offset_std=0.0)),
    ("f32-d64-b64-C1", dict(heads=1, head_dim=64, chunk_tokens=128, past_chunks=1, block=64, top_k=3,
                            dtype="f32", mean_offset_std=0.0)),
]


@pytest.mark.parametrize("label,kw", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shapes_full_parity(label, kw):
    base = get_config("small")
    kw = dict(kw)
    kw.setdefault("seeds", (7,) * kw.get("batch", 1))
    cfg = base.with_(name=label, **kw)
    x = make_inputs(cfg)
    say(f"edge {label}: {cfg}")
    gi, gc, out = run_layer(x)
    r = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    check_selection(gi, gc, r["m"], r["kth"], r["kv_idx"], cfg.k_eff, cfg.nk - cfg.ncur)
    ref, _ = O.attn(x.q, x.k, x.v, gi, gc, cfg.block)  # lists are valid; the oracle attends the same ones
    check_close(out_to_f64(out), ref, *tol(cfg))


def test_keep_all_equals_dense():
    cfg = get_config("small").with_(heads=2, chunk_tokens=256, past_chunks=5, top_k=10_000)
    x = make_inputs(cfg)
    gi, gc, out = run_layer(x, top_k=cfg.top_k)
    assert np.all(gc == cfg.nk) and np.all(gi[..., :cfg.nk] == np.arange(cfg.nk)) and np.all(gi[..., cfg.nk:] == -1)
    dense, _ = O.dense_attn(x.q, x.k, x.v)
    check_close(out_to_f64(out), dense, *tol(cfg))


def test_current_only_lists():
    cfg = get_config("small").with_(heads=2, chunk_tokens=256, past_chunks=5)
    x = make_inputs(cfg)
    gi, gc, out = run_layer(x, top_k=cfg.ncur)
    assert np.all(gi == np.arange(cfg.nk - cfg.ncur, cfg.nk))
    T = cfg.chunk_tokens
    ref, _ = O.dense_attn(x.q, x.k[:, :, -T:], x.v[:, :, -T:])
    check_close(out_to_f64(out), ref, *tol(cfg))


def test_zero_alpha_and_uncovered_give_native_routing():
    x = cached_inputs("small")
    cfg = x.cfg
    g0, _, o0 = run_layer(x, alpha=0.0)
    g1, _, o1 = run_layer(x, covered=np.zeros_like(x.covered))
    assert np.array_equal(g0, g1)
    assert torch.equal(o0, o1)
    r = O.route(x.q, x.k, x.overlap, np.zeros_like(x.covered), cfg.block, cfg.top_k, 0.0)
    check_selection(g0, np.full(g0.shape[:3], cfg.k_eff, np.int32), r["m"], r["kth"], r["kv_idx"], cfg.k_eff,
                    cfg.nk - cfg.ncur)


def test_poisoned_skipped_blocks_do_not_change_output():
    x = cached_inputs("small")
    cfg = x.cfg
    gi, gc, out = run_layer(x)
    k2, v2 = x.k.copy(), x.v.copy()
    kept = np.zeros((cfg.batch, cfg.heads, cfg.nk), bool)
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            kept[b, h, np.unique(gi[b, h, :, :cfg.k_eff])] = True
    nan_bf16 = np.uint16(0x7FC0)
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            for j in np.nonzero(~kept[b, h])[0]:
                k2[b, h, j * cfg.block:(j + 1) * cfg.block] = nan_bf16
                v2[b, h, j * cfg.block:(j + 1) * cfg.block] = nan_bf16
    assert (~kept).any()
    d = dev_inputs(x)
    out2 = velox.sparse_attn(d["q"], to_dev(k2, True), to_dev(v2, True), to_dev(gi), to_dev(gc), cfg.block)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


def test_deterministic_reruns():
    x = cached_inputs("small")
    a = run_layer(x)
    b = run_layer(x)
    assert np.array_equal(a[0], b[0]) and torch.equal(a[2], b[2])


def test_zero_query_mean_of_kept_values_is_exact():
    g = json.load(open(os.path.join(GOLDEN, "ex3_zero_query_mask.json")))
    blk, C = 64, 2
    T = 64
    N = (C + 1) * T
    d = 64
    q = np.zeros((1, 1, T, d), np.float32)
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    v = np.zeros((1, 1, N, d), np.float32)
    for j, val in enumerate(g["v_fill_per_block"]):
        v[0, 0, j * blk:(j + 1) * blk] = val
    idx = np.array(g["kv_idx"], np.int32).reshape(1, 1, 1, -1)
    cnt = np.array([[[2]]], np.int32)
    for bf in (True, False):
        out, lse = velox.sparse_attn(to_dev(q, bf), to_dev(k, bf), to_dev(v, bf), to_dev(idx), to_dev(cnt), blk,
                                     return_lse=True)
        torch.cuda.synchronize()
        assert torch.all(out.float() == g["expected_out"]), bf
        assert abs(float(lse.max()) - math.log(2 * blk)) < 1e-5 and abs(float(lse.min()) - math.log(2 * blk)) < 1e-5


def test_invalid_list_entries_are_skipped():
    cfg = get_config("small").with_(heads=1, chunk_tokens=128, past_chunks=3)
    x = make_inputs(cfg)
    d = dev_inputs(x)
    nq, nk = cfg.nq, cfg.nk
    good = np.array([1, 5, 7], np.int32)
    lists = np.full((1, 1, nq, 6), -1, np.int32)
    lists[..., 0] = 1
    lists[..., 1] = -3
    lists[..., 2] = 5
    lists[..., 3] = nk + 100
    lists[..., 4] = 7
    cnt = np.full((1, 1, nq), 5, np.int32)
    cnt[0, 0, 1] = 99  # clamped to the row stride
    out = velox.sparse_attn(d["q"], d["k"], d["v"], to_dev(lists), to_dev(cnt), cfg.block)
    ref_lists = np.broadcast_to(good, (1, 1, nq, 3)).copy()
    ref, _ = O.attn(x.q, x.k, x.v, ref_lists, np.full((1, 1, nq), 3, np.int32), cfg.block)
    check_close(out_to_f64(out), ref, *tol(cfg))
    # an empty row gives zeros and lse = -inf
    cnt0 = np.zeros((1, 1, nq), np.int32)
    out0, lse0 = velox.sparse_attn(d["q"], d["k"], d["v"], to_dev(lists), to_dev(cnt0), cfg.block, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(out0 == 0) and torch.all(torch.isinf(lse0)) and torch.all(lse0 < 0)


def test_unsorted_and_repeated_lists():
    cfg = get_config("small").with_(heads=2, chunk_tokens=128, past_chunks=4)
    x = make_inputs(cfg)
    d = dev_inputs(x)
    rng = np.random.default_rng(5)
    lists = np.stack([rng.permutation(cfg.nk)[:4] for _ in range(cfg.rows)]).astype(np.int32)
    lists[:, 3] = lists[:, 0]  # a repeated block counts twice
    lists = lists.reshape(1, cfg.heads, cfg.nq, 4)
    cnt = np.full((1, cfg.heads, cfg.nq), 4, np.int32)
    out = velox.sparse_attn(d["q"], d["k"], d["v"], to_dev(lists), to_dev(cnt), cfg.block)
    ref, _ = O.attn(x.q, x.k, x.v, lists, cnt, cfg.block)
    check_close(out_to_f64(out), ref, *tol(cfg))


@pytest.mark.parametrize("case", ["dominant-block", "two-close-blocks", "float32-overflow"])
@pytest.mark.parametrize("base,extra", [("small", False), ("mid", False), ("mid", True), ("d128-blk64", False),
                                        ("d64-blk128", True)])
def test_logits_far_above_first_block_recompute_row(case, base, extra):
    """Large logits take every path of the kernel and must still match:
    two-close-blocks stays in the fast pass (base-2 logits of about 46);
    dominant-block and float32-overflow leave it (probability sums past 2^56)
    for the general pass, whose first block is then more than 40 log2-units
    below the maximum, so it reruns the row at the true maximum.  All four
    (d, blk) kernels, lists of 4 and 5 blocks (both exits of the
    two-blocks-per-turn loop)."""
    if base == "small":
        cfg = get_config("small").with_(heads=2, chunk_tokens=128, past_chunks=4)
    elif base == "d128-blk64":
        cfg = get_config("mid").with_(heads=2, chunk_tokens=256, past_chunks=4, block=64)
    elif base == "d64-blk128":
        cfg = get_config("small").with_(heads=2, chunk_tokens=256, past_chunks=4, block=128)
    else:
        cfg = get_config("mid").with_(heads=2, chunk_tokens=256, past_chunks=4)
    x = make_inputs(cfg)
    from synth import f32_to_bf16_bits
    q = np.ones((1, cfg.heads, cfg.chunk_tokens, cfg.head_dim), np.float32)
    k = x.as_f32("k").copy()
    k[:, :, 0:cfg.block] *= 0.1                      # first listed block: logits near 0
    blk = cfg.block
    if case == "dominant-block":
        k[:, :, 3 * blk:4 * blk] = 6.0               # logit 48 with q = 1, d = 64
        lists = [0, 2, 3, 5]
    elif case == "float32-overflow":
        # logit 160: exp2((160 - ~0) * log2 e) overflows float32, so this passes
        # only if the row is recomputed at its true maximum
        k[:, :, 3 * blk:4 * blk] = 20.0
        lists = [0, 1, 3, 6]
    else:
        k[:, :, 2 * blk:3 * blk] = 4.0               # logit 32
        k[:, :, 5 * blk:6 * blk] = 3.875             # logit 31, both blocks matter
        lists = [0, 2, 5, 7]
    if extra:
        lists = lists + [cfg.nk - 1]
    say(f"{base} d{cfg.head_dim} blk{cfg.block}: {case}, list {lists}")
    qb, kb = f32_to_bf16_bits(q), f32_to_bf16_bits(k)
    idx = np.broadcast_to(np.array(lists, np.int32), (1, cfg.heads, cfg.nq, len(lists))).copy()
    cnt = np.full((1, cfg.heads, cfg.nq), len(lists), np.int32)
    out, lse = velox.sparse_attn(to_dev(qb, True), to_dev(kb, True), to_dev(x.v, True), to_dev(idx), to_dev(cnt),
                                 cfg.block, return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = O.attn(qb, kb, x.v, idx, cnt, cfg.block)
    check_close(out_to_f64(out), ref, *tol(cfg))
    toks = np.arange(cfg.batch * cfg.heads * cfg.chunk_tokens)
    check_lse(lse.cpu().numpy().astype(np.float64), ref_lse, bf16_fast_lse_slack(qb, kb, idx, cnt, cfg.block, toks))
