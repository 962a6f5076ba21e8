"""Pins of the CPU oracle against facts fixed outside it (closed forms, worked
examples, brute force, invariants).  No GPU; every check uses only oracle/."""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import velox_oracle as O
from synth import bf16_bits_to_f32, f32_to_bf16_bits, get_config, make_inputs
from tests.parity_rules import check_selection

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(x):
    return math.inf if x == "inf" else float(x)


# ---------------------------------------------------------------- pooling

def test_pool_constant_block_is_exact():
    # a block whose tokens all hold the same vector pools to that vector exactly
    rng = np.random.default_rng(0)
    consts = f32_to_bf16_bits(rng.standard_normal((3, 1, 16)).astype(np.float32))
    x = np.repeat(consts, 64, axis=1).reshape(3 * 64, 16)
    out = O.pool(x, 64)
    assert np.array_equal(out, bf16_bits_to_f32(consts[:, 0, :]).astype(np.float64))


def test_pool_closed_form_ramp():
    # x[t, e] = (t mod blk) + e/2  ->  mean over a block = (blk-1)/2 + e/2 exactly
    blk, d, nb = 8, 6, 5
    t = np.arange(nb * blk) % blk
    x = (t[:, None] + 0.5 * np.arange(d)[None, :]).astype(np.float32)
    x[blk:2 * blk] += 10.0           # block 1 shifted by 10: catches a wrong block stride
    out = O.pool(x, blk)
    expect = (blk - 1) / 2 + 0.5 * np.arange(d)[None, :] + np.zeros((nb, 1))
    expect[1] += 10.0
    assert np.array_equal(out, expect)


# ---------------------------------------------------------------- scores

def test_score_blk1_is_token_logit():
    # blk = 1: the pooled score reduces to the attention logit q.k/sqrt(d); d = 4 -> /2
    q = np.array([[[[1, 2, 3, 4]]]], np.float32)
    k = np.array([[[[1, 1, 1, 1], [-1, 0, 2, 0.5], [0, 0, 0, 0]]]], np.float32)
    s = O.scores(O.pool(q, 1), O.pool(k, 1))
    assert s.shape == (1, 1, 1, 3)
    assert np.array_equal(s[0, 0, 0], [5.0, 3.5, 0.0])


def test_score_constant_blocks_closed_form():
    # Q block constant a, K block j constant b_j -> s_j = a.b_j / sqrt(d) (d = 16 -> /4)
    d, blk = 16, 4
    a = np.zeros(d, np.float32); a[0], a[3] = 2.0, -1.0
    b0 = np.zeros(d, np.float32); b0[0] = 1.0
    b1 = np.zeros(d, np.float32); b1[3] = 1.0
    q = np.tile(a, (blk, 1))[None, None]
    k = np.concatenate([np.tile(b0, (blk, 1)), np.tile(b1, (blk, 1))])[None, None]
    s = O.scores(O.pool(q, blk), O.pool(k, blk))
    assert np.array_equal(s[0, 0, 0], [0.5, -0.25])


# ---------------------------------------------------------------- several batch elements, heads and rows

# B = 2, H = 3, nq = 4 query blocks, nk = 12 KV blocks, blk = 4, d = 16 (so 1/sqrt(d) = 1/4 exactly).
# Every (b, h) pair bh = b*H + h, every query block i and every KV block j carries its own constant, and
# each block adds a zero-mean ramp (-1.5, -0.5, 0.5, 1.5) in another coordinate, so the pooled means, the
# scores and the attention outputs below are closed forms in bh, i and j: a slip in any row, head or
# block stride of the oracle changes them.
_MB, _MH, _MNQ, _MC, _MBLK, _MD = 2, 3, 4, 2, 4, 16
_MT = _MNQ * _MBLK
_MN = (_MC + 1) * _MT
_MNK = _MN // _MBLK
_RAMP = np.arange(_MBLK) - (_MBLK - 1) / 2


def _multi_head_qk():
    q = np.zeros((_MB, _MH, _MT, _MD), np.float32)
    k = np.zeros((_MB, _MH, _MN, _MD), np.float32)
    for b in range(_MB):
        for h in range(_MH):
            bh = b * _MH + h
            for i in range(_MNQ):
                q[b, h, i * _MBLK:(i + 1) * _MBLK, 0] = (bh + 1) * (i + 1)
                q[b, h, i * _MBLK:(i + 1) * _MBLK, 1] = _RAMP
            for j in range(_MNK):
                k[b, h, j * _MBLK:(j + 1) * _MBLK, 0] = j + 1 + 7 * bh
                k[b, h, j * _MBLK:(j + 1) * _MBLK, 2] = _RAMP
    return q, k


def test_pool_and_scores_multi_head_closed_form():
    q, k = _multi_head_qk()
    qbar, kbar = O.pool(q, _MBLK), O.pool(k, _MBLK)
    s = O.scores(qbar, kbar)
    assert s.shape == (_MB, _MH, _MNQ, _MNK)
    for b, h, i, j in itertools.product(range(_MB), range(_MH), range(_MNQ), range(_MNK)):
        bh = b * _MH + h
        e_q = np.zeros(_MD); e_q[0] = (bh + 1) * (i + 1)
        e_k = np.zeros(_MD); e_k[0] = j + 1 + 7 * bh
        assert np.array_equal(qbar[b, h, i], e_q) and np.array_equal(kbar[b, h, j], e_k)
        assert s[b, h, i, j] == (bh + 1) * (i + 1) * (j + 1 + 7 * bh) / 4.0, (b, h, i, j)


def _multi_head_lists():
    # a different list per row (b, h, i): distinct blocks, not sorted, lengths 1..4
    idx = np.full((_MB, _MH, _MNQ, 4), -1, np.int32)
    cnt = np.zeros((_MB, _MH, _MNQ), np.int32)
    for b, h, i in itertools.product(range(_MB), range(_MH), range(_MNQ)):
        bh = b * _MH + h
        n = 1 + (bh + i) % 4
        blocks = [(5 * bh + 3 * i + 7 * c) % _MNK for c in range(n)]
        assert len(set(blocks)) == n
        idx[b, h, i, :n] = blocks
        cnt[b, h, i] = n
    return idx, cnt


def test_attention_multi_head_zero_query_is_mean_of_kept_blocks():
    # Q = 0: every kept key has weight 1, so out = mean over the kept blocks of V's block constant
    # 10*bh + j (the within-block ramp averages to 0) and lse = log(cnt * blk).
    q = np.zeros((_MB, _MH, _MT, _MD), np.float32)
    k = np.random.default_rng(40).standard_normal((_MB, _MH, _MN, _MD)).astype(np.float32)
    v = np.zeros((_MB, _MH, _MN, _MD), np.float32)
    for b, h, j in itertools.product(range(_MB), range(_MH), range(_MNK)):
        v[b, h, j * _MBLK:(j + 1) * _MBLK, 0] = 10 * (b * _MH + h) + j
        v[b, h, j * _MBLK:(j + 1) * _MBLK, 1] = _RAMP
    idx, cnt = _multi_head_lists()
    out, lse = O.attn(q, k, v, idx, cnt, _MBLK)
    for b, h, i in itertools.product(range(_MB), range(_MH), range(_MNQ)):
        kept = idx[b, h, i, :cnt[b, h, i]]
        expect = np.zeros(_MD); expect[0] = np.mean(10 * (b * _MH + h) + kept)
        rows = out[b, h, i * _MBLK:(i + 1) * _MBLK]
        assert np.allclose(rows, expect[None], rtol=0, atol=1e-12), (b, h, i)
        assert np.allclose(lse[b, h, i * _MBLK:(i + 1) * _MBLK], math.log(cnt[b, h, i] * _MBLK), rtol=0, atol=1e-13)
    # the dense brute force over every key of a head: the mean of all its blocks' constants
    dout, dlse = O.dense_attn(q, k, v)
    for b, h in itertools.product(range(_MB), range(_MH)):
        assert np.allclose(dout[b, h, :, 0], 10 * (b * _MH + h) + (_MNK - 1) / 2, rtol=0, atol=1e-12)
        assert np.allclose(dlse[b, h], math.log(_MN), rtol=0, atol=1e-13)


def test_attention_multi_head_block_constant_keys_closed_form():
    # Keys constant over each block (kappa(bh, j) e0) and queries a(bh, t) e0: every key of block j has
    # the logit a*kappa/4, so attention over tokens reduces to a softmax over the kept blocks, each
    # counted blk times: out_0 = sum_j w_j c_j / sum_j w_j with w_j = exp(a kappa_j / 4) and c_j the
    # block constant of V, and lse = log(blk * sum_j exp(a kappa_j / 4)).
    q = np.zeros((_MB, _MH, _MT, _MD), np.float32)
    k = np.zeros((_MB, _MH, _MN, _MD), np.float32)
    v = np.zeros((_MB, _MH, _MN, _MD), np.float32)
    kappa = lambda bh, j: ((j + 2 * bh) % 5 - 2) * 1.5
    a = lambda bh, t: ((t + 3 * bh) % 7 - 3) * 0.75
    for b, h in itertools.product(range(_MB), range(_MH)):
        bh = b * _MH + h
        for t in range(_MT):
            q[b, h, t, 0] = a(bh, t)
        for j in range(_MNK):
            k[b, h, j * _MBLK:(j + 1) * _MBLK, 0] = kappa(bh, j)
            v[b, h, j * _MBLK:(j + 1) * _MBLK, 0] = 10 * bh + j
            v[b, h, j * _MBLK:(j + 1) * _MBLK, 3] = _RAMP
    idx, cnt = _multi_head_lists()
    out, lse = O.attn(q, k, v, idx, cnt, _MBLK)
    for b, h, t in itertools.product(range(_MB), range(_MH), range(_MT)):
        bh, i = b * _MH + h, t // _MBLK
        kept = idx[b, h, i, :cnt[b, h, i]]
        w = np.array([math.exp(a(bh, t) * kappa(bh, j) / 4.0) for j in kept])
        c = np.array([10 * bh + j for j in kept], np.float64)
        expect = np.zeros(_MD); expect[0] = (w * c).sum() / w.sum()
        assert np.allclose(out[b, h, t], expect, rtol=0, atol=1e-12), (b, h, t)
        assert abs(lse[b, h, t] - math.log(_MBLK * w.sum())) <= 1e-12
    # the dense brute force is the same closed form over every block of the head
    dout, dlse = O.dense_attn(q, k, v)
    for b, h, t in itertools.product(range(_MB), range(_MH), range(_MT)):
        bh = b * _MH + h
        w = np.array([math.exp(a(bh, t) * kappa(bh, j) / 4.0) for j in range(_MNK)])
        c = 10.0 * bh + np.arange(_MNK)
        assert abs(dout[b, h, t, 0] - (w * c).sum() / w.sum()) <= 1e-12, (b, h, t)
        assert abs(dlse[b, h, t] - math.log(_MBLK * w.sum())) <= 1e-12


def test_attention_list_contract_invalid_entries_and_empty_rows():
    # entries outside [0, nk) name no block and are skipped; a count above the stride is clamped; a row
    # with no valid block gives out = 0 and lse = -inf (the library's contract for caller-made lists)
    q, k = _multi_head_qk()
    v = np.random.default_rng(41).standard_normal((_MB, _MH, _MN, _MD)).astype(np.float32)
    idx, cnt = _multi_head_lists()
    ref, ref_lse = O.attn(q, k, v, idx, cnt, _MBLK)
    bad = np.full((_MB, _MH, _MNQ, 8), -1, np.int32)
    bad[..., 1:5] = idx
    bad[..., 0] = _MNK          # first entry out of range on the high side
    bad[..., 5] = -7            # and on the low side
    out, lse = O.attn(q, k, v, bad, cnt + 2, _MBLK)
    assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse)
    empty = np.full((_MB, _MH, _MNQ, 2), -1, np.int32)
    out, lse = O.attn(q, k, v, empty, np.full((_MB, _MH, _MNQ), 2, np.int32), _MBLK)
    assert np.all(out == 0) and np.all(lse == -np.inf)
    out, lse = O.attn(q, k, v, idx, np.full((_MB, _MH, _MNQ), 99, np.int32), _MBLK)
    full, full_lse = O.attn(q, k, v, idx, np.full((_MB, _MH, _MNQ), 4, np.int32), _MBLK)
    assert np.array_equal(out, full) and np.array_equal(lse, full_lse)


# ---------------------------------------------------------------- modulation + selection, worked examples

def _one_row(s, overlap, covered, alpha, k, C):
    # blk = T: one block per chunk, so chunk(j) = j and block C is the current chunk
    s = np.asarray(s, np.float64).reshape(1, 1, 1, -1)
    ov = np.asarray(overlap, np.float32).reshape(1, 1, C)
    cov = np.array([[covered]], np.uint8)
    m = O.modulate(s, ov, cov, blk=1, T=1, alpha=alpha)
    idx, cnt, kth = O.select(m, k)
    return m[0, 0, 0], idx[0, 0, 0], int(cnt[0, 0, 0])


@pytest.mark.parametrize("name", ["ex1_modulation_changes_set.json", "ex2_literal_sign.json"])
def test_worked_examples(name):
    g = golden(name)
    for case, cov in (("covered", 1), ("uncovered", 0)):
        m, idx, cnt = _one_row(g["s"], g["overlap"], cov, g["alpha"], g["top_k"], g["past_chunks"])
        assert list(m) == [_num(x) for x in g[case]["m"]], (case, m)
        assert list(idx) == g[case]["kv_idx"] and cnt == g["top_k"], (case, idx)


def test_fp32_decision_example():
    g = golden("ex6_fp32_decision.json")
    C = g["past_chunks"]
    s = np.asarray(g["s"], np.float32).reshape(1, 1, 1, -1)
    ov = np.asarray(g["overlap"], np.float32).reshape(1, 1, C)
    cov = np.ones((1, 1), np.uint8)
    m64 = O.modulate(s.astype(np.float64), ov, cov, 1, 1, g["alpha"])
    m32 = O.modulate(s, ov, cov, 1, 1, g["alpha"], fp32=True)
    assert list(O.select(m64, g["top_k"])[0][0, 0, 0]) == g["fp64"]["kv_idx"]
    assert list(m32[0, 0, 0]) == [_num(x) for x in g["fp32"]["m"]]
    assert list(O.select(m32, g["top_k"])[0][0, 0, 0]) == g["fp32"]["kv_idx"]


def test_zero_alpha_zero_overlap_uncovered_are_native():
    rng = np.random.default_rng(1)
    B, H, nq, C, blk, T = 2, 3, 4, 5, 2, 8
    nk = (C + 1) * T // blk
    s = rng.standard_normal((B, H, nq, nk))
    ov = rng.random((B, nq, C)).astype(np.float32)
    cur = np.arange(nk) * blk // T == C
    native = np.where(cur, np.inf, s)
    cov1 = np.ones((B, nq), np.uint8)
    assert np.array_equal(O.modulate(s, ov, cov1, blk, T, 0.0), native)
    assert np.array_equal(O.modulate(s, np.zeros_like(ov), cov1, blk, T, 3.0), native)
    assert np.array_equal(O.modulate(s, ov, np.zeros((B, nq), np.uint8), blk, T, 3.0), native)
    # covered rows do change where overlap is non-zero
    assert not np.array_equal(O.modulate(s, ov, cov1, blk, T, 3.0), native)
    # the per-(b, query block) overlap row is used: row i of batch b reads overlap[b, i, chunk(j)]
    m = O.modulate(s, ov, cov1, blk, T, 2.0)
    b, h, i, j = 1, 2, 3, 5
    c = j * blk // T
    assert m[b, h, i, j] == s[b, h, i, j] * (1.0 + 2.0 * float(ov[b, i, c]))


def _brute_force_topk(m_row, k):
    """The unique subset S of size k with: j in S, j' not in S => m_j > m_j' or (m_j == m_j' and j < j')."""
    nk = len(m_row)
    keff = min(k, nk)
    found = []
    for S in itertools.combinations(range(nk), keff):
        Sset = set(S)
        ok = all((m_row[a] > m_row[b]) or (m_row[a] == m_row[b] and a < b)
                 for a in Sset for b in range(nk) if b not in Sset)
        if ok:
            found.append(S)
    assert len(found) == 1
    return list(found[0])


def test_select_matches_brute_force_with_ties():
    rng = np.random.default_rng(2)
    vals = np.array([-1.0, -0.5, -0.0, 0.0, 0.5, 1.0, np.inf])
    for trial in range(60):
        nk = int(rng.integers(1, 10))
        k = int(rng.integers(1, 12))
        m = rng.choice(vals, size=nk)
        idx, cnt, kth = O.select(m[None], k)
        keff = min(k, nk)
        expect = _brute_force_topk(list(m), k)
        assert list(idx[0, :keff]) == expect and int(cnt[0]) == keff
        assert np.all(idx[0, keff:] == -1)
        assert kth[0] == min(m[j] for j in expect) or kth[0] == m[sorted(expect, key=lambda j: (-m[j], j))[-1]]


def test_select_keep_all_and_current_only():
    rng = np.random.default_rng(3)
    B, H, nq, C, blk, T = 1, 2, 2, 4, 2, 4
    nk, ncur = (C + 1) * T // blk, T // blk
    s = rng.standard_normal((B, H, nq, nk))
    m = O.modulate(s, rng.random((B, nq, C)).astype(np.float32), np.ones((B, nq), np.uint8), blk, T, 1.0)
    idx, cnt, _ = O.select(m, nk + 3)
    assert np.all(cnt == nk) and np.all(idx[..., :nk] == np.arange(nk)) and np.all(idx[..., nk:] == -1)
    idx, cnt, kth = O.select(m, ncur)
    assert np.all(idx == np.arange(nk - ncur, nk)) and np.all(np.isinf(kth))


def test_raising_overlap_keeps_positive_blocks():
    # for s_j > 0, raising the overlap of chunk(j) never removes j
    rng = np.random.default_rng(4)
    C, blk, T, k = 6, 1, 1, 4
    nk = C + 1
    for _ in range(200):
        s = rng.standard_normal((1, 1, 1, nk))
        ov = rng.random((1, 1, C)).astype(np.float32)
        cov = np.ones((1, 1), np.uint8)
        before = set(O.select(O.modulate(s, ov, cov, blk, T, 1.5), k)[0][0, 0, 0])
        j = int(rng.integers(0, C))
        if s[0, 0, 0, j] <= 0 or j not in before:
            continue
        ov2 = ov.copy()
        ov2[0, 0, j] = min(1.0, ov2[0, 0, j] + 0.5)
        after = set(O.select(O.modulate(s, ov2, cov, blk, T, 1.5), k)[0][0, 0, 0])
        assert j in after


# ---------------------------------------------------------------- sign-safe (probability) modulation

def test_sign_safe_worked_example():
    g = golden("ex7_sign_safe.json")
    C = g["past_chunks"]
    s = np.asarray(g["s"], np.float64).reshape(1, 1, 1, -1)
    ov = np.asarray(g["overlap"], np.float32).reshape(1, 1, C)
    for case, cov in (("covered", 1), ("uncovered", 0)):
        c = np.full((1, 1), cov, np.uint8)
        m = O.modulate(s, ov, c, 1, 1, g["alpha"], mode=1)[0, 0, 0]
        np.testing.assert_allclose(m[:2], [_num(x) for x in g[case]["m"][:2]], rtol=0, atol=1e-15)
        assert np.isinf(m[2])
        m32 = O.modulate(s.astype(np.float32), ov, c, 1, 1, g["alpha"], fp32=True, mode=1)[0, 0, 0]
        assert list(m32) == [_num(x) for x in g[case]["m_fp32"]]
        for mm in (m[None, None, None], m32[None, None, None]):
            assert list(O.select(mm, g["top_k"])[0][0, 0, 0]) == g[case]["kv_idx"]


def _topk_by_value(v, k):
    order = sorted(range(len(v)), key=lambda j: (-v[j], j))
    return sorted(order[:min(k, len(v))])


def test_sign_safe_mode_ranks_by_modulated_softmax_probability():
    """Brute force on the probability form: p_j = softmax(s)_j, importance p_j*(1+alpha*o) on past
    blocks of covered rows, p_j on uncovered rows, current blocks always kept."""
    rng = np.random.default_rng(21)
    B, H, nq, C, blk, T = 2, 2, 3, 5, 2, 4
    nk = (C + 1) * T // blk
    for trial in range(20):
        s = rng.standard_normal((B, H, nq, nk)) * rng.choice([0.3, 2.0, 6.0]) - rng.choice([0.0, 3.0])
        ov = rng.random((B, nq, C)).astype(np.float32)
        cov = (rng.random((B, nq)) > 0.3).astype(np.uint8)
        alpha = float(rng.choice([0.5, 2.0, 7.0]))
        k = int(rng.integers(T // blk, nk + 1))
        idx, cnt, _ = O.select(O.modulate(s, ov, cov, blk, T, alpha, mode=1), k)
        for b, h, i in itertools.product(range(B), range(H), range(nq)):
            row = s[b, h, i]
            p = np.exp(row - row.max())
            p /= p.sum()
            imp = []
            for j in range(nk):
                c = j * blk // T
                if c >= C:
                    imp.append(math.inf)
                elif cov[b, i]:
                    imp.append(p[j] * (1.0 + alpha * float(ov[b, i, c])))
                else:
                    imp.append(p[j])
            assert list(idx[b, h, i, :cnt[b, h, i]]) == _topk_by_value(imp, k)


def test_sign_safe_mode_reduces_to_native_without_modulation():
    rng = np.random.default_rng(22)
    B, H, nq, C, blk, T = 1, 2, 3, 4, 2, 4
    nk = (C + 1) * T // blk
    s = rng.standard_normal((B, H, nq, nk))
    ov = rng.random((B, nq, C)).astype(np.float32)
    native = np.where(np.arange(nk) * blk // T == C, np.inf, s)
    one = np.ones((B, nq), np.uint8)
    assert np.array_equal(O.modulate(s, ov, one, blk, T, 0.0, mode=1), native)
    assert np.array_equal(O.modulate(s, np.zeros_like(ov), one, blk, T, 2.0, mode=1), native)
    assert np.array_equal(O.modulate(s, ov, np.zeros((B, nq), np.uint8), blk, T, 2.0, mode=1), native)


def test_sign_safe_raising_overlap_never_drops_a_block():
    # unlike s*(1+alpha*o), raising chunk(j)'s overlap keeps j for scores of either sign
    rng = np.random.default_rng(23)
    C, blk, T, k = 6, 1, 1, 4
    nk = C + 1
    checked_negative = 0
    for _ in range(300):
        s = rng.standard_normal((1, 1, 1, nk)) - 0.5
        ov = rng.random((1, 1, C)).astype(np.float32)
        cov = np.ones((1, 1), np.uint8)
        before = set(O.select(O.modulate(s, ov, cov, blk, T, 1.5, mode=1), k)[0][0, 0, 0])
        j = int(rng.integers(0, C))
        if j not in before:
            continue
        checked_negative += s[0, 0, 0, j] < 0
        ov2 = ov.copy()
        ov2[0, 0, j] = min(1.0, ov2[0, 0, j] + 0.5)
        after = set(O.select(O.modulate(s, ov2, cov, blk, T, 1.5, mode=1), k)[0][0, 0, 0])
        assert j in after
    assert checked_negative > 10


# ---------------------------------------------------------------- frustum-slice overlap

def _geom(yaws, past, qdep):
    return (np.asarray([yaws], np.float32), np.asarray([past], np.float32).reshape(1, -1, 2),
            np.asarray([qdep], np.float32).reshape(1, -1, 2))


def test_frustum_overlap_closed_forms():
    # same view and same depth interval: every strip fully covered
    o, cov = O.frustum_overlap(*_geom([0.0, 0.0], [[2.0, 9.0]], [[2.0, 9.0]] * 4), 90.0)
    assert np.array_equal(o, np.ones((1, 4, 1))) and cov.all()
    # turned by exactly one field of view: the slices only touch, overlap 0, uncovered
    o, cov = O.frustum_overlap(*_geom([90.0, 0.0], [[2.0, 9.0]], [[2.0, 9.0]] * 2), 90.0)
    assert np.all(o == 0) and not cov.any()
    # turned by half a field of view: the right strip is covered, the left one is not
    o, _ = O.frustum_overlap(*_geom([45.0, 0.0], [[2.0, 9.0]], [[2.0, 9.0]] * 2), 90.0)
    assert list(o[0, :, 0]) == [0.0, 1.0]
    # depth fractions: query [2,4] against [3,10] -> 1/2, [5,6] -> 0, [0,100] -> 1
    o, _ = O.frustum_overlap(*_geom([0.0, 0.0, 0.0, 0.0], [[3.0, 10.0], [5.0, 6.0], [0.0, 100.0]], [[2.0, 4.0]]),
                             90.0)
    assert list(o[0, 0]) == [0.5, 0.0, 1.0]
    # angle wrap: yaw 350 against a current yaw of 10 is 20 degrees to the left: strip [-45,45] vs [-65,25]
    o, _ = O.frustum_overlap(*_geom([350.0, 10.0], [[1.0, 5.0]], [[1.0, 5.0]]), 90.0)
    assert abs(o[0, 0, 0] - 70.0 / 90.0) < 1e-15
    # no past chunk: nothing is covered
    o, cov = O.frustum_overlap(np.zeros((1, 1), np.float32), np.zeros((1, 0, 2), np.float32),
                               np.asarray([[[1.0, 2.0]] * 3], np.float32), 90.0)
    assert o.shape == (1, 3, 0) and not cov.any()


def test_frustum_overlap_is_the_covered_measure_monte_carlo():
    """O is the fraction of the strip x depth box (uniform measure) inside the chunk's
    angular and depth intervals: estimate it by sampling and compare within 5 sigma."""
    rng = np.random.default_rng(31)
    nq, C, fov, n = 5, 6, 90.0, 200000
    yaw = np.concatenate([rng.uniform(-200, 200, C), [rng.uniform(-30, 30)]]).astype(np.float32)
    past = np.sort(rng.uniform(1, 20, (C, 2)), axis=1).astype(np.float32)
    qdep = np.sort(rng.uniform(1, 20, (nq, 2)), axis=1).astype(np.float32)
    o, _ = O.frustum_overlap(yaw[None], past[None], qdep[None], fov)
    for i in range(nq):
        a = -fov / 2 + fov * (i + rng.random(n)) / nq               # angle relative to the current view
        dep = qdep[i, 0] + (qdep[i, 1] - qdep[i, 0]) * rng.random(n)
        for c in range(C):
            diff = (a - (yaw[c] - yaw[C]) + 180.0) % 360.0 - 180.0  # angle relative to chunk c, wrapped
            inside = (np.abs(diff) <= fov / 2) & (dep >= past[c, 0]) & (dep <= past[c, 1])
            est = inside.mean()
            sigma = math.sqrt(max(est * (1 - est), 1.0 / n) / n)
            assert abs(est - o[0, i, c]) <= 5 * sigma + 1e-9, (i, c, est, o[0, i, c])


def test_workload_overlap_equals_oracle_overlap():
    from synth import draw_frustum_geometry, frustum_overlap
    for seed in (3, 4, 5):
        g = draw_frustum_geometry(np.random.default_rng(seed), 32, 48)
        o, cov = O.frustum_overlap(g.yaw[None], g.past_depth[None], g.query_depth[None], g.fov)
        w = frustum_overlap(g)
        assert np.allclose(w, o[0], rtol=0, atol=1e-6)
        assert np.array_equal((w > 0).any(axis=1), cov[0].astype(bool))


# ---------------------------------------------------------------- attention

def test_two_key_closed_form():
    # blk = 1, d = 4: logits 0 and q.k1/2 = 1 -> out = (v0 + e v1)/(1 + e), lse = log(1 + e)
    q = np.array([[[[2, 0, 0, 0]]]], np.float32)
    k = np.array([[[[0, 0, 0, 0], [1, 0, 0, 0]]]], np.float32)
    v = np.array([[[[1, 2, 3, 4], [-1, 0, 5, 8]]]], np.float32)
    e = math.e
    expect = (np.array([1, 2, 3, 4]) + e * np.array([-1, 0, 5, 8])) / (1 + e)
    for out, lse in (O.dense_attn(q, k, v),
                     O.attn(q, k, v, np.array([[[[0, 1]]]], np.int32), np.array([[[2]]], np.int32), 1)):
        assert np.allclose(out[0, 0, 0], expect, rtol=0, atol=1e-14)
        assert abs(lse[0, 0, 0] - math.log(1 + e)) < 1e-14


def test_zero_query_mean_of_kept_values_and_poison():
    g = golden("ex3_zero_query_mask.json")
    blk, T, C, d = g["block"], g["chunk_tokens"], g["past_chunks"], g["head_dim"]
    N = (C + 1) * T
    q = np.zeros((1, 1, T, d), np.float32)
    rng = np.random.default_rng(5)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    v = np.zeros((1, 1, N, d), np.float32)
    for j, val in enumerate(g["v_fill_per_block"]):
        v[0, 0, j * blk:(j + 1) * blk] = val
    nq = T // blk
    idx = np.array(g["kv_idx"], np.int32)[None, None, None].repeat(nq, axis=2)
    cnt = np.full((1, 1, nq), len(g["kv_idx"]), np.int32)
    out, lse = O.attn(q, k, v, idx, cnt, blk)
    assert np.all(out == g["expected_out"])
    assert np.allclose(lse, math.log(len(g["kv_idx"]) * blk), rtol=0, atol=1e-14)
    # poison the skipped block with NaN: nothing changes
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, blk:2 * blk] = np.nan
    v2[0, 0, blk:2 * blk] = np.nan
    out2, lse2 = O.attn(q, k2, v2, idx, cnt, blk)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_keep_all_equals_dense_and_list_order_is_irrelevant():
    cfg = get_config("tiny").with_(chunk_tokens=64, past_chunks=3, block=16, top_k=1000)
    x = make_inputs(cfg)
    r = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    assert np.all(r["kv_cnt"] == cfg.nk)
    out, lse = O.attn(x.q, x.k, x.v, r["kv_idx"], r["kv_cnt"], cfg.block)
    dout, dlse = O.dense_attn(x.q, x.k, x.v)
    assert np.max(np.abs(out - dout)) <= 1e-12 and np.max(np.abs(lse - dlse)) <= 1e-12
    perm = r["kv_idx"][..., :cfg.nk][..., ::-1].copy()
    pout, _ = O.attn(x.q, x.k, x.v, perm, r["kv_cnt"], cfg.block)
    assert np.max(np.abs(pout - out)) <= 1e-12


def test_single_block_zero_keys_gives_block_mean_of_values():
    d, blk, T = 8, 4, 4
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 1, T, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, 3 * T, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, 3 * T, d)).astype(np.float32)
    k[0, 0, 2 * blk:3 * blk] = 0.0
    out, _ = O.attn(q, k, v, np.array([[[[2]]]], np.int32), np.array([[[1]]], np.int32), blk)
    expect = v[0, 0, 2 * blk:3 * blk].astype(np.float64).sum(0) / blk
    assert np.allclose(out[0, 0], expect[None, :], rtol=0, atol=1e-14)


def test_current_only_attends_within_current_chunk():
    cfg = get_config("tiny").with_(chunk_tokens=32, past_chunks=2, block=16, top_k=2)
    x = make_inputs(cfg)
    r = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    assert np.all(r["kv_idx"] == np.arange(cfg.nk - cfg.ncur, cfg.nk))
    out, _ = O.attn(x.q, x.k, x.v, r["kv_idx"], r["kv_cnt"], cfg.block)
    T = cfg.chunk_tokens
    dout, _ = O.dense_attn(x.q, x.k[:, :, -T:], x.v[:, :, -T:])
    assert np.max(np.abs(out - dout)) <= 1e-12


def test_bf16_inputs_are_widened_exactly():
    # the oracle reads bf16 bit patterns exactly: same result as the widened float32 values
    cfg = get_config("small").with_(heads=1, chunk_tokens=128, past_chunks=2, top_k=4)
    x = make_inputs(cfg)
    a = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    b = O.route(x.as_f32("q"), x.as_f32("k"), x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    assert np.array_equal(a["s"], b["s"]) and np.array_equal(a["kv_idx"], b["kv_idx"])


# ---------------------------------------------------------------- the comparison rule itself

def test_gap_rule_accepts_oracle_and_rejects_planted_errors():
    cfg = get_config("small").with_(heads=2, chunk_tokens=256, past_chunks=6, top_k=10)
    x = make_inputs(cfg)
    r = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    cur_first = cfg.nk - cfg.ncur
    st = check_selection(r["kv_idx"], r["kv_cnt"], r["m"], r["kth"], r["kv_idx"], cfg.k_eff, cur_first)
    assert st["rows_differing"] == 0
    # plant: replace the kept block with the lowest score by the best dropped block -> must fail
    bad = r["kv_idx"].copy()
    m0 = r["m"][0, 0, 0]
    kept = [j for j in bad[0, 0, 0, :cfg.k_eff] if j < cur_first]
    worst = min(kept, key=lambda j: m0[j])
    dropped = [j for j in range(cur_first) if j not in set(bad[0, 0, 0])]
    best = max(dropped, key=lambda j: m0[j])
    if abs(m0[best] - r["kth"][0, 0, 0]) > 1e-4 or abs(m0[worst] - r["kth"][0, 0, 0]) > 1e-4:
        row = sorted(set(bad[0, 0, 0, :cfg.k_eff]) - {worst} | {best})
        bad[0, 0, 0, :cfg.k_eff] = row
        with pytest.raises(AssertionError):
            check_selection(bad, r["kv_cnt"], r["m"], r["kth"], r["kv_idx"], cfg.k_eff, cur_first)
    # plant: drop a current block -> must fail
    bad2 = r["kv_idx"].copy()
    bad2[0, 0, 0, cfg.k_eff - 1] = bad2[0, 0, 0, 0] - 1 if bad2[0, 0, 0, 0] > 0 else 0
    with pytest.raises(AssertionError):
        check_selection(bad2, r["kv_cnt"], r["m"], r["kth"], r["kv_idx"], cfg.k_eff, cur_first)
