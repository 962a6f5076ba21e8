"""Row selection (velox_select) on score patterns that stress the radix select:
all scores equal, two values, only negative values, magnitudes over sixty
decades, and tie groups straddling the k-th position, at list lengths that
take each register layout of the selection kernel (4, 8, 16 and 32 keys per
thread).  The decision is taken in float32 on both sides, so the lists must
be identical to the oracle's (ties to the lower block index)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import geometry_routed_block_velox_amd as velox
from oracle import velox_oracle as O
from tests.gpu_helpers import say, to_dev

pytestmark = pytest.mark.gpu

# (nq, past chunks, block, top_k): nk = (C+1)*nq = 400, 1568, 3136, 8192
SHAPES = [(16, 24, 128, 64), (32, 48, 128, 256), (32, 97, 128, 256), (64, 127, 64, 300)]
CASES = ["all-equal", "two-values", "negative", "wide-range", "tie-at-kth"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    velox.lib()


def scores(case, shape, rng):
    if case == "all-equal":
        return np.full(shape, 0.5, np.float32)
    if case == "two-values":
        return rng.choice(np.array([1.0, 2.0], np.float32), size=shape)
    if case == "negative":
        return -np.abs(rng.standard_normal(shape)).astype(np.float32) - np.float32(1e-3)
    if case == "wide-range":
        mag = np.float32(10.0) ** rng.uniform(-30, 30, shape).astype(np.float32)
        return (mag * rng.choice(np.array([-1.0, 1.0], np.float32), size=shape)).astype(np.float32)
    # tie-at-kth: a few distinct levels, so the kept set ends inside a large tie group
    return rng.integers(0, 6, shape).astype(np.float32) * np.float32(0.125)


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("nq,C,blk,top_k", SHAPES, ids=[f"nk{(s[1] + 1) * s[0]}" for s in SHAPES])
def test_select_patterns_bit_exact(nq, C, blk, top_k, case):
    rng = np.random.default_rng(17)
    B, H = 1, 2
    nk = (C + 1) * nq
    s = scores(case, (B, H, nq, nk), rng)
    ov = rng.random((B, nq, C)).astype(np.float32)
    cov = (rng.random((B, nq)) > 0.3).astype(np.uint8)
    alpha = 2.0
    say(f"{case}: nq {nq} nk {nk} top-k {top_k}")
    kv_idx, kv_cnt = velox.select(to_dev(s), to_dev(ov), to_dev(cov), blk, top_k, alpha)
    m = O.modulate(s, ov, cov, blk, nq * blk, alpha, fp32=True)
    ref_idx, ref_cnt, _ = O.select(m, top_k)
    torch.cuda.synchronize()
    assert np.array_equal(kv_cnt.cpu().numpy(), ref_cnt)
    assert np.array_equal(kv_idx.cpu().numpy(), ref_idx)
