"""The largest shapes the library accepts (VELOX_MAX_QUERY_BLOCKS = 64 query blocks per
chunk, VELOX_MAX_KV_BLOCKS = 8192 KV blocks), against the oracle.

* d = 64 / blk = 64: T = 4096 (64 query blocks), 127 past chunks (nk = 8192): routing
  with top-k 1000 under the gap rule, attention over the oracle's lists (every row,
  8 queries per block), and keep-all (lists of 8192 blocks) against the oracle.
* d = 128 / blk = 128 at 64 query blocks (T = 8192) with 31 past chunks (nk = 2048):
  routing and attention (every row, 8 queries per block).
Same bars as the workload parity tests.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import geometry_routed_block_velox_amd as velox
from oracle import velox_oracle as O
from synth import make_inputs
from synth.configs import Config
from tests.gpu_helpers import dev_inputs, every_row_tokens, out_to_f64, say, to_dev
from tests.parity_rules import (BF16_MAX_ABS, BF16_MEAN_ABS, bf16_fast_lse_slack, check_close, check_lse,
                                check_selection)

pytestmark = pytest.mark.gpu

LIMIT64 = Config("limits-d64", 1, 1, 64, 4096, 127, 64, 1000, 2.0, "bf16", "beta25", 0.20, 0.5, (11,))
LIMIT128 = Config("limits-d128", 1, 1, 128, 8192, 31, 128, 300, 2.0, "bf16", "beta25", 0.20, 0.5, (12,))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    velox.lib()


@pytest.mark.parametrize("cfg", [LIMIT64, LIMIT128], ids=lambda c: c.name)
def test_route_and_attention_at_the_limits(cfg):
    assert cfg.nq == 64 and cfg.nk in (8192, 2048)
    x = make_inputs(cfg)
    d = dev_inputs(x)
    say(f"{cfg.name}: nq {cfg.nq} nk {cfg.nk} top-k {cfg.top_k}: velox_route")
    kv_idx, kv_cnt = velox.route(d["q"], d["k"], d["overlap"], d["covered"], cfg.block, cfg.top_k, cfg.alpha)
    torch.cuda.synchronize()
    r = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    st = check_selection(kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), r["m"], r["kth"], r["kv_idx"], cfg.k_eff,
                         cfg.nk - cfg.ncur)
    say(f"{cfg.name}: selection {st}")
    toks = every_row_tokens(cfg, seed=5)
    out = velox.sparse_attn(d["q"], d["k"], d["v"], to_dev(r["kv_idx"]), to_dev(r["kv_cnt"]), cfg.block)
    torch.cuda.synchronize()
    ref, _ = O.attn(x.q, x.k, x.v, r["kv_idx"], r["kv_cnt"], cfg.block, tokens=toks)
    mx, mn = check_close(out_to_f64(out).reshape(-1, cfg.head_dim)[toks], ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    say(f"{cfg.name}: attention max {mx:.3g} mean {mn:.3g}")


def test_keep_all_with_8192_blocks():
    cfg = LIMIT64
    x = make_inputs(cfg)
    d = dev_inputs(x)
    B, H, nq, nk = cfg.batch, cfg.heads, cfg.nq, cfg.nk
    full = np.broadcast_to(np.arange(nk, dtype=np.int32), (B, H, nq, nk)).copy()
    cnt = np.full((B, H, nq), nk, np.int32)
    say(f"{cfg.name}: keep-all, lists of {nk} blocks")
    out, lse = velox.sparse_attn(d["q"], d["k"], d["v"], to_dev(full), to_dev(cnt), cfg.block, return_lse=True)
    torch.cuda.synchronize()
    toks = np.array([0, 63, 64 * 17 + 5, cfg.chunk_tokens - 1], np.int64)
    ref, ref_lse = O.attn(x.q, x.k, x.v, full, cnt, cfg.block, tokens=toks)
    mx, mn = check_close(out_to_f64(out).reshape(-1, cfg.head_dim)[toks], ref, BF16_MAX_ABS, BF16_MEAN_ABS)
    slack = bf16_fast_lse_slack(x.q, x.k, full, cnt, cfg.block, toks)
    lmx, smx = check_lse(lse.cpu().numpy().astype(np.float64).reshape(-1)[toks], ref_lse, slack)
    say(f"keep-all: max {mx:.3g} mean {mn:.3g}, lse max excess over slack {lmx:.3g} (slack <= {smx:.3g})")
