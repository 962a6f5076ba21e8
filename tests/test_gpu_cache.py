"""Incremental pooled-key cache (velox_pool_keys, velox_route_cached) on the GPU.

* Pooled keys against the fp64 oracle's block means.
* Routing from the cache is bit-identical to velox_route (same pooled keys,
  same score arithmetic), on every workload, with the cache filled chunk by
  chunk into a buffer with room for later chunks.
* Rows the contract says are not read (the current chunk's, when no scores are
  returned) are poisoned with NaN and must not change the result.
* The cached route also meets the oracle's gap rule directly.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import geometry_routed_block_velox_amd as velox
from oracle import velox_oracle as O
from tests.gpu_helpers import cached_inputs, dev_inputs, say
from tests.parity_rules import check_selection

pytestmark = pytest.mark.gpu

ALL = ["tiny", "small", "mid", "headline", "stress"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    velox.lib()


def fill_cache_by_chunk(k, cfg, spare_chunks=2, upto_chunk=None):
    """Pool chunk after chunk into a cache with room for `spare_chunks` more; rows past
    the pooled chunks are NaN."""
    B, H, N, d = k.shape
    nq = cfg.nq
    upto = cfg.past_chunks if upto_chunk is None else upto_chunk
    cap = (cfg.past_chunks + 1 + spare_chunks) * nq
    kbar = torch.full((B, H, cap, d), float("nan"), dtype=torch.float32, device=k.device)
    for c in range(upto):
        velox.pool_keys(k, cfg.chunk_tokens, cfg.block, c * nq, nq, kbar=kbar)
    return kbar


@pytest.mark.parametrize("name", ["tiny", "small", "mid"])
def test_pool_keys_matches_oracle(name):
    x = cached_inputs(name)
    cfg = x.cfg
    d = dev_inputs(x)
    say(f"{name}: velox_pool_keys over all {cfg.nk} blocks")
    kbar = velox.pool_keys(d["k"], cfg.chunk_tokens, cfg.block, 0, cfg.nk).cpu().numpy().astype(np.float64)
    ref = O.pool(x.k, cfg.block)
    err = np.abs(kbar - ref)
    bound = 2e-6 + 2e-6 * np.abs(ref)
    say(f"{name}: pooled-key max err {err.max():.3g}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("name", ALL)
def test_route_cached_is_bit_identical_to_route(name):
    x = cached_inputs(name)
    cfg = x.cfg
    d = dev_inputs(x)
    say(f"{name}: cache filled chunk by chunk, current chunk left as NaN")
    kbar = fill_cache_by_chunk(d["k"], cfg)
    ref_idx, ref_cnt, ref_s = velox.route(d["q"], d["k"], d["overlap"], d["covered"], cfg.block, cfg.top_k,
                                          cfg.alpha, return_scores=True)
    say(f"{name}: velox_route_cached without scores")
    idx, cnt = velox.route_cached(d["q"], kbar, cfg.past_chunks, d["overlap"], d["covered"], cfg.block, cfg.top_k,
                                  cfg.alpha)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx) and torch.equal(cnt, ref_cnt)
    say(f"{name}: current chunk pooled, velox_route_cached with scores")
    velox.pool_keys(d["k"], cfg.chunk_tokens, cfg.block, cfg.past_chunks * cfg.nq, cfg.nq, kbar=kbar)
    idx2, cnt2, s2 = velox.route_cached(d["q"], kbar, cfg.past_chunks, d["overlap"], d["covered"], cfg.block,
                                        cfg.top_k, cfg.alpha, return_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(idx2, ref_idx) and torch.equal(cnt2, ref_cnt)
    assert torch.equal(s2.view(torch.int32), ref_s.view(torch.int32)), "scores differ bitwise"


@pytest.mark.parametrize("name", ["small", "mid"])
def test_route_cached_matches_oracle(name):
    x = cached_inputs(name)
    cfg = x.cfg
    d = dev_inputs(x)
    kbar = fill_cache_by_chunk(d["k"], cfg, spare_chunks=0)
    idx, cnt = velox.route_cached(d["q"], kbar, cfg.past_chunks, d["overlap"], d["covered"], cfg.block, cfg.top_k,
                                  cfg.alpha)
    torch.cuda.synchronize()
    r = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    st = check_selection(idx.cpu().numpy(), cnt.cpu().numpy(), r["m"], r["kth"], r["kv_idx"], cfg.k_eff,
                         cfg.nk - cfg.ncur)
    say(f"{name}: cached selection {st}")


def test_route_cached_without_history():
    """C = 0: nothing is read from the cache unless scores are requested."""
    x = cached_inputs("small")
    cfg = x.cfg.with_(past_chunks=0, top_k=x.cfg.nq)
    T = cfg.chunk_tokens
    d = dev_inputs(x)
    q, k = d["q"], d["k"][:, :, -T:].contiguous()
    kbar = torch.full((cfg.batch, cfg.heads, 1, cfg.head_dim), float("nan"), device=q.device)
    idx, cnt = velox.route_cached(q, kbar, 0, None, d["covered"], cfg.block, cfg.top_k, cfg.alpha)
    ref_idx, ref_cnt = velox.route(q, k, None, d["covered"], cfg.block, cfg.top_k, cfg.alpha)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx) and torch.equal(cnt, ref_cnt)
    assert torch.equal(idx[..., :cfg.nq].cpu(), torch.arange(cfg.nq, dtype=torch.int32).expand_as(idx.cpu()))


def test_cache_rejects_short_cache():
    x = cached_inputs("small")
    cfg = x.cfg
    d = dev_inputs(x)
    kbar = torch.zeros((cfg.batch, cfg.heads, cfg.past_chunks * cfg.nq - 1, cfg.head_dim), device=d["q"].device)
    with pytest.raises(velox.VeloxError):
        velox.route_cached(d["q"], kbar, cfg.past_chunks, d["overlap"], d["covered"], cfg.block, cfg.top_k, cfg.alpha)
    with pytest.raises(velox.VeloxError):
        velox.pool_keys(d["k"], cfg.chunk_tokens, cfg.block, cfg.nk - 2, 3)


# query-block counts that leave the scoring's 16-row tiles partly empty (24 -> two
# tiles, 40 -> four), for both head sizes
ODD_TILES = [
    ("nq24-d64-b64", "small", dict(heads=2, chunk_tokens=1536, past_chunks=3, block=64, top_k=36)),
    ("nq40-d128-b128", "mid", dict(heads=1, chunk_tokens=5120, past_chunks=2, block=128, top_k=56)),
]


@pytest.mark.parametrize("label,base,kw", ODD_TILES, ids=[t[0] for t in ODD_TILES])
def test_partial_query_tiles(label, base, kw):
    """velox_route against the oracle's gap rule, and velox_route_cached bit-identical to it
    (lists and returned scores), where the last query tile is only partly filled."""
    from synth import get_config, make_inputs
    cfg = get_config(base).with_(name=label, **kw)
    assert cfg.nq % 16 != 0
    x = make_inputs(cfg)
    d = dev_inputs(x)
    say(f"{label}: nq {cfg.nq} nk {cfg.nk}: velox_route")
    ref_idx, ref_cnt, ref_s = velox.route(d["q"], d["k"], d["overlap"], d["covered"], cfg.block, cfg.top_k,
                                          cfg.alpha, return_scores=True)
    torch.cuda.synchronize()
    r = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    st = check_selection(ref_idx.cpu().numpy(), ref_cnt.cpu().numpy(), r["m"], r["kth"], r["kv_idx"], cfg.k_eff,
                         cfg.nk - cfg.ncur)
    say(f"{label}: selection {st}")
    say(f"{label}: velox_route_cached with scores")
    kbar = fill_cache_by_chunk(d["k"], cfg, spare_chunks=1, upto_chunk=cfg.past_chunks + 1)
    idx, cnt, s = velox.route_cached(d["q"], kbar, cfg.past_chunks, d["overlap"], d["covered"], cfg.block,
                                     cfg.top_k, cfg.alpha, return_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx) and torch.equal(cnt, ref_cnt)
    assert torch.equal(s.view(torch.int32), ref_s.view(torch.int32)), "scores differ bitwise"
