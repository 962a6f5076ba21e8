"""velox_route_noalloc (routing with the library's per-GPU scratch array as its
workspace) against velox_route on the same inputs: kv_idx, kv_cnt and the
raw scores must be identical (the same kernels run).  Two calls in a row, the
second on a smaller problem, then the largest workload, and a problem whose
score matrix does not fit the scratch array (rejected before any device work
unless the caller takes the scores)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import geometry_routed_block_velox_amd as velox
from synth import make_inputs
from synth.configs import get_config
from tests.gpu_helpers import dev_inputs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    velox.lib()


def outputs(cfg, device="cuda"):
    shape = (cfg.batch, cfg.heads, cfg.nq)
    return (torch.full(shape + (cfg.top_k,), -5, dtype=torch.int32, device=device),
            torch.full(shape, -5, dtype=torch.int32, device=device))


def check_same(cfg, d, with_scores):
    kv_idx, kv_cnt, s_ref = velox.route(d["q"], d["k"], d["overlap"], d["covered"], cfg.block, cfg.top_k, cfg.alpha,
                                        return_scores=True)
    out = outputs(cfg)
    scores = torch.full((cfg.batch, cfg.heads, cfg.nq, cfg.nk), float("nan"), device="cuda") if with_scores else None
    say(f"{cfg.name}: velox_route_noalloc (scores {'returned' if with_scores else 'in scratch'})")
    velox.route_noalloc(d["q"], d["k"], d["overlap"], d["covered"], cfg.block, cfg.top_k, cfg.alpha, out,
                        scores=scores)
    torch.cuda.synchronize()
    assert torch.equal(out[0], kv_idx) and torch.equal(out[1], kv_cnt)
    if with_scores:
        assert torch.equal(scores, s_ref)


def test_two_calls_second_smaller():
    for name in ("headline", "small"):
        cfg = get_config(name)
        d = dev_inputs(make_inputs(cfg))
        check_same(cfg, d, with_scores=False)
    cfg = get_config("small")
    check_same(cfg, dev_inputs(make_inputs(cfg)), with_scores=True)


def test_largest_workload_fits():
    cfg = get_config("stress")
    d = dev_inputs(make_inputs(cfg))
    check_same(cfg, d, with_scores=False)


def test_over_the_limit_is_rejected_unless_scores_are_returned():
    # 12 heads x 64 query blocks x 8192 KV blocks of float32 scores: 25.2 MB > 24 MiB
    cfg = get_config("small").with_(name="over-limit", heads=12, chunk_tokens=4096, past_chunks=127, top_k=64)
    assert cfg.nq == 64 and cfg.nk == 8192
    p = velox.problem_for((cfg.batch, cfg.heads, cfg.chunk_tokens, cfg.head_dim), cfg.kv_tokens, cfg.block,
                          cfg.top_k, cfg.alpha, velox.VELOX_BF16)
    assert velox.velox_route_workspace_bytes(p) > (24 << 20)
    g = torch.Generator(device="cuda").manual_seed(7)
    B, H, T, N, dd = cfg.batch, cfg.heads, cfg.chunk_tokens, cfg.kv_tokens, cfg.head_dim
    d = dict(q=torch.randn((B, H, T, dd), generator=g, device="cuda").to(torch.bfloat16),
             k=torch.randn((B, H, N, dd), generator=g, device="cuda").to(torch.bfloat16),
             overlap=torch.rand((B, cfg.nq, cfg.past_chunks), generator=g, device="cuda"),
             covered=torch.ones((B, cfg.nq), dtype=torch.uint8, device="cuda"))
    out = outputs(cfg)
    say(f"{cfg.name}: velox_route_noalloc without scores (must be rejected)")
    with pytest.raises(velox.VeloxError) as e:
        velox.route_noalloc(d["q"], d["k"], d["overlap"], d["covered"], cfg.block, cfg.top_k, cfg.alpha, out)
    assert e.value.status == velox.Status.WORKSPACE
    torch.cuda.synchronize()
    assert int((out[0] != -5).sum()) == 0  # nothing was launched
    check_same(cfg, d, with_scores=True)
