"""The layer (velox_route + velox_sparse_attn, caller-owned buffers) captured in a HIP graph
and replayed: every replay, with eager work and synchronisations in between, gives
results bit-identical to the eager calls.  The path records no memset node (its kernels
write every output element themselves), so replays after the first stay correct."""
import pytest

torch = pytest.importorskip("torch")

import geometry_routed_block_velox_amd as velox
from tests.gpu_helpers import cached_inputs, dev_inputs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    velox.lib()


@pytest.mark.parametrize("name", ["small", "mid"])
def test_layer_graph_replays_match_eager(name):
    x = cached_inputs(name)
    cfg = x.cfg
    d = dev_inputs(x)
    q, k, v = d["q"], d["k"], d["v"]
    B, H, nq = cfg.batch, cfg.heads, cfg.nq
    p = velox.problem_for(tuple(q.shape), k.shape[2], cfg.block, cfg.top_k, cfg.alpha, velox.VELOX_BF16)
    ws = torch.empty(velox.velox_route_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    kv_idx = torch.empty((B, H, nq, cfg.top_k), dtype=torch.int32, device="cuda")
    kv_cnt = torch.empty((B, H, nq), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)

    def layer(stream=None):
        velox.route(q, k, d["overlap"], d["covered"], cfg.block, cfg.top_k, cfg.alpha, out=(kv_idx, kv_cnt),
                    workspace=ws, stream=stream)
        velox.sparse_attn(q, k, v, kv_idx, kv_cnt, cfg.block, out=out, stream=stream)

    layer()
    torch.cuda.synchronize()
    ref_idx, ref_cnt, ref_out = kv_idx.clone(), kv_cnt.clone(), out.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer(side)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(torch.cuda.current_stream())
    for rep in range(3):
        kv_idx.fill_(-7)
        kv_cnt.zero_()
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"{name}: graph replay {rep}")
        assert torch.equal(kv_idx, ref_idx) and torch.equal(kv_cnt, ref_cnt)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        layer()  # eager work between replays
        torch.cuda.synchronize()
