"""The Python binding rejects caller-provided buffers that do not fit, before any launch:
wrong shape, dtype or device of `out` / `workspace` arguments raise instead of letting a
kernel write outside them."""
import pytest

torch = pytest.importorskip("torch")

import geometry_routed_block_velox_amd as velox
from tests.gpu_helpers import cached_inputs, dev_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    velox.lib()


def test_outputs_are_checked():
    x = cached_inputs("small")
    cfg = x.cfg
    d = dev_inputs(x)
    B, H, nq = cfg.batch, cfg.heads, cfg.nq
    good_idx = torch.empty((B, H, nq, cfg.top_k), dtype=torch.int32, device="cuda")
    good_cnt = torch.empty((B, H, nq), dtype=torch.int32, device="cuda")
    bad = [
        (torch.empty((B, H, nq, cfg.top_k - 1), dtype=torch.int32, device="cuda"), good_cnt),
        (good_idx.to(torch.int64), good_cnt),
        (good_idx, torch.empty((B, H, nq), dtype=torch.int32)),  # host memory
    ]
    for out in bad:
        with pytest.raises((ValueError, TypeError)):
            velox.route(d["q"], d["k"], d["overlap"], d["covered"], cfg.block, cfg.top_k, cfg.alpha, out=out)
    with pytest.raises(ValueError):
        velox.route(d["q"], d["k"], d["overlap"], d["covered"], cfg.block, cfg.top_k, cfg.alpha,
                    workspace=torch.empty(1 << 20, dtype=torch.uint8))  # host workspace
    kv_idx, kv_cnt = velox.route(d["q"], d["k"], d["overlap"], d["covered"], cfg.block, cfg.top_k, cfg.alpha,
                                 out=(good_idx, good_cnt))
    for out in (torch.empty_like(d["q"])[:, :, :-1], torch.empty(d["q"].shape, dtype=torch.float32, device="cuda")):
        with pytest.raises((ValueError, TypeError)):
            velox.sparse_attn(d["q"], d["k"], d["v"], kv_idx, kv_cnt, cfg.block, out=out)
    o = velox.sparse_attn(d["q"], d["k"], d["v"], kv_idx, kv_cnt, cfg.block, out=torch.empty_like(d["q"]))
    torch.cuda.synchronize()
    assert o.shape == d["q"].shape
