"""On-device frustum-slice overlap (velox_frustum_overlap) and the scoring step
(velox_score), separately and run concurrently on two streams.

* Overlap against the oracle's fp64 implementation: max-abs 2e-5 (float32
  angles in degrees and depths in metres); coverage flags exact wherever the
  oracle's largest overlap of the row is not within 1e-5 of zero.
* velox_score's scores are bit-identical to velox_route's.
* The asynchronous pattern: overlap built on a side stream while the scores
  are computed on the main stream, joined by an event before velox_select;
  the lists equal velox_route's on the same overlap, bit for bit.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import geometry_routed_block_velox_amd as velox
from oracle import velox_oracle as O
from tests.gpu_helpers import cached_inputs, dev_inputs, say

pytestmark = pytest.mark.gpu

OV_ATOL = 2e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    velox.lib()


def stack_geometry(geoms):
    yaw = np.stack([g.yaw for g in geoms]).astype(np.float32)
    pd = np.stack([g.past_depth for g in geoms]).astype(np.float32)
    qd = np.stack([g.query_depth for g in geoms]).astype(np.float32)
    return yaw, pd, qd


def check_builder(yaw, pd, qd, fov, what):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    say(f"{what}: velox_frustum_overlap B{yaw.shape[0]} nq{qd.shape[1]} C{yaw.shape[1] - 1}")
    o, cov = velox.frustum_overlap(dev(yaw), dev(pd), dev(qd), fov)
    torch.cuda.synchronize()
    ref, ref_cov = O.frustum_overlap(yaw, pd, qd, fov)
    o = o.cpu().numpy().astype(np.float64)
    err = np.abs(o - ref)
    assert err.size == 0 or err.max() <= OV_ATOL, f"overlap max err {err.max():.3g}"
    mx = ref.max(axis=2) if ref.shape[2] else np.zeros(ref_cov.shape)
    decisive = (mx == 0.0) | (mx >= 1e-5)
    assert np.array_equal(cov.cpu().numpy()[decisive], ref_cov[decisive])
    say(f"{what}: max err {err.max() if err.size else 0:.3g}, covered rows {int(ref_cov.sum())} of {ref_cov.size}")
    return o, cov


@pytest.mark.parametrize("name", ["mid", "headline", "stress"])
def test_builder_matches_oracle_on_workload_geometry(name):
    x = cached_inputs(name)
    assert x.geometry is not None
    yaw, pd, qd = stack_geometry(x.geometry)
    o, _ = check_builder(yaw, pd, qd, x.geometry[0].fov, name)
    # the workload's own overlap is the same quantity
    assert np.abs(o - x.overlap).max() <= OV_ATOL


@pytest.mark.parametrize("seed,nq,C,fov", [(1, 32, 48, 90.0), (2, 7, 130, 60.0), (3, 64, 5, 180.0),
                                           (4, 1, 1, 90.0), (5, 16, 300, 120.0)])
def test_builder_matches_oracle_on_random_geometry(seed, nq, C, fov):
    rng = np.random.default_rng(seed)
    B = 3
    yaw = rng.uniform(-400.0, 400.0, (B, C + 1)).astype(np.float32)
    yaw[:, -1] = rng.uniform(-20.0, 20.0, B)
    yaw[0, :C // 2] = yaw[0, -1] + rng.choice([0.0, fov / 2, -fov / 2, fov, -fov, 360.0], C // 2)  # edge cases
    pd = np.sort(rng.uniform(0.5, 25.0, (B, C, 2)), axis=2).astype(np.float32)
    qd = np.sort(rng.uniform(0.5, 25.0, (B, nq, 2)), axis=2).astype(np.float32)
    qd[1, 0] = [3.0, 3.0]  # zero-length depth interval
    check_builder(yaw, pd, qd, fov, f"random seed {seed}")


def test_builder_without_history():
    qd = torch.tensor([[[1.0, 2.0], [3.0, 9.0]]], device="cuda")
    yaw = torch.zeros((1, 1), device="cuda")
    o, cov = velox.frustum_overlap(yaw, None, qd, 90.0)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0) and int(cov.sum()) == 0


@pytest.mark.parametrize("name", ["small", "headline"])
def test_score_equals_route_scores(name):
    x = cached_inputs(name)
    cfg = x.cfg
    d = dev_inputs(x)
    s = velox.score(d["q"], d["k"], cfg.block)
    _, _, ref = velox.route(d["q"], d["k"], d["overlap"], d["covered"], cfg.block, cfg.top_k, cfg.alpha,
                            return_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(s.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("name", ["mid", "headline"])
def test_overlap_on_side_stream_joins_before_selection(name):
    x = cached_inputs(name)
    cfg = x.cfg
    d = dev_inputs(x)
    yaw, pd, qd = (torch.from_numpy(a).cuda() for a in stack_geometry(x.geometry))
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ready = torch.cuda.Event()
    torch.cuda.synchronize()
    say(f"{name}: overlap on a side stream, scores on the main stream")
    with torch.cuda.stream(side):
        ov, cov = velox.frustum_overlap(yaw, pd, qd, x.geometry[0].fov, stream=side)
        ready.record(side)
    s = velox.score(d["q"], d["k"], cfg.block, stream=main)
    main.wait_event(ready)
    idx, cnt = velox.select(s, ov, cov, cfg.block, cfg.top_k, cfg.alpha, stream=main)
    torch.cuda.synchronize()
    ref_idx, ref_cnt = velox.route(d["q"], d["k"], ov, cov, cfg.block, cfg.top_k, cfg.alpha)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx) and torch.equal(cnt, ref_cnt)
