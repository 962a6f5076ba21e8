"""Host-side logic that needs no GPU: workload sizes, generator determinism and
recipe, and the benchmark's own guards.

* Derived sizes of the five workloads (block counts, executed and dense FLOPs)
  against the values computed by hand from their shapes: the headline keeps
  256 of 1568 KV blocks and executes 1.649 TFLOP of 10.10 TFLOP dense.
* The generator is deterministic per seed and independent of its thread count;
  uncovered query blocks follow the stated rounding (round(p * nq) per
  rollout); frustum workloads mark a row covered exactly when some overlap is
  positive.
* bench.py refuses more than one GPU before touching the GPU, and reports
  HBM traffic only while the profiled kernel source is unchanged.
"""
import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

from synth import get_config, make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name,nq,nk,f_exec,f_dense", [
    ("tiny", 4, 36, 50_331_648, 150_994_944),
    ("small", 16, 208, 3_221_225_472, 13_958_643_712),
    ("mid", 16, 400, 137_438_953_472, 858_993_459_200),
    ("headline", 32, 1568, 1_649_267_441_664, 10_101_763_080_192),
    ("stress", 32, 3104, 3_298_534_883_328, 39_994_735_460_352),
])
def test_workload_sizes(name, nq, nk, f_exec, f_dense):
    cfg = get_config(name)
    assert (cfg.nq, cfg.nk) == (nq, nk)
    assert cfg.flops_exec() == f_exec
    assert cfg.flops_dense() == f_dense
    # every executed tile is blk x blk: F_exec = 4 d blk^2 * rows * k_eff
    assert f_exec == 4 * cfg.head_dim * cfg.block ** 2 * cfg.rows * cfg.k_eff


def test_generator_is_deterministic_and_thread_independent():
    cfg = get_config("small").with_(heads=3)
    a = make_inputs(cfg, threads=1)
    b = make_inputs(cfg, threads=3)
    for name in ("q", "k", "v", "overlap", "covered"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    c = make_inputs(cfg, seeds=(cfg.seeds[0] + 1,), threads=1)
    assert not np.array_equal(a.q, c.q)


@pytest.mark.parametrize("name,uncovered", [("tiny", 1), ("small", 3)])
def test_uncovered_count_rounding(name, uncovered):
    cfg = get_config(name)
    x = make_inputs(cfg)
    assert int((x.covered == 0).sum()) == uncovered * cfg.batch
    assert x.overlap.min() >= 0.0 and x.overlap.max() <= 1.0


def test_frustum_coverage_rule():
    cfg = get_config("mid").with_(heads=1)
    x = make_inputs(cfg)
    assert np.array_equal(x.covered.astype(bool), (x.overlap > 0).any(axis=2))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_bench_traffic_only_for_the_profiled_source(tmp_path):
    bench = _bench_module()
    other = tmp_path / "other.hip"
    other.write_text("// not the profiled kernel\n")
    assert bench.traffic_from_profiles(str(other)) is None
    import json
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic_sparse_fa_headline.json")))
    src = os.path.join(ROOT, "geometry_routed_block_velox_amd", "csrc", "sparse_fa.hip")
    expected = rec["hbm_bytes_per_launch"] if rec["kernel_source_sha"] == bench.file_sha(src) else None
    assert bench.traffic_from_profiles(src) == expected


@pytest.mark.parametrize("kind", ["random", "constant-q", "large-logits"])
def test_lse_slack_bounds_a_scaled_q_log_sum_exp(kind):
    """The LSE slack of the parity rules is a bound: the log-sum-exp taken with
    bf16(c q) in place of c q (exact fp64 arithmetic otherwise) stays within the
    slack of the exact one, also when every q component rounds the same way."""
    from synth.generate import bf16_bits_to_f32, f32_to_bf16_bits
    from tests.parity_rules import bf16_fast_lse_slack
    rng = np.random.default_rng(21)
    B, H, T, d, blk, nk, k = 1, 2, 128, 64, 64, 6, 3
    q = rng.standard_normal((B, H, T, d)).astype(np.float32)
    kk = rng.standard_normal((B, H, nk * blk, d)).astype(np.float32)
    if kind == "constant-q":
        q[:] = 1.0
    if kind == "large-logits":
        kk[:, :, 2 * blk:3 * blk] += 4.0
    qb, kb = f32_to_bf16_bits(q), f32_to_bf16_bits(kk)
    idx = np.stack([rng.permutation(nk)[:k] for _ in range(B * H * (T // blk))]).reshape(B, H, T // blk, k)
    idx = idx.astype(np.int32)
    cnt = np.full((B, H, T // blk), k, np.int32)
    toks = np.arange(B * H * T)
    slack = bf16_fast_lse_slack(qb, kb, idx, cnt, blk, toks)
    qf = bf16_bits_to_f32(qb).reshape(-1, d).astype(np.float64)
    c32 = np.float32(1.4426950408889634) / np.sqrt(np.float32(d))
    qs = bf16_bits_to_f32(f32_to_bf16_bits(bf16_bits_to_f32(qb).reshape(-1, d) * c32)).astype(np.float64)
    c = np.log2(np.e) / np.sqrt(d)
    for t in toks:
        bh, i = divmod(int(t) // blk, T // blk)
        b, h = divmod(bh, H)
        keys = (idx[b, h, i][:, None] * blk + np.arange(blk)).reshape(-1)
        K = bf16_bits_to_f32(kb[b, h, keys]).astype(np.float64)
        exact = K @ qf[t] * c
        scaled = K @ qs[t]
        lse_exact = np.log(2) * (exact.max() + np.log2(np.exp2(exact - exact.max()).sum()))
        lse_scaled = np.log(2) * (scaled.max() + np.log2(np.exp2(scaled - scaled.max()).sum()))
        assert abs(lse_scaled - lse_exact) <= slack[t] + 1e-9, (kind, t, lse_scaled - lse_exact, slack[t])
    assert slack.max() > 0
