"""Benchmark of one routed attention layer (velox_route + velox_sparse_attn) on one MI355X.

A step is one full layer over one batch of synthetic input resident in HBM:
pooled block scoring, overlap modulation + per-row top-k, and block-skipping
attention, for every head of the workload.  Prints one JSON line:
value = effective TFLOP/s (QK^T + PV FLOPs of the executed tiles / layer time);
ms_per_step = ms per layer.  Also reports the dense-equivalent rate, per-kernel
times, the roofline fraction of the attention kernel (HIP events on the launch
stream), the routing phase's HBM fraction, and the CPU oracle timed on a
bounded sample of the same workload on this host.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true", help="skip the keep-all comparison")
    ap.add_argument("--cold-reps", type=int, default=20, help="layers timed after a 1 GiB cache-flushing write")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 1 GiB device-to-device copy first (reference for HBM counter scaling)")
    return ap.parse_args()


def timed_ahead(fn, reps, stream):
    """GPU time per call of `fn` run back to back: the stream first runs a spin kernel
    long enough for the host to enqueue all `reps` calls behind it, so the figure is
    the calls' device time, not the host's launch rate (these calls take tens of us)."""
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spin = getattr(torch.cuda, "_sleep", None)  # a private torch helper; without it the host is not ahead
    if spin is not None:
        with torch.cuda.stream(stream):
            spin(400_000 * reps)  # >= ~150 us of host time per call at <= 2.4 GHz
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def file_sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_from_profiles(kernel_src):
    """HBM bytes per launch measured with rocprofv3 PMC counters, if the committed
    measurement was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_sparse_fa_headline.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha") != file_sha(kernel_src):
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer runs on a single MI355X "
              "(head sharding across GPUs is a design note, not built); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import geometry_routed_block_velox_amd as velox
    from synth import get_config, make_inputs

    cfg = get_config(args.config)
    t0 = time.time()
    x = make_inputs(cfg)
    print(f"[bench] inputs for {cfg.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    bf = cfg.dtype == "bf16"

    def up(a, cast=False):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if cast and a.dtype == np.uint16:
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.cuda()

    q, k, v = up(x.q, bf), up(x.k, bf), up(x.v, bf)
    ov, cov = up(x.overlap), up(x.covered)
    B, H, nq = cfg.batch, cfg.heads, cfg.nq
    kv_idx = torch.empty((B, H, nq, cfg.top_k), dtype=torch.int32, device="cuda")
    kv_cnt = torch.empty((B, H, nq), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    p = velox.problem_for(tuple(q.shape), k.shape[2], cfg.block, cfg.top_k, cfg.alpha,
                          velox.VELOX_BF16 if bf else velox.VELOX_F32)
    ws = torch.empty(velox.velox_route_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def step(e=None):
        if e is not None:
            e[0].record(stream)
        velox.route(q, k, ov, cov, cfg.block, cfg.top_k, cfg.alpha, out=(kv_idx, kv_cnt), workspace=ws)
        if e is not None:
            e[1].record(stream)
        velox.sparse_attn(q, k, v, kv_idx, kv_cnt, cfg.block, out=out)
        if e is not None:
            e[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    route_ms = [a.elapsed_time(b) for a, b, _ in ev]
    attn_ms = [b.elapsed_time(c) for _, b, c in ev]
    layer_ms = [a.elapsed_time(c) for a, _, c in ev]
    ms_step = wall * 1e3 / args.steps

    # cold protocol: a 1 GiB scratch write (4x the 256 MB MALL) before each timed layer
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    cold_ms = []
    for _ in range(args.cold_reps):
        scratch.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        cold_ms.append(e0.elapsed_time(e1))
    # measured device-copy bandwidth (1 GiB read + 1 GiB written per copy): the practical HBM ceiling
    dst = torch.empty_like(scratch)
    dst.copy_(scratch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        dst.copy_(scratch)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2.0 * scratch.numel() * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del scratch, dst

    cnt = kv_cnt.cpu().numpy()
    f_exec = 4.0 * cfg.head_dim * cfg.block * cfg.block * float(cnt.sum())
    f_dense = float(cfg.flops_dense())
    gi = kv_idx.cpu().numpy()
    union_blocks = sum(len(np.unique(gi[b, h][gi[b, h] >= 0])) for b in range(B) for h in range(H))
    el = 2 if bf else 4
    kv_block_bytes = 2 * cfg.block * cfg.head_dim * el
    attn_bytes = 2 * q.numel() * el + union_blocks * kv_block_bytes
    route_bytes = (q.numel() + k.numel()) * el + x.overlap.nbytes + x.covered.nbytes + gi.nbytes + cnt.nbytes
    attn_avg = float(np.mean(attn_ms))
    route_avg = float(np.mean(route_ms))
    achieved = f_exec / (attn_avg * 1e-3) / 1e12
    kernel_src = os.path.join(ROOT, "geometry_routed_block_velox_amd", "csrc", "sparse_fa.hip")
    res = {
        "metric": "ms/layer + effective TFLOP/s of routed sparse attention at chunk 48, 1 GPU",
        "value": round(f_exec / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: B{B} H{H} d{cfg.head_dim} T{cfg.chunk_tokens} chunk{cfg.past_chunks} "
                        f"(N={cfg.kv_tokens}) blk{cfg.block} top-k{cfg.top_k} alpha{cfg.alpha}",
            "global_batch": B, "seq_len": cfg.kv_tokens, "parallelism": "none (1 GPU)",
        },
        "ms_per_layer_events_median": round(float(np.median(layer_ms)), 4),
        "ms_per_layer_cold_median": round(float(np.median(cold_ms)), 4) if cold_ms else None,
        "route_ms": round(route_avg, 4),
        "attn_ms": round(attn_avg, 4),
        "dense_equiv_tflops": round(f_dense / (ms_step * 1e-3) / 1e12, 2),
        "flops_exec": f_exec,
        "flops_dense": f_dense,
        "route_hbm": {"bytes": route_bytes, "achieved_GBs": round(route_bytes / (route_avg * 1e-3) / 1e9, 1),
                      "peak_GBs": PEAK_HBM_GBS,
                      "frac": round(route_bytes / (route_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                      "measured_copy_GBs": round(copy_gbs, 1),
                      "frac_of_measured_copy": round(route_bytes / (route_avg * 1e-3) / 1e9 / copy_gbs, 4)},
        "roofline": {
            "kernel": "velox_sparse_fa (sparse_fa_bf16_kernel)" if bf else "sparse_fa_f32_kernel",
            "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_from_profiles(kernel_src),
            "algorithmic_bytes": attn_bytes,
            "kv_union_blocks": union_blocks,
        },
    }

    if not args.no_context:
        # keep-all through the same kernel: the same-kernel "dense" comparison at this chunk
        full_idx = torch.arange(cfg.nk, dtype=torch.int32, device="cuda").expand(B, H, nq, cfg.nk).contiguous()
        full_cnt = torch.full((B, H, nq), cfg.nk, dtype=torch.int32, device="cuda")
        velox.sparse_attn(q, k, v, full_idx, full_cnt, cfg.block, out=out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        reps = 3
        for _ in range(reps):
            velox.sparse_attn(q, k, v, full_idx, full_cnt, cfg.block, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        keep_all_ms = e0.elapsed_time(e1) / reps
        res["context_keep_all"] = {"attn_ms": round(keep_all_ms, 4),
                                   "tflops": round(f_dense / (keep_all_ms * 1e-3) / 1e12, 2),
                                   "attention_speedup_vs_keep_all": round(keep_all_ms / attn_avg, 3),
                                   "layer_speedup_vs_keep_all": round(keep_all_ms / ms_step, 3)}

    if x.geometry is not None:
        res["overlap_builder"] = bench_overlap_builder(velox, cfg, x, q, k, ws, stream)
    res["route_log_prob"] = bench_route_log_prob(velox, cfg, q, k, ov, cov, kv_idx, ws, stream)
    res["route_cached"] = bench_route_cached(velox, cfg, q, k, ov, cov, kv_idx, kv_cnt, ws, stream, el,
                                             x.overlap.nbytes + x.covered.nbytes + gi.nbytes + cnt.nbytes)

    res["split_kv_small"] = bench_split_small(velox, stream)

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, x, gi, cnt)
    print(json.dumps(res), flush=True)


def bench_overlap_builder(velox, cfg, x, q, k, ws, stream, reps=20):
    """The frustum-overlap builder alone, and the routing phase with the builder run
    (a) after the scoring on the same stream and (b) on a side stream next to it,
    joined by an event before the selection."""
    import numpy as np
    import torch
    g = x.geometry
    yaw = torch.from_numpy(np.stack([e.yaw for e in g])).cuda()
    pd = torch.from_numpy(np.stack([e.past_depth for e in g])).cuda()
    qd = torch.from_numpy(np.stack([e.query_depth for e in g])).cuda()
    fov = g[0].fov
    B, H, nq, nk = cfg.batch, cfg.heads, cfg.nq, cfg.nk
    ov = torch.empty((B, nq, cfg.past_chunks), dtype=torch.float32, device="cuda")
    cov = torch.empty((B, nq), dtype=torch.uint8, device="cuda")
    s = torch.empty((B, H, nq, nk), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, H, nq, cfg.top_k), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, H, nq), dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    ready = torch.cuda.Event()

    def sequential():
        velox.score(q, k, cfg.block, scores=s, workspace=ws, stream=stream)
        velox.frustum_overlap(yaw, pd, qd, fov, out=(ov, cov), stream=stream)
        velox.select(s, ov, cov, cfg.block, cfg.top_k, cfg.alpha, stream=stream)

    def concurrent():
        side.wait_stream(stream)
        velox.frustum_overlap(yaw, pd, qd, fov, out=(ov, cov), stream=side)
        ready.record(side)
        velox.score(q, k, cfg.block, scores=s, workspace=ws, stream=stream)
        stream.wait_event(ready)
        velox.select(s, ov, cov, cfg.block, cfg.top_k, cfg.alpha, stream=stream)

    def timed(fn):
        return timed_ahead(fn, reps, stream)

    t_builder = timed(lambda: velox.frustum_overlap(yaw, pd, qd, fov, out=(ov, cov), stream=stream))
    t_seq, t_conc = timed(sequential), timed(concurrent)
    return {"builder_ms": round(t_builder, 4), "route_with_builder_same_stream_ms": round(t_seq, 4),
            "route_with_builder_side_stream_ms": round(t_conc, 4),
            "note": "score -> select with the overlap built from the synthetic frustum geometry on the GPU; "
                    "side stream = built concurrently with the scoring, joined by an event"}


def bench_split_small(velox, stream, reps=50):
    """Split-KV attention on the Small workload (64 rows for 256 CUs): one workgroup per
    row against velox_sparse_attn_split with the automatic split count."""
    import numpy as np
    import torch
    from synth import get_config, make_inputs
    cfg = get_config("small")
    x = make_inputs(cfg)
    up = lambda a: (torch.from_numpy(a).view(torch.int16).view(torch.bfloat16) if a.dtype == np.uint16
                    else torch.from_numpy(a)).cuda()
    q, k, v = up(x.q), up(x.k), up(x.v)
    kv_idx, kv_cnt = velox.route(q, k, up(x.overlap), up(x.covered), cfg.block, cfg.top_k, cfg.alpha)
    p = velox.problem_for(tuple(q.shape), k.shape[2], cfg.block, cfg.top_k, cfg.alpha, velox.VELOX_BF16)
    n = velox.auto_splits(p)
    ws = torch.empty(max(velox.velox_sparse_attn_split_workspace_bytes(p, n), 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    f_exec = 4.0 * cfg.head_dim * cfg.block * cfg.block * float(kv_cnt.sum())

    def timed(splits):
        return timed_ahead(lambda: velox.sparse_attn(q, k, v, kv_idx, kv_cnt, cfg.block, out=out, splits=splits,
                                                     workspace=ws), reps, stream)

    t1, ts = timed(None), timed(n)
    return {"workload": f"small: B1 H4 d64 T1024 chunk12 blk64 top-k48 ({cfg.rows} rows)", "splits": n,
            "unsplit_ms": round(t1, 4), "split_ms": round(ts, 4), "speedup": round(t1 / ts, 3),
            "unsplit_tflops": round(f_exec / (t1 * 1e-3) / 1e12, 2),
            "split_tflops": round(f_exec / (ts * 1e-3) / 1e12, 2),
            "split_frac_of_peak": round(f_exec / (ts * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def bench_route_log_prob(velox, cfg, q, k, ov, cov, kv_idx, ws, stream, reps=20):
    """velox_route with the sign-safe (log-probability) modulation: same kernels and bytes,
    different modulation arithmetic in the select kernel."""
    import torch
    idx2 = torch.empty_like(kv_idx)
    cnt2 = torch.empty((cfg.batch, cfg.heads, cfg.nq), dtype=torch.int32, device="cuda")
    call = lambda: velox.route(q, k, ov, cov, cfg.block, cfg.top_k, cfg.alpha, out=(idx2, cnt2), workspace=ws,
                               modulation=velox.MOD_LOG_PROB)
    call()
    torch.cuda.synchronize()
    changed = int((idx2 != kv_idx).any(dim=-1).sum())
    return {"ms": round(timed_ahead(call, reps, stream), 4), "rows_with_different_list": changed,
            "rows": cfg.rows}


def bench_route_cached(velox, cfg, q, k, ov, cov, kv_idx, kv_cnt, ws, stream, el, small_bytes, reps=20):
    """Routing from the pooled-key cache: the past chunks' pooled keys are filled once
    (not timed), then velox_route_cached reads Q and the cached rows instead of K."""
    import torch
    B, H, nq, d = cfg.batch, cfg.heads, cfg.nq, cfg.head_dim
    past = cfg.past_chunks * nq
    kbar = torch.empty((B, H, max(past, 1), d), dtype=torch.float32, device="cuda")
    velox.pool_keys(k, cfg.chunk_tokens, cfg.block, 0, past, kbar=kbar)
    idx2 = torch.empty_like(kv_idx)
    cnt2 = torch.empty_like(kv_cnt)
    call = lambda: velox.route_cached(q, kbar, cfg.past_chunks, ov, cov, cfg.block, cfg.top_k, cfg.alpha,
                                      out=(idx2, cnt2), workspace=ws)
    call()
    torch.cuda.synchronize()
    same = bool(torch.equal(idx2, kv_idx) and torch.equal(cnt2, kv_cnt))
    ms = timed_ahead(call, reps, stream)
    nbytes = q.numel() * el + B * H * past * d * 4 + small_bytes
    gbs = nbytes / (ms * 1e-3) / 1e9
    # one-time cost per finished chunk: pooling its nq blocks into the cache
    pool_ms = timed_ahead(lambda: velox.pool_keys(k, cfg.chunk_tokens, cfg.block, max(past - nq, 0), min(nq, past),
                                                  kbar=kbar), reps, stream)
    return {"ms": round(ms, 4), "algorithmic_bytes": nbytes, "achieved_GBs": round(gbs, 1),
            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "identical_to_route": same,
            "pool_one_chunk_ms": round(pool_ms, 4),
            "note": "velox_route_cached with the past chunks' pooled keys cached; pool_one_chunk_ms is the "
                    "once-per-chunk velox_pool_keys cost of appending a finished chunk; device time of "
                    "back-to-back calls (the host enqueues them behind a spin kernel)"}


def cpu_model_name():
    """lscpu's model name (falls back to /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def oracle_layer_seconds(O, cfg, x, kv_idx=None, kv_cnt=None):
    """Wall time of the oracle's whole layer: routing of every row, then fp64
    attention of every query token over the given lists (the oracle's own if None)."""
    t0 = time.perf_counter()
    r = O.route(x.q, x.k, x.overlap, x.covered, cfg.block, cfg.top_k, cfg.alpha)
    t_route = time.perf_counter() - t0
    if kv_idx is None:
        kv_idx, kv_cnt = r["kv_idx"], r["kv_cnt"]
    t0 = time.perf_counter()
    O.attn(x.q, x.k, x.v, kv_idx, kv_cnt, cfg.block)
    return t_route, time.perf_counter() - t0


def cpu_baseline(cfg, x, gi, cnt):
    """The oracle (fp64, OpenMP) on this host, unsampled: routing of every row plus
    attention of every query token of the workload over the GPU's block lists,
    then the Tiny and Small workloads on one thread."""
    from oracle import velox_oracle as O
    from synth import get_config, make_inputs

    threads = O.num_threads()
    t_route, t_attn = oracle_layer_seconds(O, cfg, x, gi, cnt)
    t_layer = t_route + t_attn
    f_exec = 4.0 * cfg.head_dim * cfg.block * cfg.block * float(cnt.sum())
    single = {}
    O.set_threads(1)
    try:
        for name in ("tiny", "small"):
            c = get_config(name)
            xs = make_inputs(c)
            tr, ta = oracle_layer_seconds(O, c, xs)
            single[name] = {"ms_per_layer": round((tr + ta) * 1e3, 1), "route_ms": round(tr * 1e3, 1),
                            "attn_ms": round(ta * 1e3, 1)}
    finally:
        O.set_threads(threads)
    total = cfg.batch * cfg.heads * cfg.chunk_tokens
    return {"value": round(f_exec / t_layer / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "sampled": False, "ms_per_layer": round(t_layer * 1e3, 1),
            "route_s": round(t_route, 3), "attn_s": round(t_attn, 3), "cpu_model": cpu_model_name(),
            "single_thread": single,
            "sample": f"unsampled: routing of all {cfg.rows} rows and fp64 attention of all {total} query "
                      f"tokens over the GPU's block lists, {threads} OpenMP threads; Tiny and Small whole "
                      f"layers (oracle routing and attention) on one thread"}


if __name__ == "__main__":
    main()
