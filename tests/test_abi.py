"""The C ABI library without a GPU: it loads, exports every declared symbol, and
validates arguments on the host before any launch."""
import ctypes as C
import os
import re

import pytest

import geometry_routed_block_velox_amd as velox
from geometry_routed_block_velox_amd import Problem, Status

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "velox.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(velox_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"velox_check", "velox_route", "velox_select", "velox_sparse_attn", "velox_route_workspace_bytes",
            "velox_status_string", "velox_last_hip_error", "velox_pool_keys", "velox_route_cached", "velox_sparse_attn_split",
            "velox_sparse_attn_split_workspace_bytes", "velox_sparse_attn_auto_splits", "velox_score",
            "velox_frustum_overlap"} <= set(names)
    lib = C.CDLL(velox.library_path)
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"


def headline():
    return Problem(1, 24, 128, 4096, 48, 128, 256, 2.0, velox.VELOX_BF16)


def test_check_accepts_every_workload():
    from synth import CONFIGS
    for cfg in CONFIGS.values():
        p = Problem(cfg.batch, cfg.heads, cfg.head_dim, cfg.chunk_tokens, cfg.past_chunks, cfg.block, cfg.top_k,
                    cfg.alpha, velox.VELOX_BF16 if cfg.dtype == "bf16" else velox.VELOX_F32)
        assert velox.velox_check(p) == Status.OK, cfg.name


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, Status.BAD_SHAPE), ("heads", 0, Status.BAD_SHAPE), ("past_chunks", -1, Status.BAD_SHAPE),
    ("chunk_tokens", 4000, Status.BAD_SHAPE), ("chunk_tokens", 64, Status.BAD_SHAPE),
    ("top_k", 31, Status.BAD_SHAPE), ("alpha", -1.0, Status.BAD_SHAPE), ("alpha", float("nan"), Status.BAD_SHAPE),
    ("alpha", float("inf"), Status.BAD_SHAPE), ("head_dim", 96, Status.UNSUPPORTED),
    ("block", 32, Status.UNSUPPORTED), ("dtype", 7, Status.UNSUPPORTED),
    ("chunk_tokens", 128 * 65, Status.UNSUPPORTED), ("past_chunks", 300, Status.UNSUPPORTED),
    ("heads", 65536, Status.UNSUPPORTED),
])
def test_check_rejects(field, value, status):
    p = headline()
    setattr(p, field, value)
    assert velox.velox_check(p) == status
    assert velox.velox_route_workspace_bytes(p) == 0


def test_check_null_and_limits():
    assert velox.lib().velox_check(None) == Status.NULL_POINTER
    p = headline()
    p.top_k = 10_000  # above nk: keep-all, still valid
    assert velox.velox_check(p) == Status.OK
    p = headline()
    p.past_chunks = 255  # nk = 256*32 = 8192, the limit
    assert velox.velox_check(p) == Status.OK


def test_workspace_bytes():
    p = headline()
    rows = 24 * 32
    expect = rows * 128 * 4 + ((rows * 1568 * 4 + 255) // 256) * 256
    assert velox.velox_route_workspace_bytes(p) == expect


def test_entry_points_validate_before_launch():
    # Every call below fails host-side validation, so nothing touches a GPU.
    L = velox.lib()
    p = headline()
    fake = C.c_void_p(0x100000)
    mis = C.c_void_p(0x100001)
    ws_need = velox.velox_route_workspace_bytes(p)
    assert L.velox_route(C.byref(p), None, fake, fake, fake, fake, fake, None, fake, ws_need, None) == Status.NULL_POINTER
    assert L.velox_route(C.byref(p), fake, fake, None, fake, fake, fake, None, fake, ws_need, None) == Status.NULL_POINTER
    assert L.velox_route(C.byref(p), mis, fake, fake, fake, fake, fake, None, fake, ws_need, None) == Status.MISALIGNED
    assert L.velox_route(C.byref(p), fake, fake, fake, fake, fake, fake, None, fake, ws_need - 1, None) == Status.WORKSPACE
    assert L.velox_route(C.byref(p), fake, fake, fake, fake, fake, fake, None, None, ws_need, None) == Status.NULL_POINTER
    assert L.velox_route(C.byref(p), fake, fake, fake, fake, fake, fake, None, C.c_void_p(0x100010), ws_need,
                         None) == Status.WORKSPACE
    bad = headline()
    bad.top_k = 3
    assert L.velox_route(C.byref(bad), fake, fake, fake, fake, fake, fake, None, fake, ws_need, None) == Status.BAD_SHAPE
    assert L.velox_select(C.byref(p), None, fake, fake, fake, fake, None) == Status.NULL_POINTER
    assert L.velox_sparse_attn(C.byref(p), fake, fake, mis, fake, fake, fake, None, None) == Status.MISALIGNED
    assert L.velox_sparse_attn(C.byref(p), fake, fake, fake, None, fake, fake, None, None) == Status.NULL_POINTER
    # attention accepts a list stride below ncur (user lists), routing does not
    short = headline()
    short.top_k = 4
    assert L.velox_sparse_attn(C.byref(short), fake, fake, fake, None, fake, fake, None, None) == Status.NULL_POINTER
    assert velox.velox_check(short) == Status.BAD_SHAPE
    assert L.velox_last_hip_error() == 0


def test_cache_entry_points_validate_before_launch():
    L = velox.lib()
    p = headline()  # nq = 32, nk = 1568, C = 48
    fake = C.c_void_p(0x100000)
    mis = C.c_void_p(0x100008)
    nk = 1568
    assert L.velox_pool_keys(C.byref(p), None, fake, nk, 0, 1, None) == Status.NULL_POINTER
    assert L.velox_pool_keys(C.byref(p), fake, mis, nk, 0, 1, None) == Status.MISALIGNED
    assert L.velox_pool_keys(C.byref(p), fake, fake, nk, -1, 1, None) == Status.BAD_SHAPE
    assert L.velox_pool_keys(C.byref(p), fake, fake, nk, 0, -1, None) == Status.BAD_SHAPE
    assert L.velox_pool_keys(C.byref(p), fake, fake, nk, nk - 3, 4, None) == Status.BAD_SHAPE   # past nk
    assert L.velox_pool_keys(C.byref(p), fake, fake, 100, 90, 11, None) == Status.BAD_SHAPE     # past the cache
    assert L.velox_pool_keys(C.byref(p), fake, fake, nk, 5, 0, None) == Status.OK               # empty: no launch
    small_k = headline()
    small_k.top_k = 1  # pooling does not route: any top_k >= 1 is valid
    assert L.velox_pool_keys(C.byref(small_k), fake, fake, nk, 5, 0, None) == Status.OK
    ws = velox.velox_route_workspace_bytes(p)
    args = lambda kbar, cb, scores=None, w=ws: (C.byref(p), fake, kbar, cb, fake, fake, fake, fake, scores, fake, w,
                                                None)
    assert L.velox_route_cached(*args(None, nk)) == Status.NULL_POINTER
    assert L.velox_route_cached(*args(mis, nk)) == Status.MISALIGNED
    assert L.velox_route_cached(*args(fake, 48 * 32 - 1)) == Status.BAD_SHAPE       # past rows not covered
    assert L.velox_route_cached(*args(fake, 48 * 32, fake)) == Status.BAD_SHAPE     # scores need all nk rows
    assert L.velox_route_cached(*args(fake, nk, None, ws - 1)) == Status.WORKSPACE
    assert L.velox_route_cached(C.byref(p), fake, fake, nk, None, fake, fake, fake, None, fake, ws,
                                None) == Status.NULL_POINTER                           # overlap needed when C > 0
    assert L.velox_last_hip_error() == 0


def test_modulation_mode_is_validated():
    p = headline()
    assert p.modulation == velox.MOD_SCALE          # zero-initialised default
    p.modulation = velox.MOD_LOG_PROB
    assert velox.velox_check(p) == Status.OK
    for bad in (2, -1, 7):
        p.modulation = bad
        assert velox.velox_check(p) == Status.BAD_SHAPE
        assert velox.velox_route_workspace_bytes(p) == 0
    fake = C.c_void_p(0x100000)
    assert velox.lib().velox_sparse_attn(C.byref(p), fake, fake, fake, fake, fake, fake, None,
                                         None) == Status.BAD_SHAPE


def test_split_entry_points_validate_before_launch():
    L = velox.lib()
    p = headline()
    fake = C.c_void_p(0x100000)
    assert L.velox_sparse_attn_split_workspace_bytes(C.byref(p), 0) == 0
    assert L.velox_sparse_attn_split_workspace_bytes(C.byref(p), 65) == 0
    need = L.velox_sparse_attn_split_workspace_bytes(C.byref(p), 4)
    parts = 768 * 4
    assert need == (parts * 128 * 128 * 4 + 255) // 256 * 256 + (parts * 128 * 4 + 255) // 256 * 256
    call = lambda n, ws, wb: L.velox_sparse_attn_split(C.byref(p), fake, fake, fake, fake, fake, n, fake, None, ws,
                                                       wb, None)
    assert call(0, fake, need) == Status.BAD_SHAPE
    assert call(65, fake, need) == Status.BAD_SHAPE
    assert call(4, None, need) == Status.NULL_POINTER
    assert call(4, fake, need - 1) == Status.WORKSPACE
    assert call(4, C.c_void_p(0x100040), need) == Status.WORKSPACE
    # auto splits: rows (768) fill 256 CUs -> 1; Small-like 64 rows -> 8 (two per CU), capped by list length
    assert L.velox_sparse_attn_auto_splits(C.byref(p), 256) == 1
    small = Problem(1, 4, 64, 1024, 12, 64, 48, 2.0, velox.VELOX_BF16)
    assert L.velox_sparse_attn_auto_splits(C.byref(small), 256) == 8
    tiny = Problem(1, 1, 64, 256, 8, 64, 12, 1.0, velox.VELOX_F32)
    assert L.velox_sparse_attn_auto_splits(C.byref(tiny), 256) == 3
    assert L.velox_last_hip_error() == 0


def test_score_and_overlap_builder_validate_before_launch():
    L = velox.lib()
    p = headline()
    fake = C.c_void_p(0x100000)
    ws = velox.velox_route_workspace_bytes(p)
    assert L.velox_score(C.byref(p), fake, fake, None, fake, ws, None) == Status.NULL_POINTER
    assert L.velox_score(C.byref(p), fake, fake, fake, fake, ws - 1, None) == Status.WORKSPACE
    assert L.velox_score(C.byref(p), C.c_void_p(0x100002), fake, fake, fake, ws, None) == Status.MISALIGNED
    for fov in (0.0, -5.0, 180.5, float("nan")):
        assert L.velox_frustum_overlap(C.byref(p), fake, fake, fake, fov, fake, fake, None) == Status.BAD_SHAPE
    assert L.velox_frustum_overlap(C.byref(p), fake, None, fake, 90.0, fake, fake, None) == Status.NULL_POINTER
    assert L.velox_frustum_overlap(C.byref(p), fake, fake, fake, 90.0, None, fake, None) == Status.NULL_POINTER
    assert L.velox_last_hip_error() == 0


def test_status_strings():
    L = velox.lib()
    for s in range(7):
        assert L.velox_status_string(s)
    assert L.velox_status_string(99) == b"unknown status"


def test_route_noalloc_validates_before_device_work():
    """Every check of velox_route_noalloc runs on the host before the scratch array is
    looked up, so these calls need no GPU."""
    L = velox.lib()
    fake = C.c_void_p(0x100000)
    p = headline()
    args = (fake, fake, fake, fake, fake, fake, None, None)
    assert L.velox_route_noalloc(None, *args) == Status.NULL_POINTER
    assert L.velox_route_noalloc(C.byref(p), None, fake, fake, fake, fake, fake, None, None) == Status.NULL_POINTER
    assert L.velox_route_noalloc(C.byref(p), fake, fake, fake, fake, fake, None, None, None) == Status.NULL_POINTER
    assert L.velox_route_noalloc(C.byref(p), C.c_void_p(0x100002), fake, fake, fake, fake, fake, None,
                                 None) == Status.MISALIGNED
    bad = headline()
    bad.top_k = 3
    assert L.velox_route_noalloc(C.byref(bad), *args) == Status.BAD_SHAPE
    # 12 heads x 64 query blocks x 8192 KV blocks: the score matrix (25.2 MB) exceeds the
    # 24 MiB scratch array; with the scores returned only the pooled queries are needed
    big = Problem(1, 12, 64, 4096, 127, 64, 64, 2.0, velox.VELOX_BF16)
    assert velox.velox_check(big) == Status.OK
    assert velox.velox_route_workspace_bytes(big) > (24 << 20)
    assert L.velox_route_noalloc(C.byref(big), *args) == Status.WORKSPACE
    assert L.velox_last_hip_error() == 0
