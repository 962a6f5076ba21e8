"""Velox routed block-sparse attention for MI355X (gfx950): Python binding.

Thin ctypes binding over the C ABI of libvelox.so (include/velox.h).  It only
marshals arguments: every step of the layer runs in the library's HIP
kernels.  PyTorch supplies device memory and the current HIP stream.  There is
no CPU fallback: if the library is missing or a call fails, an exception is
raised.

Entry points (same names as the C ABI):
  velox_check(problem) -> status
  velox_route_workspace_bytes(problem) -> int
  route(q, k, overlap, covered, block, top_k, alpha, ...) -> (kv_idx, kv_cnt[, scores])
  score(q, k, block, ...) -> scores
  frustum_overlap(yaw, past_depth, query_depth, fov_deg) -> (overlap, covered)
  pool_keys(k, chunk_tokens, block, first_block, num_blocks, ...) -> kbar cache
  route_cached(q, kbar, past_chunks, overlap, covered, block, top_k, alpha, ...) -> as route
  select(scores, overlap, covered, block, top_k, alpha) -> (kv_idx, kv_cnt)
  sparse_attn(q, k, v, kv_idx, kv_cnt, block, ..., splits=None|n|"auto") -> out[, lse]
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

__all__ = [
    "VeloxError", "Problem", "Status", "lib", "library_path", "velox_check", "velox_route_workspace_bytes",
    "route", "route_noalloc", "select", "sparse_attn", "problem_for", "pool_keys", "route_cached", "auto_splits", "score",
    "frustum_overlap",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libvelox.so")

VELOX_F32, VELOX_BF16 = 0, 1
MOD_SCALE, MOD_LOG_PROB = 0, 1   # velox_modulation
MAX_QUERY_BLOCKS, MAX_KV_BLOCKS = 64, 8192


class Status:
    OK, NULL_POINTER, BAD_SHAPE, UNSUPPORTED, MISALIGNED, WORKSPACE, HIP = range(7)


class VeloxError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().velox_status_string(status).decode()
        if status == Status.HIP:
            msg += f" (hipError_t {lib().velox_last_hip_error()})"
        super().__init__(f"{where}: {msg}")
        self.status = status


class Problem(C.Structure):
    """Mirror of `velox_problem` in include/velox.h."""
    _fields_ = [
        ("batch", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32), ("chunk_tokens", C.c_int32),
        ("past_chunks", C.c_int32), ("block", C.c_int32), ("top_k", C.c_int32), ("alpha", C.c_float),
        ("dtype", C.c_int32), ("modulation", C.c_int32),
    ]

    @property
    def nq(self):
        return self.chunk_tokens // self.block

    @property
    def nk(self):
        return (self.past_chunks + 1) * self.chunk_tokens // self.block

    def __repr__(self):
        return "Problem(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


_lib = None


def lib():
    """Load libvelox.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise ImportError(f"{library_path} is missing: build it with geometry_routed_block_velox_amd/build.py "
                              "(or __graft_entry__.build())")
        L = C.CDLL(library_path)
        P, V = C.POINTER(Problem), C.c_void_p
        L.velox_check.argtypes = [P]
        L.velox_check.restype = C.c_int
        L.velox_route_workspace_bytes.argtypes = [P]
        L.velox_route_workspace_bytes.restype = C.c_size_t
        L.velox_route.argtypes = [P, V, V, V, V, V, V, V, V, C.c_size_t, V]
        L.velox_route.restype = C.c_int
        L.velox_route_noalloc.argtypes = [P, V, V, V, V, V, V, V, V]
        L.velox_route_noalloc.restype = C.c_int
        L.velox_score.argtypes = [P, V, V, V, V, C.c_size_t, V]
        L.velox_score.restype = C.c_int
        L.velox_frustum_overlap.argtypes = [P, V, V, V, C.c_float, V, V, V]
        L.velox_frustum_overlap.restype = C.c_int
        L.velox_pool_keys.argtypes = [P, V, V, C.c_int32, C.c_int32, C.c_int32, V]
        L.velox_pool_keys.restype = C.c_int
        L.velox_route_cached.argtypes = [P, V, V, C.c_int32, V, V, V, V, V, V, C.c_size_t, V]
        L.velox_route_cached.restype = C.c_int
        L.velox_select.argtypes = [P, V, V, V, V, V, V]
        L.velox_select.restype = C.c_int
        L.velox_sparse_attn.argtypes = [P, V, V, V, V, V, V, V, V]
        L.velox_sparse_attn.restype = C.c_int
        L.velox_sparse_attn_split_workspace_bytes.argtypes = [P, C.c_int32]
        L.velox_sparse_attn_split_workspace_bytes.restype = C.c_size_t
        L.velox_sparse_attn_auto_splits.argtypes = [P, C.c_int32]
        L.velox_sparse_attn_auto_splits.restype = C.c_int32
        L.velox_sparse_attn_split.argtypes = [P, V, V, V, V, V, C.c_int32, V, V, V, C.c_size_t, V]
        L.velox_sparse_attn_split.restype = C.c_int
        L.velox_status_string.argtypes = [C.c_int]
        L.velox_status_string.restype = C.c_char_p
        L.velox_last_hip_error.argtypes = []
        L.velox_last_hip_error.restype = C.c_int
        _lib = L
    return _lib


def velox_check(p: Problem) -> int:
    return lib().velox_check(C.byref(p))


def velox_route_workspace_bytes(p: Problem) -> int:
    return lib().velox_route_workspace_bytes(C.byref(p))


def velox_sparse_attn_split_workspace_bytes(p: Problem, num_splits: int) -> int:
    return lib().velox_sparse_attn_split_workspace_bytes(C.byref(p), int(num_splits))


def _raise(status: int, where: str):
    if status != Status.OK:
        raise VeloxError(status, where)


# ---------------------------------------------------------------- torch front end

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return VELOX_BF16
    if t.dtype == torch.float32:
        return VELOX_F32
    raise TypeError(f"Q/K/V must be bfloat16 or float32, got {t.dtype}")


def _dev(t, name, dtype=None, ndim=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    return t


def _out(t, name, shape, dtype):
    """A caller-provided output (or workspace) buffer: GPU, contiguous, exact dtype and shape."""
    _dev(t, name, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _workspace(ws, need, device):
    """The caller's workspace if it is a large enough GPU uint8 buffer, else a new one."""
    torch = _torch()
    if ws is None or ws.numel() < need:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _dev(ws, "workspace", torch.uint8, ndim=1)
    return ws


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def problem_for(q_shape, kv_tokens: int, block: int, top_k: int, alpha: float, dtype: int,
                modulation: int = MOD_SCALE) -> Problem:
    """Build a Problem from Q's shape [B,H,T,d] and the KV length N = (C+1)*T."""
    B, H, T, d = q_shape
    if T <= 0 or kv_tokens % T:
        raise ValueError(f"KV length {kv_tokens} is not a whole number of chunks of {T} tokens")
    return Problem(B, H, d, T, kv_tokens // T - 1, block, top_k, float(alpha), dtype, modulation)


def route(q, k, overlap, covered, block: int, top_k: int, alpha: float, return_scores: bool = False,
          out=None, workspace=None, stream=None, modulation: int = MOD_SCALE):
    """velox_route: returns (kv_idx [B,H,nq,top_k] int32, kv_cnt [B,H,nq] int32[, scores fp32])."""
    torch = _torch()
    _dev(q, "q", ndim=4)
    _dev(k, "k", q.dtype, ndim=4)
    p = problem_for(tuple(q.shape), k.shape[2], block, top_k, alpha, _dtype_code(q), modulation)
    _raise(velox_check(p), "velox_route")
    B, H, T, d = q.shape
    if tuple(k.shape) != (B, H, k.shape[2], d):
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    C_ = p.past_chunks
    if C_ > 0:
        _dev(overlap, "overlap", torch.float32)
        if tuple(overlap.shape) != (B, p.nq, C_):
            raise ValueError(f"overlap must be [{B},{p.nq},{C_}], got {tuple(overlap.shape)}")
    else:
        overlap = None
    _dev(covered, "covered", torch.uint8)
    if tuple(covered.shape) != (B, p.nq):
        raise ValueError(f"covered must be [{B},{p.nq}], got {tuple(covered.shape)}")
    if out is None:
        kv_idx = torch.empty((B, H, p.nq, top_k), dtype=torch.int32, device=q.device)
        kv_cnt = torch.empty((B, H, p.nq), dtype=torch.int32, device=q.device)
    else:
        kv_idx = _out(out[0], "kv_idx", (B, H, p.nq, top_k), torch.int32)
        kv_cnt = _out(out[1], "kv_cnt", (B, H, p.nq), torch.int32)
    scores = torch.empty((B, H, p.nq, p.nk), dtype=torch.float32, device=q.device) if return_scores else None
    workspace = _workspace(workspace, velox_route_workspace_bytes(p), q.device)
    st = lib().velox_route(C.byref(p), _ptr(q), _ptr(k), _ptr(overlap), _ptr(covered), _ptr(kv_idx), _ptr(kv_cnt),
                           _ptr(scores), _ptr(workspace), workspace.numel(), _stream(stream))
    _raise(st, "velox_route")
    return (kv_idx, kv_cnt, scores) if return_scores else (kv_idx, kv_cnt)


def route_noalloc(q, k, overlap, covered, block: int, top_k: int, alpha: float, out, scores=None, stream=None,
                  modulation: int = MOD_SCALE):
    """velox_route_noalloc: velox_route with the library's per-GPU scratch array as its
    workspace.  The caller passes the outputs: out = (kv_idx [B,H,nq,top_k] int32,
    kv_cnt [B,H,nq] int32), and optionally scores [B,H,nq,nk] float32; nothing is
    allocated.  Calls that overlap on one GPU race on the scratch array."""
    torch = _torch()
    _dev(q, "q", ndim=4)
    _dev(k, "k", q.dtype, ndim=4)
    p = problem_for(tuple(q.shape), k.shape[2], block, top_k, alpha, _dtype_code(q), modulation)
    _raise(velox_check(p), "velox_route_noalloc")
    B, H, T, d = q.shape
    if tuple(k.shape) != (B, H, k.shape[2], d):
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if p.past_chunks > 0:
        _dev(overlap, "overlap", torch.float32)
        if tuple(overlap.shape) != (B, p.nq, p.past_chunks):
            raise ValueError(f"overlap must be [{B},{p.nq},{p.past_chunks}], got {tuple(overlap.shape)}")
    else:
        overlap = None
    _dev(covered, "covered", torch.uint8)
    if tuple(covered.shape) != (B, p.nq):
        raise ValueError(f"covered must be [{B},{p.nq}], got {tuple(covered.shape)}")
    kv_idx = _out(out[0], "kv_idx", (B, H, p.nq, top_k), torch.int32)
    kv_cnt = _out(out[1], "kv_cnt", (B, H, p.nq), torch.int32)
    if scores is not None:
        scores = _out(scores, "scores", (B, H, p.nq, p.nk), torch.float32)
    st = lib().velox_route_noalloc(C.byref(p), _ptr(q), _ptr(k), _ptr(overlap), _ptr(covered), _ptr(kv_idx),
                                   _ptr(kv_cnt), _ptr(scores), _stream(stream))
    _raise(st, "velox_route_noalloc")
    return kv_idx, kv_cnt


def score(q, k, block: int, scores=None, workspace=None, stream=None):
    """velox_score: raw importance s [B,H,nq,nk] float32 (the scoring step of route)."""
    torch = _torch()
    _dev(q, "q", ndim=4)
    _dev(k, "k", q.dtype, ndim=4)
    B, H, T, d = q.shape
    p = problem_for(tuple(q.shape), k.shape[2], block, T // block, 0.0, _dtype_code(q))
    _raise(velox_check(p), "velox_score")
    if scores is None:
        scores = torch.empty((B, H, p.nq, p.nk), dtype=torch.float32, device=q.device)
    _dev(scores, "scores", torch.float32, ndim=4)
    if tuple(scores.shape) != (B, H, p.nq, p.nk):
        raise ValueError(f"scores must be [{B},{H},{p.nq},{p.nk}]")
    workspace = _workspace(workspace, velox_route_workspace_bytes(p), q.device)
    _raise(lib().velox_score(C.byref(p), _ptr(q), _ptr(k), _ptr(scores), _ptr(workspace), workspace.numel(),
                             _stream(stream)), "velox_score")
    return scores


def frustum_overlap(yaw, past_depth, query_depth, fov_deg: float, out=None, stream=None):
    """velox_frustum_overlap: yaw [B,C+1], past_depth [B,C,2], query_depth [B,nq,2] (float32, GPU)
    -> (overlap [B,nq,C] float32, covered [B,nq] uint8)."""
    torch = _torch()
    _dev(yaw, "yaw", torch.float32, ndim=2)
    _dev(query_depth, "query_depth", torch.float32, ndim=3)
    B, C1 = yaw.shape
    nq = query_depth.shape[1]
    C_ = C1 - 1
    if tuple(query_depth.shape) != (B, nq, 2):
        raise ValueError("query_depth must be [B,nq,2]")
    if C_ > 0:
        _dev(past_depth, "past_depth", torch.float32, ndim=3)
        if tuple(past_depth.shape) != (B, C_, 2):
            raise ValueError("past_depth must be [B,C,2]")
    # the problem only carries the shapes: nq query blocks of 64 tokens, C past chunks
    p = Problem(B, 1, 64, nq * 64, C_, 64, nq, 0.0, VELOX_F32)
    if out is None:
        overlap = torch.empty((B, nq, C_), dtype=torch.float32, device=yaw.device)
        covered = torch.empty((B, nq), dtype=torch.uint8, device=yaw.device)
    else:
        overlap = _out(out[0], "overlap", (B, nq, C_), torch.float32)
        covered = _out(out[1], "covered", (B, nq), torch.uint8)
    st = lib().velox_frustum_overlap(C.byref(p), _ptr(yaw), _ptr(past_depth if C_ > 0 else None),
                                     _ptr(query_depth), float(fov_deg), _ptr(overlap if C_ > 0 else None),
                                     _ptr(covered), _stream(stream))
    _raise(st, "velox_frustum_overlap")
    return overlap, covered


def pool_keys(k, chunk_tokens: int, block: int, first_block: int, num_blocks: int, kbar=None,
              cache_blocks: int | None = None, stream=None):
    """velox_pool_keys: pool KV blocks [first_block, first_block+num_blocks) of k [B,H,N,d] into the
    float32 cache kbar [B,H,cache_blocks,d] (allocated with cache_blocks = N/block rows if not given)."""
    torch = _torch()
    _dev(k, "k", ndim=4)
    B, H, N, d = k.shape
    p = problem_for((B, H, chunk_tokens, d), N, block, 1, 0.0, _dtype_code(k))
    if kbar is None:
        cache_blocks = p.nk if cache_blocks is None else cache_blocks
        kbar = torch.empty((B, H, cache_blocks, d), dtype=torch.float32, device=k.device)
    _dev(kbar, "kbar", torch.float32, ndim=4)
    if tuple(kbar.shape[:2]) != (B, H) or kbar.shape[3] != d:
        raise ValueError(f"kbar shape {tuple(kbar.shape)} does not match k {tuple(k.shape)}")
    st = lib().velox_pool_keys(C.byref(p), _ptr(k), _ptr(kbar), kbar.shape[2], first_block, num_blocks,
                               _stream(stream))
    _raise(st, "velox_pool_keys")
    return kbar


def route_cached(q, kbar, past_chunks: int, overlap, covered, block: int, top_k: int, alpha: float,
                 return_scores: bool = False, out=None, workspace=None, stream=None, modulation: int = MOD_SCALE):
    """velox_route_cached: route from pooled keys kbar [B,H,cache_blocks,d] (float32) instead of K."""
    torch = _torch()
    _dev(q, "q", ndim=4)
    _dev(kbar, "kbar", torch.float32, ndim=4)
    B, H, T, d = q.shape
    p = problem_for(tuple(q.shape), (past_chunks + 1) * T, block, top_k, alpha, _dtype_code(q), modulation)
    _raise(velox_check(p), "velox_route_cached")
    if tuple(kbar.shape[:2]) != (B, H) or kbar.shape[3] != d:
        raise ValueError(f"kbar shape {tuple(kbar.shape)} does not match q {tuple(q.shape)}")
    if past_chunks > 0:
        _dev(overlap, "overlap", torch.float32)
        if tuple(overlap.shape) != (B, p.nq, past_chunks):
            raise ValueError(f"overlap must be [{B},{p.nq},{past_chunks}], got {tuple(overlap.shape)}")
    else:
        overlap = None
    _dev(covered, "covered", torch.uint8)
    if tuple(covered.shape) != (B, p.nq):
        raise ValueError(f"covered must be [{B},{p.nq}], got {tuple(covered.shape)}")
    if out is None:
        kv_idx = torch.empty((B, H, p.nq, top_k), dtype=torch.int32, device=q.device)
        kv_cnt = torch.empty((B, H, p.nq), dtype=torch.int32, device=q.device)
    else:
        kv_idx = _out(out[0], "kv_idx", (B, H, p.nq, top_k), torch.int32)
        kv_cnt = _out(out[1], "kv_cnt", (B, H, p.nq), torch.int32)
    scores = torch.empty((B, H, p.nq, p.nk), dtype=torch.float32, device=q.device) if return_scores else None
    workspace = _workspace(workspace, velox_route_workspace_bytes(p), q.device)
    st = lib().velox_route_cached(C.byref(p), _ptr(q), _ptr(kbar), kbar.shape[2], _ptr(overlap), _ptr(covered),
                                  _ptr(kv_idx), _ptr(kv_cnt), _ptr(scores), _ptr(workspace), workspace.numel(),
                                  _stream(stream))
    _raise(st, "velox_route_cached")
    return (kv_idx, kv_cnt, scores) if return_scores else (kv_idx, kv_cnt)


def select(scores, overlap, covered, block: int, top_k: int, alpha: float, stream=None,
           modulation: int = MOD_SCALE):
    """velox_select: modulation + top-k from given scores [B,H,nq,nk] (float32)."""
    torch = _torch()
    _dev(scores, "scores", torch.float32, ndim=4)
    B, H, nq, nk = scores.shape
    if nk % nq:
        raise ValueError("nk must be a whole number of chunks of nq blocks")
    p = Problem(B, H, 64, nq * block, nk // nq - 1, block, top_k, float(alpha), VELOX_F32, modulation)
    _raise(velox_check(p), "velox_select")
    if p.past_chunks > 0:
        _dev(overlap, "overlap", torch.float32)
        if tuple(overlap.shape) != (B, nq, p.past_chunks):
            raise ValueError("overlap shape mismatch")
    else:
        overlap = None
    _dev(covered, "covered", torch.uint8)
    if tuple(covered.shape) != (B, nq):
        raise ValueError("covered shape mismatch")
    kv_idx = torch.empty((B, H, nq, top_k), dtype=torch.int32, device=scores.device)
    kv_cnt = torch.empty((B, H, nq), dtype=torch.int32, device=scores.device)
    st = lib().velox_select(C.byref(p), _ptr(scores), _ptr(overlap), _ptr(covered), _ptr(kv_idx), _ptr(kv_cnt),
                            _stream(stream))
    _raise(st, "velox_select")
    return kv_idx, kv_cnt


def auto_splits(p: Problem, num_cus: int | None = None) -> int:
    """velox_sparse_attn_auto_splits for the current device's compute-unit count."""
    if num_cus is None:
        num_cus = _torch().cuda.get_device_properties(_torch().cuda.current_device()).multi_processor_count
    return int(lib().velox_sparse_attn_auto_splits(C.byref(p), int(num_cus)))


def sparse_attn(q, k, v, kv_idx, kv_cnt, block: int, return_lse: bool = False, out=None, stream=None,
                splits=None, workspace=None):
    """velox_sparse_attn: returns out [B,H,T,d] (dtype of q)[, lse [B,H,T] float32].

    ``splits``: None = one workgroup per row (velox_sparse_attn); an int or "auto" =
    velox_sparse_attn_split with that many list segments per row."""
    torch = _torch()
    _dev(q, "q", ndim=4)
    _dev(k, "k", q.dtype, ndim=4)
    _dev(v, "v", q.dtype, ndim=4)
    _dev(kv_idx, "kv_idx", torch.int32, ndim=4)
    _dev(kv_cnt, "kv_cnt", torch.int32, ndim=3)
    B, H, T, d = q.shape
    p = problem_for(tuple(q.shape), k.shape[2], block, kv_idx.shape[3], 0.0, _dtype_code(q))
    if tuple(k.shape) != tuple(v.shape) or tuple(k.shape[:2]) != (B, H) or k.shape[3] != d:
        raise ValueError("k/v shape mismatch")
    if tuple(kv_idx.shape[:3]) != (B, H, p.nq) or tuple(kv_cnt.shape) != (B, H, p.nq):
        raise ValueError("kv_idx/kv_cnt shape mismatch")
    o = _out(out, "out", q.shape, q.dtype) if out is not None else torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if return_lse else None
    if splits is None:
        st = lib().velox_sparse_attn(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(kv_idx), _ptr(kv_cnt), _ptr(o),
                                     _ptr(lse), _stream(stream))
        _raise(st, "velox_sparse_attn")
    else:
        n = auto_splits(p) if splits == "auto" else int(splits)
        workspace = _workspace(workspace, velox_sparse_attn_split_workspace_bytes(p, n), q.device)
        st = lib().velox_sparse_attn_split(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(kv_idx), _ptr(kv_cnt), n,
                                           _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream))
        _raise(st, "velox_sparse_attn_split")
    return (o, lse) if return_lse else o
