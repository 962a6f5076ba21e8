"""TEST INFRASTRUCTURE: numpy front end of the CPU oracle (libvelox_oracle.so).

Argument marshalling only; every step is computed by the plain fp64 C code in
velox_oracle.c.  Only the tests, the package smoke check and the benchmark's
CPU-baseline leg may import this module.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libvelox_oracle.so")
_lib = None

_P = C.c_void_p
_I = C.c_int
_L = C.c_int64
_D = C.c_double
_F = C.c_float


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from .build import build_oracle
            build_oracle()
        L = C.CDLL(_LIB_PATH)
        L.velox_oracle_num_threads.restype = _I
        L.velox_oracle_set_threads.argtypes = [_I]
        L.velox_oracle_set_threads.restype = None
        L.velox_oracle_pool.argtypes = [_P, _I, _L, _I, _I, _P]
        L.velox_oracle_scores.argtypes = [_P, _P, _L, _I, _I, _I, _P]
        L.velox_oracle_modulate.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _D, _P]
        L.velox_oracle_modulate_f32.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P]
        L.velox_oracle_frustum_overlap.argtypes = [_P, _P, _P, _D, _I, _I, _I, _P, _P]
        L.velox_oracle_modulate_logprob.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _D, _P]
        L.velox_oracle_modulate_logprob_f32.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P]
        L.velox_oracle_select.argtypes = [_P, _L, _I, _I, _P, _P, _P]
        L.velox_oracle_attn.argtypes = [_P, _P, _P, _I, _I, _I, _I, _L, _I, _I, _P, _P, _I, _L, _P, _P, _P]
        L.velox_oracle_dense_attn.argtypes = [_P, _P, _P, _I, _I, _I, _I, _L, _I, _P, _P]
        for name in ("pool", "scores", "modulate", "modulate_f32", "select", "attn", "dense_attn"):
            getattr(L, "velox_oracle_" + name).restype = _I
        _lib = L
    return _lib


def num_threads() -> int:
    return lib().velox_oracle_num_threads()


def set_threads(n: int) -> None:
    """OpenMP threads for the following oracle calls (timing only; results do not depend on it)."""
    lib().velox_oracle_set_threads(int(n))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError(f"oracle takes float32 or bf16 bit patterns (uint16), got {a.dtype}")


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"velox_oracle_{what} failed with {rc}")


def pool(x: np.ndarray, blk: int) -> np.ndarray:
    """Mean over each group of ``blk`` rows: [..., n*blk, d] -> [..., n, d] (float64)."""
    x = np.ascontiguousarray(x)
    *lead, rows, d = x.shape
    if rows % blk:
        raise ValueError("row count must be a multiple of blk")
    out = np.empty((*lead, rows // blk, d), np.float64)
    nblocks = int(np.prod(lead, dtype=np.int64)) * (rows // blk)
    _check(lib().velox_oracle_pool(_ptr(x), _dtype_code(x), nblocks, blk, d, _ptr(out)), "pool")
    return out


def scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """s[..., i, j] = <qbar_i, kbar_j> / sqrt(d); qbar [...,nq,d], kbar [...,nk,d]."""
    qbar = np.ascontiguousarray(qbar, np.float64)
    kbar = np.ascontiguousarray(kbar, np.float64)
    *lead, nq, d = qbar.shape
    nk = kbar.shape[-2]
    bh = int(np.prod(lead, dtype=np.int64))
    s = np.empty((*lead, nq, nk), np.float64)
    _check(lib().velox_oracle_scores(_ptr(qbar), _ptr(kbar), bh, nq, nk, d, _ptr(s)), "scores")
    return s


def modulate(s: np.ndarray, overlap: np.ndarray, covered: np.ndarray, blk: int, T: int, alpha: float,
             fp32: bool = False, mode: int = 0) -> np.ndarray:
    """Modulated importance m from s [B,H,nq,nk], overlap [B,nq,C], covered [B,nq].

    ``mode`` 0: m = s*(1 + alpha*o); 1 (sign-safe, probability reading): m = s + log1p(alpha*o).
    ``fp32=True`` takes the decision in float32 (s must then be float32)."""
    if mode not in (0, 1):
        raise ValueError(f"unknown modulation mode {mode}")
    B, H, nq, nk = s.shape
    C_ = overlap.shape[-1] if overlap.ndim == 3 else 0
    ov = np.ascontiguousarray(overlap, np.float32)
    cov = np.ascontiguousarray(covered, np.uint8)
    m = np.empty(s.shape, np.float64)
    L = lib()
    if fp32:
        s32 = np.ascontiguousarray(s, np.float32)
        fn = L.velox_oracle_modulate_logprob_f32 if mode == 1 else L.velox_oracle_modulate_f32
        rc = fn(_ptr(s32), _ptr(ov), _ptr(cov), B, H, nq, nk, blk, T, C_, float(np.float32(alpha)), _ptr(m))
    else:
        s64 = np.ascontiguousarray(s, np.float64)
        fn = L.velox_oracle_modulate_logprob if mode == 1 else L.velox_oracle_modulate
        rc = fn(_ptr(s64), _ptr(ov), _ptr(cov), B, H, nq, nk, blk, T, C_, float(alpha), _ptr(m))
    _check(rc, "modulate")
    return m


def frustum_overlap(yaw: np.ndarray, past_depth: np.ndarray, query_depth: np.ndarray, fov: float):
    """Overlap [B,nq,C] (fp64) and covered [B,nq] (uint8) of frustum slices: yaw [B,C+1],
    past_depth [B,C,2], query_depth [B,nq,2] (float32; see velox_oracle_frustum_overlap)."""
    yaw = np.ascontiguousarray(yaw, np.float32)
    pd = np.ascontiguousarray(past_depth, np.float32)
    qd = np.ascontiguousarray(query_depth, np.float32)
    B, C1 = yaw.shape
    nq = qd.shape[1]
    C = C1 - 1
    o = np.empty((B, nq, C), np.float64)
    cov = np.empty((B, nq), np.uint8)
    _check(lib().velox_oracle_frustum_overlap(_ptr(yaw), _ptr(pd), _ptr(qd), float(fov), B, nq, C, _ptr(o),
                                              _ptr(cov)), "frustum_overlap")
    return o, cov


def select(m: np.ndarray, k: int):
    """Top-k per row under (m desc, index asc); returns kv_idx [...,k], kv_cnt [...], kth [...]."""
    m = np.ascontiguousarray(m, np.float64)
    *lead, nk = m.shape
    rows = int(np.prod(lead, dtype=np.int64))
    kv_idx = np.empty((*lead, k), np.int32)
    kv_cnt = np.empty(tuple(lead), np.int32)
    kth = np.empty(tuple(lead), np.float64)
    _check(lib().velox_oracle_select(_ptr(m), rows, nk, k, _ptr(kv_idx), _ptr(kv_cnt), _ptr(kth)), "select")
    return kv_idx, kv_cnt, kth


def route(q: np.ndarray, k: np.ndarray, overlap: np.ndarray, covered: np.ndarray, blk: int, top_k: int,
          alpha: float, mode: int = 0) -> dict:
    """Pool, score, modulate (``mode`` as in modulate) and select for q [B,H,T,d], k [B,H,N,d]."""
    T = q.shape[2]
    qbar = pool(q, blk)
    kbar = pool(k, blk)
    s = scores(qbar, kbar)
    m = modulate(s, overlap, covered, blk, T, alpha, mode=mode)
    kv_idx, kv_cnt, kth = select(m, top_k)
    return dict(qbar=qbar, kbar=kbar, s=s, m=m, kv_idx=kv_idx, kv_cnt=kv_cnt, kth=kth)


def attn(q: np.ndarray, k: np.ndarray, v: np.ndarray, kv_idx: np.ndarray, kv_cnt: np.ndarray, blk: int,
         tokens: Optional[np.ndarray] = None):
    """Attention of query tokens over their row's kept blocks.

    q [B,H,T,d]; k, v [B,H,N,d]; kv_idx [B,H,nq,kmax]; kv_cnt [B,H,nq].
    ``tokens``: optional flat indices (b*H + h)*T + t; returns (out [n,d], lse [n]),
    or (out [B,H,T,d], lse [B,H,T]) for all tokens."""
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    B, H, T, d = q.shape
    N = k.shape[2]
    kv_idx = np.ascontiguousarray(kv_idx, np.int32)
    kv_cnt = np.ascontiguousarray(kv_cnt, np.int32)
    kmax = kv_idx.shape[-1]
    if tokens is None:
        ntok, tok = B * H * T, None
    else:
        tok = np.ascontiguousarray(tokens, np.int64)
        ntok = tok.size
    out = np.empty((ntok, d), np.float64)
    lse = np.empty(ntok, np.float64)
    _check(lib().velox_oracle_attn(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, T, N, d, blk,
                                   _ptr(kv_idx), _ptr(kv_cnt), kmax, ntok, _ptr(tok), _ptr(out), _ptr(lse)),
           "attn")
    if tokens is None:
        return out.reshape(B, H, T, d), lse.reshape(B, H, T)
    return out, lse


def dense_attn(q: np.ndarray, k: np.ndarray, v: np.ndarray):
    """Brute-force dense softmax attention over all keys: (out [B,H,T,d], lse [B,H,T])."""
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    B, H, T, d = q.shape
    N = k.shape[2]
    out = np.empty((B, H, T, d), np.float64)
    lse = np.empty((B, H, T), np.float64)
    _check(lib().velox_oracle_dense_attn(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, T, N, d,
                                         _ptr(out), _ptr(lse)), "dense_attn")
    return out, lse
