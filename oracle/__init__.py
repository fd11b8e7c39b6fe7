"""Python access to the CPU oracle (oracle/liboracle.so).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's
CPU-baseline leg import this package; the HIP library and its binding never
do. The oracle shares no code with the HIP path.

This module only marshals numpy arrays into the C functions of
``moe_oracle.c``; all arithmetic is there. bf16 arrays are passed as raw
``uint16`` bit patterns (dtype 0), fp32 as ``float32`` (dtype 1).
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB_OVERRIDE lets the mutation test load a deliberately broken copy.
_LIB_PATH = os.environ.get("ORACLE_LIB_OVERRIDE") or os.path.join(_HERE, "liboracle.so")
_lib = None

_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = C.CDLL(_LIB_PATH)
    lib.oracle_route.restype = C.c_int64
    lib.oracle_route.argtypes = [C.c_int64, C.c_int32, C.c_int64, C.c_int32, _i64p,
                                 _i32p, _i32p, _i32p, _i32p, _i32p]
    lib.oracle_route_padded.restype = C.c_int64
    lib.oracle_route_padded.argtypes = [C.c_int64, C.c_int32, C.c_int64, C.c_int32, C.c_int32,
                                        _i32p, _i64p, _i32p, _i32p, _i32p, _i32p, _i32p]
    lib.oracle_compact_rows.restype = C.c_int64
    lib.oracle_compact_rows.argtypes = [C.c_int64, C.c_int32, _i32p, C.c_int64, C.c_void_p,
                                        C.c_void_p, C.c_int32]
    lib.oracle_expand.restype = None
    lib.oracle_expand.argtypes = [C.c_int64, C.c_int64, C.c_int32, C.c_void_p, _i32p, C.c_void_p]
    lib.oracle_expert_mlp.restype = None
    lib.oracle_expert_mlp.argtypes = [C.c_int64, C.c_int64, C.c_int32, C.c_void_p, C.c_void_p,
                                      C.c_void_p, _f64p]
    lib.oracle_expert_rows.restype = None
    lib.oracle_expert_rows.argtypes = [C.c_int64, _i32p, _i64p, C.c_int64, C.c_int64, C.c_int32,
                                       C.c_void_p, C.c_void_p, C.c_void_p, _f64p, C.c_int32]
    lib.oracle_combine.restype = None
    lib.oracle_combine.argtypes = [C.c_int64, C.c_int32, C.c_int64, C.c_int32, _i32p,
                                   C.c_void_p, C.c_void_p, _f64p]
    lib.oracle_combine_epilogue.restype = None
    lib.oracle_combine_epilogue.argtypes = [C.c_int64, C.c_int32, C.c_int64, C.c_int32, _i32p,
                                            C.c_void_p, _f64p]
    lib.oracle_forward.restype = None
    lib.oracle_forward.argtypes = [C.c_int64, C.c_int32, C.c_int64, C.c_int32, C.c_int64,
                                   C.c_int64, C.c_int32, C.c_void_p, _i64p, C.c_void_p,
                                   C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, _f64p,
                                   C.c_int32]
    lib.oracle_silu.restype = C.c_double
    lib.oracle_silu.argtypes = [C.c_double]
    lib.oracle_threads.restype = C.c_int32
    lib.oracle_threads.argtypes = [C.c_int32]
    _lib = lib
    return lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 0
    if a.dtype == np.float32:
        return 1
    raise TypeError(f"oracle takes bf16 bits (uint16) or float32, got {a.dtype}")


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def threads(nthreads: int = 0) -> int:
    return int(_load().oracle_threads(nthreads))


def silu(z: float) -> float:
    return float(_load().oracle_silu(float(z)))


def route(idx: np.ndarray, E: int, expert_begin: int = 0, block_rows: int = 0,
          block_counts: Optional[np.ndarray] = None):
    """Returns dict(counts, offsets, row_map [T,K], row_src [R], row_k [R], R).

    block_rows > 0: a padded buffer whose block j carries queries in its
    first block_counts[j] rows only (SGLang PR #6092)."""
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    T, K = idx.shape
    if block_rows:
        bc = np.ascontiguousarray(block_counts, dtype=np.int32)
        assert bc.shape == (-(-T // block_rows),)
    else:
        bc = np.zeros(1, np.int32)
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    row_map = np.zeros(T * K, np.int32)
    cap = max(T * K, 1)
    row_src = np.full(cap, -1, np.int32)
    row_k = np.full(cap, -1, np.int32)
    R = _load().oracle_route_padded(T, K, expert_begin, E, int(block_rows), bc, idx.reshape(-1),
                                    counts, offsets, row_map, row_src, row_k)
    return dict(counts=counts, offsets=offsets, row_map=row_map.reshape(T, K),
                row_src=row_src[:R].copy(), row_k=row_k[:R].copy(), R=int(R))


def compact_rows(src: np.ndarray, block_rows: int, block_counts: np.ndarray,
                 to_padded: bool = False, dst: Optional[np.ndarray] = None):
    """Carrying rows of a padded buffer in compact order (to_padded False:
    returns (compact array of n rows, n)), or compact rows written back into a
    copy of the padded dst (to_padded True: returns (that copy, n))."""
    src = np.ascontiguousarray(src)
    bc = np.ascontiguousarray(block_counts, dtype=np.int32)
    if to_padded:
        out = np.array(dst, copy=True, order="C")
        T = out.shape[0]
    else:
        T = src.shape[0]
        out = np.zeros_like(src)
    row_bytes = int(np.prod(src.shape[1:], dtype=np.int64)) * src.itemsize
    assert bc.shape == (-(-T // block_rows),) and out.dtype == src.dtype
    n = _load().oracle_compact_rows(T, int(block_rows), bc, row_bytes,
                                    src.ctypes.data_as(C.c_void_p),
                                    out.ctypes.data_as(C.c_void_p), 1 if to_padded else 0)
    return (out, int(n)) if to_padded else (out[:n].copy(), int(n))


def expand(x: np.ndarray, row_src: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    _dtype_code(x)
    row_src = np.ascontiguousarray(row_src, dtype=np.int32)
    R, H = row_src.shape[0], x.shape[1]
    Xe = np.empty((R, H), dtype=x.dtype)
    _load().oracle_expand(R, H, x.itemsize, _ptr(x), row_src, _ptr(Xe))
    return Xe


def expert_mlp(w1e: np.ndarray, w2e: np.ndarray, xrow: np.ndarray) -> np.ndarray:
    w1e, w2e, xrow = (np.ascontiguousarray(a) for a in (w1e, w2e, xrow))
    dt = _dtype_code(xrow)
    assert w1e.dtype == xrow.dtype and w2e.dtype == xrow.dtype
    H = xrow.shape[-1]
    I = w1e.shape[0] // 2
    assert w1e.shape == (2 * I, H) and w2e.shape == (H, I)
    out = np.empty(H, np.float64)
    _load().oracle_expert_mlp(H, I, dt, _ptr(w1e), _ptr(w2e), _ptr(xrow), out)
    return out


def expert_rows(experts, tokens, x, w1, w2, nthreads: int = 0) -> np.ndarray:
    """out[i] = MLP_{experts[i]}(x[tokens[i]]) in double."""
    experts = np.ascontiguousarray(experts, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    x, w1, w2 = (np.ascontiguousarray(a) for a in (x, w1, w2))
    dt = _dtype_code(x)
    E, I2, H = w1.shape
    I = I2 // 2
    assert w2.shape == (E, H, I) and x.shape[1] == H
    n = experts.shape[0]
    assert tokens.shape[0] == n
    if n:
        assert 0 <= experts.min() and experts.max() < E
        assert 0 <= tokens.min() and tokens.max() < x.shape[0]
    out = np.empty((n, H), np.float64)
    _load().oracle_expert_rows(n, experts, tokens, H, I, dt, _ptr(x), _ptr(w1), _ptr(w2), out,
                               nthreads)
    return out


def combine(row_map: np.ndarray, weights: Optional[np.ndarray], O: np.ndarray) -> np.ndarray:
    row_map = np.ascontiguousarray(row_map, dtype=np.int32)
    T, K = row_map.shape
    O = np.ascontiguousarray(O)
    dt = _dtype_code(O)
    H = O.shape[1]
    if row_map.size and row_map.max() >= O.shape[0]:
        raise ValueError("row_map points past the expert-output rows")
    w = None if weights is None else np.ascontiguousarray(weights, dtype=np.float32)
    y = np.empty((T, H), np.float64)
    _load().oracle_combine(T, K, H, dt, row_map.reshape(-1), _ptr(w), _ptr(O), y)
    return y


def combine_epilogue(src: np.ndarray, recv: np.ndarray) -> np.ndarray:
    """Cross-rank epilogue: y[t] = sum over j of recv[src[t][j]] (src >= 0), double."""
    src = np.ascontiguousarray(src, dtype=np.int32)
    T, J = src.shape
    recv = np.ascontiguousarray(recv)
    dt = _dtype_code(recv)
    H = recv.shape[1]
    if src.size and src.max() >= recv.shape[0]:
        raise ValueError("src points past the received rows")
    y = np.empty((T, H), np.float64)
    _load().oracle_combine_epilogue(T, J, H, dt, src.reshape(-1), _ptr(recv), y)
    return y


def forward(x, idx, weights, w1, w2, E: int, expert_begin: int = 0, tokens=None,
            nthreads: int = 0) -> np.ndarray:
    """Whole layer for the listed tokens (default all), double [n, H]."""
    x, w1, w2 = (np.ascontiguousarray(a) for a in (x, w1, w2))
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    dt = _dtype_code(x)
    T, K = idx.shape
    H = x.shape[1]
    assert w1.shape[0] == E and w1.shape[2] == H
    I = w1.shape[1] // 2
    assert w2.shape == (E, H, I)
    w = None if weights is None else np.ascontiguousarray(weights, dtype=np.float32)
    tk = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    n = T if tk is None else tk.shape[0]
    y = np.empty((n, H), np.float64)
    _load().oracle_forward(T, K, expert_begin, E, H, I, dt, _ptr(x), idx.reshape(-1), _ptr(w),
                           _ptr(w1), _ptr(w2), _ptr(tk), n, y, nthreads)
    return y
