"""Python access to the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
bench's CPU-baseline leg, never by the library.  It takes the workload's raw
host arrays (the same bytes the GPU reads) and returns fp64 results.

``build()`` compiles ``liboracle.so`` with gcc (-O2, OpenMP).  ``load()``
compiles only if no library is present.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    _lib = declare(ctypes.CDLL(_LIB))
    return _lib


def declare(lib):
    """Attach argument/return types to a loaded oracle library."""
    P = ctypes.c_void_p
    i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_paged_attn.restype = i32
    lib.oracle_paged_attn.argtypes = [P, i32, dbl, P, i32, i32, P, P, i32, P, P, i32, i32, i32, i32,
                                      dbl, dbl, P, P, P, i32, i32, i32, dbl, i32, P, i64, P, P,
                                      P, i32]
    lib.oracle_merge_states.restype = i32
    lib.oracle_merge_states.argtypes = [P, P, i32, i64, i32, P, P]
    lib.oracle_decode.restype = None
    lib.oracle_decode.argtypes = [P, i32, i64, P]
    lib.oracle_num_threads.restype = i32
    lib.oracle_num_threads.argtypes = []
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def decode(codes: np.ndarray, dtype: int) -> np.ndarray:
    """Oracle's own decoding of raw storage codes to fp64."""
    codes = np.ascontiguousarray(codes)
    out = np.empty(codes.size, dtype=np.float64)
    load().oracle_decode(_ptr(codes), dtype, codes.size, _ptr(out))
    return out.reshape(codes.shape)


def attention(w, rows: Optional[Sequence[int]] = None, num_kv_splits: Optional[int] = None,
              num_threads: int = 0, causal: Optional[bool] = None):
    """Run the oracle on workload ``w`` (``workloads.Workload``).

    Returns (O, LSE, MAX) in fp64.  Without ``rows``: O is
    [S, total_q, Hq, Dvo] and LSE/MAX are [S, total_q, Hq]; with ``rows``
    (ids t*Hq + h): O is [S, len(rows), Dvo], LSE/MAX [S, len(rows)].
    S = num_kv_splits (default: the workload's).  The leading S axis is
    dropped when S == 1.
    """
    lib = load()
    S = w.num_kv_splits if num_kv_splits is None else num_kv_splits
    caus = w.causal if causal is None else causal
    q = np.ascontiguousarray(w.q)
    k = np.ascontiguousarray(w.k)
    v = k if w.v is None else np.ascontiguousarray(w.v)
    ks = np.asarray(w.k_stride, dtype=np.int64)
    vs = np.asarray(w.v_stride, dtype=np.int64)
    qo = np.ascontiguousarray(w.qo_indptr, dtype=np.int32)
    ip = np.ascontiguousarray(w.kv_indptr, dtype=np.int32)
    ix = np.ascontiguousarray(w.kv_indices, dtype=np.int32)
    if ix.size == 0:
        ix = np.zeros(1, dtype=np.int32)
    lp = np.ascontiguousarray(w.kv_last_page_len, dtype=np.int32)
    if rows is None:
        nrows = w.total_q * w.num_qo_heads
        rws = None
    else:
        rws = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rws.size
    o = np.empty((S, nrows, w.head_dim_vo), dtype=np.float64)
    lse = np.empty((S, nrows), dtype=np.float64)
    mx = np.empty((S, nrows), dtype=np.float64)
    rc = lib.oracle_paged_attn(_ptr(q), w.q_dtype, w.q_scale, _ptr(qo), w.batch, w.num_qo_heads, _ptr(k),
                               _ptr(v), w.kv_dtype, _ptr(ks), _ptr(vs), w.num_kv_heads,
                               w.page_size, w.head_dim_qk, w.head_dim_vo, w.k_scale, w.v_scale,
                               _ptr(ip), _ptr(ix), _ptr(lp), w.num_kv_batches,
                               int(w.kv_broadcast), int(caus), w.sm_scale, S, _ptr(rws),
                               nrows, _ptr(o), _ptr(lse), _ptr(mx), num_threads)
    if rc != 0:
        raise ValueError(f"oracle rejected the arguments (rc={rc})")
    if rows is None:
        o = o.reshape(S, w.total_q, w.num_qo_heads, w.head_dim_vo)
        lse = lse.reshape(S, w.total_q, w.num_qo_heads)
        mx = mx.reshape(S, w.total_q, w.num_qo_heads)
    if S == 1:
        return o[0], lse[0], mx[0]
    return o, lse, mx


def merge_states(v: np.ndarray, s: np.ndarray):
    """v [S, rows, D], s [S, rows] (natural-log LSE) -> (v_out [rows, D], s_out [rows])."""
    lib = load()
    v = np.ascontiguousarray(v, dtype=np.float64)
    s = np.ascontiguousarray(s, dtype=np.float64)
    S, rows, D = v.shape
    vo = np.empty((rows, D), dtype=np.float64)
    so = np.empty(rows, dtype=np.float64)
    rc = lib.oracle_merge_states(_ptr(v), _ptr(s), S, rows, D, _ptr(vo), _ptr(so))
    if rc != 0:
        raise ValueError(f"oracle merge rejected the arguments (rc={rc})")
    return vo, so


def num_threads() -> int:
    return int(load().oracle_num_threads())
