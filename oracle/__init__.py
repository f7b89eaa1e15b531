"""fp64 CPU oracle for MLA decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and the
oracle imports nothing from it.

The arithmetic lives in ``mla_oracle.c`` (plain C, double precision, OpenMP
over rows); this file builds it with gcc and marshals numpy arrays through
ctypes.  What it computes and the readings it takes are stated in the C file's
header ("FlashMLA-ETAP", gist.science technical summary, Methodology).

Parity status: pinned.  ``tests/test_oracle.py`` checks it against closed
forms, exact special cases, invariances, an independent 50-digit brute force
on tiny shapes and a large-N distributional law.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "_build", "liboracle.so")
# A test may point the loader at another build of the same source (a copy
# with a planted mistake) to show that the pins reject it.
_LIB_OVERRIDE = os.environ.get("MLA_ORACLE_LIB")
_lib = None


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    tmp = _LIB + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
         "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB
        if _LIB_OVERRIDE is None and not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        lib.oracle_mla_decode.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                          i64, i32, i32, f32, P, P, P, i64]
        lib.oracle_mla_decode.restype = i32
        lib.oracle_mla_decode_transposed.argtypes = [P, P, P, P, i32, i32, i32, i32, i32,
                                                     i64, i32, i32, f32, P, P]
        lib.oracle_mla_decode_transposed.restype = i32
        lib.oracle_lse_combine.argtypes = [i32, i64, i32, P, P, P, P]
        lib.oracle_lse_combine.restype = i32
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _prep(q, kv, block_table, seqlens):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kv = np.ascontiguousarray(kv, dtype=np.uint16)
    seqlens = np.ascontiguousarray(seqlens, dtype=np.int32)
    B, s_q, H, d_qk = q.shape
    if block_table is None:
        cap, page_size, max_pages = kv.shape[1], 0, 0
    else:
        block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        cap, page_size, max_pages = 0, kv.shape[1], block_table.shape[1]
    return q, kv, block_table, seqlens, (B, s_q, H, d_qk), (cap, page_size, max_pages)


def mla_decode(q, kv, block_table, seqlens, scale, d_v=512, window=None,
               return_probs=False, threads: Optional[int] = None):
    """Attention in the standard order S = QK^T, P = softmax(S), O = PV.

    q: [B, s_q, H, 576] bf16 bits; kv: contiguous [B, cap, 576] or paged pool
    [P, page, 576]; block_table: None or [B, max_pages]; seqlens: [B].
    window: optional (begin[B], end[B]) key windows.  Returns (O, LSE) as
    float64 arrays [B, s_q, H, d_v] and [B, s_q, H] (and P if asked).
    """
    lib = _load()
    q, kv, block_table, seqlens, (B, s_q, H, d_qk), (cap, ps, mp) = _prep(
        q, kv, block_table, seqlens)
    out = np.empty((B, s_q, H, d_v), dtype=np.float64)
    lse = np.empty((B, s_q, H), dtype=np.float64)
    wb = we = None
    if window is not None:
        wb = np.ascontiguousarray(window[0], dtype=np.int32)
        we = np.ascontiguousarray(window[1], dtype=np.int32)
    probs, stride = None, 0
    if return_probs:
        stride = int(seqlens.max()) if B else 0
        probs = np.empty((B, s_q, H, stride), dtype=np.float64)
    _set_threads(threads)
    rc = lib.oracle_mla_decode(_ptr(q), _ptr(kv), _ptr(block_table), _ptr(seqlens),
                               _ptr(wb), _ptr(we), B, s_q, H, d_qk, d_v, cap, ps, mp,
                               float(scale), _ptr(out), _ptr(lse), _ptr(probs), stride)
    if rc != 0:
        raise ValueError("oracle_mla_decode rejected its arguments")
    return (out, lse, probs) if return_probs else (out, lse)


def mla_decode_transposed(q, kv, block_table, seqlens, scale, d_v=512,
                          threads: Optional[int] = None):
    """The same attention in the transposed order S^T = KQ^T, P^T, O = (V^T P^T)^T."""
    lib = _load()
    q, kv, block_table, seqlens, (B, s_q, H, d_qk), (cap, ps, mp) = _prep(
        q, kv, block_table, seqlens)
    out = np.empty((B, s_q, H, d_v), dtype=np.float64)
    lse = np.empty((B, s_q, H), dtype=np.float64)
    _set_threads(threads)
    rc = lib.oracle_mla_decode_transposed(_ptr(q), _ptr(kv), _ptr(block_table),
                                          _ptr(seqlens), B, s_q, H, d_qk, d_v, cap,
                                          ps, mp, float(scale), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_mla_decode_transposed rejected its arguments")
    return out, lse


def lse_combine(lse_parts: np.ndarray, o_parts: np.ndarray):
    """Exact merge of per-part (O_s, lse_s); shapes [n, ...] and [n, ..., d_v]."""
    lib = _load()
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    n = lse_parts.shape[0]
    rows = int(np.prod(lse_parts.shape[1:]))
    d_v = o_parts.shape[-1]
    lse = np.empty(lse_parts.shape[1:], dtype=np.float64)
    out = np.empty(o_parts.shape[1:], dtype=np.float64)
    rc = lib.oracle_lse_combine(n, rows, d_v, _ptr(lse_parts), _ptr(o_parts),
                                _ptr(lse), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_lse_combine rejected its arguments")
    return out, lse


def _set_threads(threads: Optional[int]) -> None:
    if threads is None:
        return
    try:
        omp = ctypes.CDLL("libgomp.so.1")
        omp.omp_set_num_threads(int(threads))
    except OSError:
        pass
