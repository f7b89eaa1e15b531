"""Python binding of the gfx950 MLA decode library (``include/mla_decode.h``).

Argument marshalling only: every step of the attention runs in the HIP
kernels of ``libmla_decode.so``.  PyTorch supplies device memory and the
stream.  There is no fallback: when the library is missing, every call raises.

    import torch, decode_attention_mla_amd as mla
    ctx = mla.Context()                       # bound to torch's current stream
    out, lse = mla.mla_decode(ctx, q, kv_cache, block_table, seqlens, scale,
                              seqlens_host=seqlens_cpu)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_lib", "libmla_decode.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "mla_decode.h")

HEAD_DIM_QK = 576
HEAD_DIM_V = 512
KEY_BLOCK = 16

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = 0, -1, -2, -3, -4
MLA_OPT_NUM_SPLITS, MLA_OPT_MIN_CHUNK, MLA_OPT_KERNEL_TIMING = 1, 2, 3


class MlaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mla_decode error {code}: {msg}")
        self.code = code


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("s_q", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("kv_capacity", ctypes.c_int64),
        ("num_pages", ctypes.c_int64),
        ("max_pages", ctypes.c_int32),
        ("seqlens_host", ctypes.POINTER(ctypes.c_int32)),
    ]


class PlanSegment(ctypes.Structure):
    _fields_ = [("group", ctypes.c_int32), ("seq", ctypes.c_int32),
                ("key_begin", ctypes.c_int32), ("key_end", ctypes.c_int32),
                ("slot", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int64), ("total_keys", ctypes.c_int64),
                ("active_groups", ctypes.c_int32), ("split_sequences", ctypes.c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libmla_decode.so (built by ``decode_attention_mla_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m decode_attention_mla_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.mla_ctx_create.argtypes = [ctypes.POINTER(P), P]
    lib.mla_ctx_destroy.argtypes = [P]
    lib.mla_ctx_reserve.argtypes = [P, i32, i32]
    lib.mla_ctx_set_option.argtypes = [P, ctypes.c_int, i64]
    lib.mla_last_error.argtypes = [P]
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_decode.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, ctypes.POINTER(Problem)]
    lib.mla_validate.argtypes = [P, P, P, P, ctypes.c_float, P, P, ctypes.POINTER(Problem)]
    lib.mla_plan.argtypes = [P, i32, i32, i64, ctypes.POINTER(PlanSegment), i32,
                             ctypes.POINTER(i32), ctypes.POINTER(PlanInfo)]
    lib.mla_ctx_kernel_times.argtypes = [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64),
                                         ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    lib.mla_append_kv.argtypes = [P, P, P, P, P, ctypes.POINTER(Problem)]
    lib.mla_absorb_q.argtypes = [P, P, P, P, P, i32, i32, i32]
    lib.mla_project_out.argtypes = [P, P, P, P, i32, i32, i32]
    lib.mla_version.restype = ctypes.c_char_p
    for name in ("mla_ctx_create", "mla_ctx_destroy", "mla_ctx_reserve", "mla_ctx_set_option",
                 "mla_decode", "mla_validate", "mla_plan", "mla_ctx_kernel_times",
                 "mla_append_kv", "mla_absorb_q", "mla_project_out"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def last_error(ctx_handle=None) -> str:
    return load().mla_last_error(ctx_handle).decode()


def _check(rc: int, handle=None) -> None:
    if rc != MLA_OK:
        raise MlaError(rc, last_error(handle))


def version() -> str:
    return load().mla_version().decode()


def make_problem(batch, s_q, num_heads, page_size=0, kv_capacity=0, num_pages=0, max_pages=0,
                 seqlens_host: Optional[np.ndarray] = None):
    """Fill an mla_problem; returns (struct, keep-alive array or None)."""
    pr = Problem(batch, s_q, num_heads, HEAD_DIM_QK, HEAD_DIM_V, page_size, kv_capacity,
                 num_pages, max_pages, None)
    keep = None
    if seqlens_host is not None:
        keep = np.ascontiguousarray(seqlens_host, dtype=np.int32)
        pr.seqlens_host = keep.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    return pr, keep


def mla_plan(seqlens: Sequence[int], num_splits: int, min_chunk: int = 64):
    """Host mirror of the device split plan: (segments as dicts, info dict)."""
    lib = load()
    lens = np.ascontiguousarray(seqlens, dtype=np.int32)
    n = ctypes.c_int32(0)
    info = PlanInfo()
    _check(lib.mla_plan(lens.ctypes.data, len(lens), num_splits, min_chunk, None, 0,
                        ctypes.byref(n), ctypes.byref(info)))
    segs = (PlanSegment * max(1, n.value))()
    _check(lib.mla_plan(lens.ctypes.data, len(lens), num_splits, min_chunk, segs, n.value,
                        ctypes.byref(n), ctypes.byref(info)))
    out = [dict(group=s.group, seq=s.seq, key_begin=s.key_begin, key_end=s.key_end, slot=s.slot)
           for s in segs[: n.value]]
    return out, dict(chunk=info.chunk, total_keys=info.total_keys,
                     active_groups=info.active_groups, split_sequences=info.split_sequences)


class Context:
    """An mla_ctx bound to a HIP stream (default: torch's current stream)."""

    def __init__(self, stream=None):
        import torch

        lib = load()
        if stream is None:
            stream = torch.cuda.current_stream()
        self.stream = stream
        handle = ctypes.c_void_p()
        _check(lib.mla_ctx_create(ctypes.byref(handle), ctypes.c_void_p(stream.cuda_stream)))
        self.handle = handle

    def reserve(self, s_q: int, num_heads: int) -> None:
        _check(load().mla_ctx_reserve(self.handle, s_q, num_heads), self.handle)

    def set_option(self, option: int, value: int) -> None:
        _check(load().mla_ctx_set_option(self.handle, option, value), self.handle)

    def kernel_times(self):
        """(split_ms_total, split_launches, combine_ms_total, combine_launches)
        since the last query; synchronizes the stream."""
        sm, cm = ctypes.c_double(), ctypes.c_double()
        sn, cn = ctypes.c_int64(), ctypes.c_int64()
        _check(load().mla_ctx_kernel_times(self.handle, ctypes.byref(sm), ctypes.byref(sn),
                                           ctypes.byref(cm), ctypes.byref(cn)), self.handle)
        return sm.value, sn.value, cm.value, cn.value

    def close(self) -> None:
        if self.handle is not None and self.handle.value:
            load().mla_ctx_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def mla_decode(ctx: Context, q, kv_cache, block_table, seqlens, scale: float, out=None, lse=None,
               seqlens_host: Optional[np.ndarray] = None, kv_capacity: Optional[int] = None):
    """Run mla_decode on torch tensors (device memory on ctx's device).

    q [B, s_q, H, 576] bf16; kv_cache contiguous [B, cap, 576] or paged pool
    [P, page, 576] bf16; block_table None or [B, max_pages] int32; seqlens
    [B] int32 on the device; out [B, s_q, H, 512] fp32 and lse [B, s_q, H]
    fp32 are allocated when not given.  Returns (out, lse).
    """
    import torch

    B, s_q, H, dqk = q.shape
    if out is None:
        out = torch.empty((B, s_q, H, HEAD_DIM_V), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, s_q, H), dtype=torch.float32, device=q.device)
    for name, t, dt in (("q", q, torch.bfloat16), ("kv_cache", kv_cache, torch.bfloat16),
                        ("seqlens", seqlens, torch.int32), ("out", out, torch.float32),
                        ("lse", lse, torch.float32)):
        if t.dtype != dt or not t.is_contiguous() or t.device.type != "cuda":
            raise TypeError(f"{name} must be a contiguous {dt} CUDA tensor")
    if block_table is None:
        page_size, num_pages, max_pages = 0, 0, 0
        cap = kv_cache.shape[1] if kv_capacity is None else kv_capacity
        bt_ptr = None
    else:
        if block_table.dtype != torch.int32 or not block_table.is_contiguous():
            raise TypeError("block_table must be a contiguous int32 CUDA tensor")
        page_size, num_pages, max_pages = kv_cache.shape[1], kv_cache.shape[0], block_table.shape[1]
        cap = 0
        bt_ptr = block_table.data_ptr()
    pr, keep = make_problem(B, s_q, H, page_size, cap, num_pages, max_pages, seqlens_host)
    pr.head_dim_qk = dqk
    rc = load().mla_decode(ctx.handle, q.data_ptr(), kv_cache.data_ptr(), bt_ptr,
                           seqlens.data_ptr(), float(scale), out.data_ptr(), lse.data_ptr(),
                           ctypes.byref(pr))
    del keep
    _check(rc, ctx.handle)
    return out, lse


def _need(name, t, dtype, ndim=None):
    import torch

    if t.dtype != dtype or not t.is_contiguous() or t.device.type != "cuda":
        raise TypeError(f"{name} must be a contiguous {dtype} CUDA tensor")
    if ndim is not None and t.dim() != ndim:
        raise TypeError(f"{name} must have {ndim} dimensions, has {t.dim()}")


def mla_append_kv(ctx: Context, new_rows, kv_cache, block_table, seqlens,
                  seqlens_host: Optional[np.ndarray] = None, kv_capacity: Optional[int] = None):
    """Write the latent rows of the new tokens into the cache, in place.

    new_rows [B, s_q, 576] bf16; kv_cache, block_table and seqlens as for
    ``mla_decode`` (seqlens are the lengths including the new tokens).
    Returns kv_cache.
    """
    import torch

    _need("new_rows", new_rows, torch.bfloat16, 3)
    _need("kv_cache", kv_cache, torch.bfloat16, 3)
    _need("seqlens", seqlens, torch.int32, 1)
    B, s_q, dqk = new_rows.shape
    if block_table is None:
        page_size, num_pages, max_pages, bt_ptr = 0, 0, 0, None
        cap = kv_cache.shape[1] if kv_capacity is None else kv_capacity
    else:
        _need("block_table", block_table, torch.int32, 2)
        page_size, num_pages, max_pages = kv_cache.shape[1], kv_cache.shape[0], block_table.shape[1]
        cap, bt_ptr = 0, block_table.data_ptr()
    pr, keep = make_problem(B, s_q, 1, page_size, cap, num_pages, max_pages, seqlens_host)
    pr.head_dim_qk = dqk
    rc = load().mla_append_kv(ctx.handle, new_rows.data_ptr(), kv_cache.data_ptr(), bt_ptr,
                              seqlens.data_ptr(), ctypes.byref(pr))
    del keep
    _check(rc, ctx.handle)
    return kv_cache


def mla_absorb_q(ctx: Context, q_nope, q_rope, w_uk, q_out=None):
    """Absorbed query [..., H, 576] bf16 from q_nope [..., H, d_nope],
    q_rope [..., H, 64] (bf16) and w_uk [H, 512, d_nope] bf16."""
    import torch

    _need("q_nope", q_nope, torch.bfloat16)
    _need("q_rope", q_rope, torch.bfloat16)
    _need("w_uk", w_uk, torch.bfloat16, 3)
    H, lat, d_nope = w_uk.shape
    lead = q_nope.shape[:-2]
    if q_nope.shape[-2:] != (H, d_nope) or q_rope.shape != (*lead, H, HEAD_DIM_QK - HEAD_DIM_V):
        raise TypeError("q_nope / q_rope shapes do not match w_uk")
    rows = int(np.prod(lead)) if len(lead) else 1
    if q_out is None:
        q_out = torch.empty((*lead, H, HEAD_DIM_QK), dtype=torch.bfloat16, device=q_nope.device)
    _need("q_out", q_out, torch.bfloat16)
    if q_out.numel() != rows * H * HEAD_DIM_QK:
        raise TypeError("q_out has the wrong size")
    _check(load().mla_absorb_q(ctx.handle, q_nope.data_ptr(), q_rope.data_ptr(), w_uk.data_ptr(),
                               q_out.data_ptr(), rows, H, d_nope), ctx.handle)
    return q_out


def mla_project_out(ctx: Context, o, w_uv, out=None):
    """Output up-projection [..., H, d_v] fp32 from the latent attention
    output o [..., H, 512] fp32 and w_uv [H, d_v, 512] bf16."""
    import torch

    _need("o", o, torch.float32)
    _need("w_uv", w_uv, torch.bfloat16, 3)
    H, d_v, lat = w_uv.shape
    lead = o.shape[:-2]
    if o.shape[-2:] != (H, lat):
        raise TypeError("o shape does not match w_uv")
    rows = int(np.prod(lead)) if len(lead) else 1
    if out is None:
        out = torch.empty((*lead, H, d_v), dtype=torch.float32, device=o.device)
    _need("out", out, torch.float32)
    if out.numel() != rows * H * d_v:
        raise TypeError("out has the wrong size")
    _check(load().mla_project_out(ctx.handle, o.data_ptr(), w_uv.data_ptr(), out.data_ptr(),
                                  rows, H, d_v), ctx.handle)
    return out
