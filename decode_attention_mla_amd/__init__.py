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
MLA_OPT_NUM_SPLITS, MLA_OPT_MIN_CHUNK, MLA_OPT_KERNEL_TIMING, MLA_OPT_P_BF16 = 1, 2, 3, 4


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
                ("active_groups", ctypes.c_int32), ("split_sequences", ctypes.c_int32),
                ("seq_gap", ctypes.c_int64)]


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
    lib.mla_workspace_size.argtypes = [P, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.mla_ctx_set_workspace.argtypes = [P, P, ctypes.c_size_t]
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
    lib.mla_decode_noalloc.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, ctypes.POINTER(Problem)]
    lib.mla_noalloc_scratch_bytes.argtypes = []
    lib.mla_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.mla_version.restype = ctypes.c_char_p
    for name in ("mla_ctx_create", "mla_ctx_destroy", "mla_ctx_reserve", "mla_ctx_set_option",
                 "mla_workspace_size", "mla_ctx_set_workspace", "mla_decode_noalloc",
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
                     active_groups=info.active_groups, split_sequences=info.split_sequences,
                     seq_gap=info.seq_gap)


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
        self.workspace = None  # a caller's workspace tensor, kept alive while set

    def reserve(self, s_q: int, num_heads: int) -> None:
        _check(load().mla_ctx_reserve(self.handle, s_q, num_heads), self.handle)

    def workspace_size(self, s_q: int, num_heads: int) -> int:
        """Bytes of device workspace mla_decode needs for up to s_q tokens and
        num_heads heads (with the current split option)."""
        n = ctypes.c_size_t(0)
        _check(load().mla_workspace_size(self.handle, s_q, num_heads, ctypes.byref(n)))
        return n.value

    def set_workspace(self, buf) -> None:
        """Use `buf` (a CUDA tensor on the context's device, 256-byte
        aligned) as the split workspace; None returns to a workspace the
        library allocates.  The tensor is kept alive while it is set."""
        if buf is None:
            _check(load().mla_ctx_set_workspace(self.handle, None, 0), self.handle)
            self.workspace = None
            return
        if not buf.is_contiguous() or buf.device.type != "cuda":
            raise TypeError("the workspace must be a contiguous CUDA tensor")
        nbytes = buf.numel() * buf.element_size()
        _check(load().mla_ctx_set_workspace(self.handle, buf.data_ptr(), nbytes), self.handle)
        self.workspace = buf

    def allocate_workspace(self, s_q: int, num_heads: int):
        """Allocate the workspace for up to s_q tokens and num_heads heads as
        a torch tensor on the current device, set it, and return it."""
        import torch

        buf = torch.empty(self.workspace_size(s_q, num_heads), dtype=torch.uint8, device="cuda")
        self.set_workspace(buf)
        return buf

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


def _need(name, t, dtype, shape=None, ndim=None):
    """dtype, dense layout and shape of one tensor argument (None in `shape`
    matches any size).  Checked before anything reaches the library: the C
    ABI takes bare pointers, so these are the only bounds checks a wrong
    shape meets."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, is {t.dtype}")
    if not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise TypeError(f"{name} must have {ndim} dimensions, has {t.dim()}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(d) != w for d, w in zip(t.shape, shape)):
            want = "[" + ", ".join("*" if w is None else str(w) for w in shape) + "]"
            raise TypeError(f"{name} must have shape {want}, has {list(t.shape)}")


def _on_one_device(stream, **tensors):
    """Every tensor on the same GPU as the stream the kernels are launched on
    (checked after the shapes): the library takes the pointers as they come,
    so a tensor of another GPU would be read on the wrong device."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise TypeError(f"{name} must be a CUDA tensor (is on {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise TypeError(f"{name} is on {t.device}, the other tensors on {dev}")
    if stream is not None and dev is not None and stream.device != dev:
        raise TypeError(f"the tensors are on {dev}, the stream the kernels run on is on {stream.device}")


def _stream_of(ctx):
    """The stream a context launches on (None without a context)."""
    return getattr(ctx, "stream", None)


def _cache_layout(kv_cache, block_table, batch, kv_capacity):
    """(page_size, kv_capacity, num_pages, max_pages) of a contiguous cache
    [B', cap, 576] (B' >= batch) or a paged pool [P, page, 576] with a block
    table [B', max_pages] (B' >= batch), checked against the batch."""
    import torch

    _need("kv_cache", kv_cache, torch.bfloat16, (None, None, HEAD_DIM_QK))
    if block_table is None:
        cap = int(kv_cache.shape[1]) if kv_capacity is None else int(kv_capacity)
        if cap < 1 or cap > kv_cache.shape[1]:
            raise TypeError(f"kv_capacity {cap} outside [1, {kv_cache.shape[1]}] (rows of kv_cache)")
        if batch * cap * HEAD_DIM_QK > kv_cache.numel():
            raise TypeError(f"kv_cache holds {kv_cache.numel() // HEAD_DIM_QK} rows, "
                            f"{batch} sequences of capacity {cap} need {batch * cap}")
        return 0, cap, 0, 0
    if kv_capacity is not None:
        raise TypeError("kv_capacity applies to the contiguous layout only")
    _need("block_table", block_table, torch.int32, ndim=2)
    if block_table.shape[0] < batch:
        raise TypeError(f"block_table has {block_table.shape[0]} rows for {batch} sequences")
    return int(kv_cache.shape[1]), 0, int(kv_cache.shape[0]), int(block_table.shape[1])


def _host_lengths(seqlens_host, batch):
    if seqlens_host is None:
        return None
    h = np.ascontiguousarray(seqlens_host, dtype=np.int32).reshape(-1)
    if h.shape[0] < batch:
        raise TypeError(f"seqlens_host has {h.shape[0]} entries for {batch} sequences")
    return h[:batch]


def mla_decode(ctx: Context, q, kv_cache, block_table, seqlens, scale: float, out=None, lse=None,
               seqlens_host: Optional[np.ndarray] = None, kv_capacity: Optional[int] = None):
    """Run mla_decode on torch tensors (device memory on ctx's device).

    q [B, s_q, H, 576] bf16; kv_cache contiguous [B', cap, 576] (B' >= B) or
    paged pool [P, page, 576] bf16; block_table None or [B', max_pages]
    int32; seqlens [>= B] int32 on the device; out [B, s_q, H, 512] fp32 and
    lse [B, s_q, H] fp32 are allocated when not given.  kv_capacity
    (contiguous only) overrides the per-sequence row stride, at most
    kv_cache.shape[1].  Returns (out, lse).  Every shape is checked before
    the call: a mismatch raises TypeError and launches nothing.
    """
    import torch

    _need("q", q, torch.bfloat16, (None, None, None, HEAD_DIM_QK))
    B, s_q, H, dqk = (int(x) for x in q.shape)
    page_size, cap, num_pages, max_pages = _cache_layout(kv_cache, block_table, B, kv_capacity)
    _need("seqlens", seqlens, torch.int32, ndim=1)
    if seqlens.shape[0] < B:
        raise TypeError(f"seqlens has {seqlens.shape[0]} entries for {B} sequences")
    host = _host_lengths(seqlens_host, B)
    if out is not None:
        _need("out", out, torch.float32, (B, s_q, H, HEAD_DIM_V))
    if lse is not None:
        _need("lse", lse, torch.float32, (B, s_q, H))
    _on_one_device(_stream_of(ctx), q=q, kv_cache=kv_cache, block_table=block_table, seqlens=seqlens,
                   out=out, lse=lse)
    if out is None:
        out = torch.empty((B, s_q, H, HEAD_DIM_V), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, s_q, H), dtype=torch.float32, device=q.device)
    pr, keep = make_problem(B, s_q, H, page_size, cap, num_pages, max_pages, host)
    pr.head_dim_qk = dqk
    bt_ptr = None if block_table is None else block_table.data_ptr()
    rc = load().mla_decode(ctx.handle, q.data_ptr(), kv_cache.data_ptr(), bt_ptr,
                           seqlens.data_ptr(), float(scale), out.data_ptr(), lse.data_ptr(),
                           ctypes.byref(pr))
    del keep
    _check(rc, ctx.handle)
    return out, lse


def mla_decode_noalloc(q, kv_cache, block_table, seqlens, scale: float, out, lse,
                       seqlens_host: Optional[np.ndarray] = None, kv_capacity: Optional[int] = None,
                       stream=None):
    """mla_decode without a context and without any allocation: the split
    partials go to the library's static scratch array.  out and lse must be
    given (shapes as for ``mla_decode``), on the current device; `stream`
    defaults to torch's current stream.  Returns (out, lse)."""
    import torch

    _need("q", q, torch.bfloat16, (None, None, None, HEAD_DIM_QK))
    B, s_q, H, dqk = (int(x) for x in q.shape)
    page_size, cap, num_pages, max_pages = _cache_layout(kv_cache, block_table, B, kv_capacity)
    _need("seqlens", seqlens, torch.int32, ndim=1)
    if seqlens.shape[0] < B:
        raise TypeError(f"seqlens has {seqlens.shape[0]} entries for {B} sequences")
    host = _host_lengths(seqlens_host, B)
    if out is None or lse is None:
        raise TypeError("mla_decode_noalloc writes into the caller's out and lse: pass both")
    _need("out", out, torch.float32, (B, s_q, H, HEAD_DIM_V))
    _need("lse", lse, torch.float32, (B, s_q, H))
    _on_one_device(stream, q=q, kv_cache=kv_cache, block_table=block_table, seqlens=seqlens, out=out,
                   lse=lse)
    # The library takes the scratch array of the current device.
    if q.device.index != torch.cuda.current_device():
        raise TypeError(f"the tensors are on {q.device}, the current device is "
                        f"cuda:{torch.cuda.current_device()}")
    if stream is None:
        stream = torch.cuda.current_stream()
    pr, keep = make_problem(B, s_q, H, page_size, cap, num_pages, max_pages, host)
    pr.head_dim_qk = dqk
    bt_ptr = None if block_table is None else block_table.data_ptr()
    rc = load().mla_decode_noalloc(ctypes.c_void_p(stream.cuda_stream), q.data_ptr(), kv_cache.data_ptr(),
                                   bt_ptr, seqlens.data_ptr(), float(scale), out.data_ptr(), lse.data_ptr(),
                                   ctypes.byref(pr))
    del keep
    _check(rc)
    return out, lse


def noalloc_scratch_bytes() -> int:
    return int(load().mla_noalloc_scratch_bytes())


def mla_append_kv(ctx: Context, new_rows, kv_cache, block_table, seqlens,
                  seqlens_host: Optional[np.ndarray] = None, kv_capacity: Optional[int] = None):
    """Write the latent rows of the new tokens into the cache, in place.

    new_rows [B, s_q, 576] bf16; kv_cache, block_table and seqlens as for
    ``mla_decode`` (seqlens are the lengths including the new tokens).
    Returns kv_cache.  Shapes are checked as for ``mla_decode``.
    """
    import torch

    _need("new_rows", new_rows, torch.bfloat16, (None, None, HEAD_DIM_QK))
    B, s_q, dqk = (int(x) for x in new_rows.shape)
    page_size, cap, num_pages, max_pages = _cache_layout(kv_cache, block_table, B, kv_capacity)
    _need("seqlens", seqlens, torch.int32, ndim=1)
    if seqlens.shape[0] < B:
        raise TypeError(f"seqlens has {seqlens.shape[0]} entries for {B} sequences")
    host = _host_lengths(seqlens_host, B)
    _on_one_device(_stream_of(ctx), new_rows=new_rows, kv_cache=kv_cache, block_table=block_table,
                   seqlens=seqlens)
    pr, keep = make_problem(B, s_q, 1, page_size, cap, num_pages, max_pages, host)
    pr.head_dim_qk = dqk
    bt_ptr = None if block_table is None else block_table.data_ptr()
    rc = load().mla_append_kv(ctx.handle, new_rows.data_ptr(), kv_cache.data_ptr(), bt_ptr,
                              seqlens.data_ptr(), ctypes.byref(pr))
    del keep
    _check(rc, ctx.handle)
    return kv_cache


def mla_absorb_q(ctx: Context, q_nope, q_rope, w_uk, q_out=None):
    """Absorbed query [..., H, 576] bf16 from q_nope [..., H, d_nope],
    q_rope [..., H, 64] (bf16) and w_uk [H, 512, d_nope] bf16."""
    import torch

    _need("w_uk", w_uk, torch.bfloat16, (None, HEAD_DIM_V, None))
    H, lat, d_nope = (int(x) for x in w_uk.shape)
    _need("q_nope", q_nope, torch.bfloat16)
    lead = tuple(int(x) for x in q_nope.shape[:-2])
    _need("q_nope", q_nope, torch.bfloat16, (*lead, H, d_nope))
    _need("q_rope", q_rope, torch.bfloat16, (*lead, H, HEAD_DIM_QK - HEAD_DIM_V))
    rows = int(np.prod(lead)) if len(lead) else 1
    if q_out is not None:
        _need("q_out", q_out, torch.bfloat16, (*lead, H, HEAD_DIM_QK))
    _on_one_device(_stream_of(ctx), q_nope=q_nope, q_rope=q_rope, w_uk=w_uk, q_out=q_out)
    if q_out is None:
        q_out = torch.empty((*lead, H, HEAD_DIM_QK), dtype=torch.bfloat16, device=q_nope.device)
    _check(load().mla_absorb_q(ctx.handle, q_nope.data_ptr(), q_rope.data_ptr(), w_uk.data_ptr(),
                               q_out.data_ptr(), rows, H, d_nope), ctx.handle)
    return q_out


def mla_project_out(ctx: Context, o, w_uv, out=None):
    """Output up-projection [..., H, d_v] fp32 from the latent attention
    output o [..., H, 512] fp32 and w_uv [H, d_v, 512] bf16."""
    import torch

    _need("w_uv", w_uv, torch.bfloat16, (None, None, HEAD_DIM_V))
    H, d_v, lat = (int(x) for x in w_uv.shape)
    _need("o", o, torch.float32)
    lead = tuple(int(x) for x in o.shape[:-2])
    _need("o", o, torch.float32, (*lead, H, lat))
    rows = int(np.prod(lead)) if len(lead) else 1
    if out is not None:
        _need("out", out, torch.float32, (*lead, H, d_v))
    _on_one_device(_stream_of(ctx), o=o, w_uv=w_uv, out=out)
    if out is None:
        out = torch.empty((*lead, H, d_v), dtype=torch.float32, device=o.device)
    _check(load().mla_project_out(ctx.handle, o.data_ptr(), w_uv.data_ptr(), out.data_ptr(),
                                  rows, H, d_v), ctx.handle)
    return out
