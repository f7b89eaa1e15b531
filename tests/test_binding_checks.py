"""The Python binding checks every tensor's dtype and shape before the C ABI
sees a pointer (CPU only).

The library takes bare device pointers and sizes, so a wrong shape that got
through would become out-of-bounds device accesses.  Each case below passes
CPU tensors with one thing wrong and expects a TypeError that names it; with
every shape right, the first error is the device check.  Either way the
library is never called: a context of None would fail if it were.
"""
import numpy as np
import pytest
import torch

import decode_attention_mla_amd as mla

bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32


def z(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def decode_args(B=2, s_q=1, H=16, cap=64, paged=False):
    a = dict(q=z((B, s_q, H, 576), bf), seqlens=z((B,), i32), scale=1 / 24,
             out=z((B, s_q, H, 512), f32), lse=z((B, s_q, H), f32))
    if paged:
        a.update(kv_cache=z((9, 16, 576), bf), block_table=z((B, 4), i32))
    else:
        a.update(kv_cache=z((B, cap, 576), bf), block_table=None)
    return a


def call_decode(a, **kw):
    a = dict(a)
    a.update(kw)
    return mla.mla_decode(None, a.pop("q"), a.pop("kv_cache"), a.pop("block_table"), a.pop("seqlens"),
                          a.pop("scale"), **a)


@pytest.mark.parametrize("paged", [False, True])
def test_right_shapes_reach_the_device_check(paged):
    with pytest.raises(TypeError, match="must be a CUDA tensor"):
        call_decode(decode_args(paged=paged))


@pytest.mark.parametrize("change,needle", [
    (dict(q=z((2, 1, 16, 512), bf)), "q must have shape"),
    (dict(q=z((2, 1, 16, 576), f32)), "q must be torch.bfloat16"),
    (dict(q=z((2, 16, 576), bf)), "q must have shape"),
    (dict(out=z((2, 1, 16, 576), f32)), "out must have shape"),
    (dict(out=z((3, 1, 16, 512), f32)), "out must have shape"),
    (dict(out=z((2, 1, 16, 512), bf)), "out must be torch.float32"),
    (dict(lse=z((2, 16), f32)), "lse must have shape"),
    (dict(seqlens=z((1,), i32)), "seqlens has 1 entries"),
    (dict(seqlens=z((2,), torch.int64)), "seqlens must be torch.int32"),
    (dict(kv_cache=z((2, 64, 512), bf)), "kv_cache must have shape"),
    (dict(kv_cache=z((1, 64, 576), bf)), "need 128"),
    (dict(kv_capacity=65), "kv_capacity 65 outside"),
    (dict(kv_capacity=0), "kv_capacity 0 outside"),
    (dict(seqlens_host=np.array([5], np.int32)), "seqlens_host has 1 entries"),
    (dict(out=z((2, 1, 16, 1024), f32)[..., ::2]), "out must be contiguous"),
])
def test_contiguous_decode_rejects(change, needle):
    with pytest.raises(TypeError, match=needle):
        call_decode(decode_args(), **change)


def test_smaller_capacity_fits_fewer_rows():
    # kv_capacity below the allocated rows is a valid stride: checked only
    # against what the cache holds
    with pytest.raises(TypeError, match="must be a CUDA tensor"):
        call_decode(decode_args(cap=64), kv_capacity=32)


@pytest.mark.parametrize("change,needle", [
    (dict(block_table=z((1, 4), i32)), "block_table has 1 rows"),
    (dict(block_table=z((2, 4), torch.int64)), "block_table must be torch.int32"),
    (dict(block_table=z((8,), i32)), "block_table must have 2 dimensions"),
    (dict(kv_cache=z((9, 16, 288), bf)), "kv_cache must have shape"),
    (dict(kv_capacity=16), "kv_capacity applies to the contiguous layout only"),
])
def test_paged_decode_rejects(change, needle):
    with pytest.raises(TypeError, match=needle):
        call_decode(decode_args(paged=True), **change)


def test_append_checks():
    rows, kv, lens = z((2, 1, 576), bf), z((2, 64, 576), bf), z((2,), i32)
    with pytest.raises(TypeError, match="must be a CUDA tensor"):
        mla.mla_append_kv(None, rows, kv, None, lens)
    with pytest.raises(TypeError, match="new_rows must have shape"):
        mla.mla_append_kv(None, z((2, 1, 512), bf), kv, None, lens)
    with pytest.raises(TypeError, match="need 192"):
        mla.mla_append_kv(None, z((3, 1, 576), bf), kv, None, z((3,), i32))
    with pytest.raises(TypeError, match="seqlens has 2 entries"):
        mla.mla_append_kv(None, z((3, 1, 576), bf), z((3, 64, 576), bf), None, lens)
    with pytest.raises(TypeError, match="block_table has 2 rows"):
        mla.mla_append_kv(None, z((3, 1, 576), bf), z((9, 16, 576), bf), z((2, 4), i32), z((3,), i32))


def test_absorb_and_project_checks():
    qn, qr, w = z((4, 16, 128), bf), z((4, 16, 64), bf), z((16, 512, 128), bf)
    with pytest.raises(TypeError, match="must be a CUDA tensor"):
        mla.mla_absorb_q(None, qn, qr, w)
    with pytest.raises(TypeError, match="q_rope must have shape"):
        mla.mla_absorb_q(None, qn, z((4, 16, 32), bf), w)
    with pytest.raises(TypeError, match="q_nope must have shape"):
        mla.mla_absorb_q(None, z((4, 8, 128), bf), qr, w)
    with pytest.raises(TypeError, match="w_uk must have shape"):
        mla.mla_absorb_q(None, qn, qr, z((16, 576, 128), bf))
    with pytest.raises(TypeError, match="q_out must have shape"):
        mla.mla_absorb_q(None, qn, qr, w, q_out=z((5, 16, 576), bf))
    o, wv = z((4, 16, 512), f32), z((16, 128, 512), bf)
    with pytest.raises(TypeError, match="must be a CUDA tensor"):
        mla.mla_project_out(None, o, wv)
    with pytest.raises(TypeError, match="o must have shape"):
        mla.mla_project_out(None, z((4, 8, 512), f32), wv)
    with pytest.raises(TypeError, match="w_uv must have shape"):
        mla.mla_project_out(None, o, z((16, 128, 576), bf))
    with pytest.raises(TypeError, match="out must have shape"):
        mla.mla_project_out(None, o, wv, out=z((4, 16, 64), f32))


class _OnDevice:
    """Stand-in for a tensor or a stream: only its device is read."""

    def __init__(self, dev):
        self.device = torch.device(dev)


def test_tensors_must_sit_on_the_launch_stream_device():
    # The check itself, with stand-ins (this host has no GPU): tensors of one
    # GPU launched on another GPU's stream are refused, as are mixed GPUs.
    with pytest.raises(TypeError, match="the stream the kernels run on is on cuda:1"):
        mla._on_one_device(_OnDevice("cuda:1"), q=_OnDevice("cuda:0"), out=_OnDevice("cuda:0"))
    with pytest.raises(TypeError, match="out is on cuda:1"):
        mla._on_one_device(_OnDevice("cuda:0"), q=_OnDevice("cuda:0"), out=_OnDevice("cuda:1"))
    mla._on_one_device(_OnDevice("cuda:0"), q=_OnDevice("cuda:0"), lse=None)
    mla._on_one_device(None, q=_OnDevice("cuda:1"))
