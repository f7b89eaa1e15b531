"""GPU parity of the MLA steps around the attention (cache append, absorbed
query, output up-projection) against the fp64 oracle in ``oracle/steps.py``,
through the C ABI, plus one whole decode step (absorb, append, attend,
project) against the oracle's chain of the same steps.

Bars:
* append: bit-exact, every byte of the cache (untouched slots included);
* absorb: the rotary part bit-exact; each latent channel is the bf16 rounding
  of a value within the fp32 accumulation bound d_nope 2^-24 sum|q w| of
  the exact sum (so it differs from the oracle's rounding only next to a
  rounding midpoint, by one bf16 place);
* project: |out - exact| <= 2^-16 sum|o w| per element (the hi/lo split of
  o keeps ~17 bits, the fp32 accumulation adds less), and RMSE <= 1e-4,
  max-abs <= 1e-3 as for the attention output;
* decode step: the projected output within RMSE 1e-4 and max-abs 1e-3.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from oracle import steps

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    import torch

    import decode_attention_mla_amd as mla

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    c = mla.Context()
    yield c
    c.close()


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def bits_of(t):
    import torch

    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# ---------------------------------------------------------------- checks

def check_absorb(q_bits_gpu, si):
    q_lat, q_bits = steps.absorb_q(si.q_nope, si.q_rope, si.w_uk)
    d_nope = si.q_nope.shape[-1]
    assert np.array_equal(q_bits_gpu[..., 512:], q_bits[..., 512:]), "rotary part not copied"
    mag = np.einsum("rhd,hcd->rhc", np.abs(steps.bf16_bits_to_f64(si.q_nope)),
                    np.abs(steps.bf16_bits_to_f64(si.w_uk)))
    e = d_nope * 2.0 ** -24 * mag
    lo = steps.bf16_bits_to_f64(steps.f64_to_bf16_bits(q_lat - e))
    hi = steps.bf16_bits_to_f64(steps.f64_to_bf16_bits(q_lat + e))
    g = steps.bf16_bits_to_f64(q_bits_gpu[..., :512])
    bad = ~((lo <= g) & (g <= hi))
    assert not bad.any(), f"{int(bad.sum())} latent channels outside the rounding bound"
    diff = q_bits_gpu[..., :512] != q_bits[..., :512]
    assert diff.mean() < 1e-3, f"{diff.mean():.2e} of the channels round differently"


def check_project(out_gpu, o, w_uv):
    ref = steps.project_out(o, w_uv)
    mag = steps.project_out_abs(o, w_uv)
    err = np.abs(out_gpu.astype(np.float64) - ref)
    assert np.isfinite(out_gpu).all()
    bad = err > 2.0 ** -16 * mag
    assert not bad.any(), f"{int(bad.sum())} outputs past 2^-16 sum|o w| (worst {err.max():.3g})"
    assert float(np.sqrt(np.mean(err ** 2))) <= 1e-4 and float(err.max()) <= 1e-3


# ---------------------------------------------------------------- absorb

ABSORB = [
    # (rows, H, d_nope)
    (1, 16, 128),
    (16, 16, 128),
    (17, 16, 128),
    (128, 16, 128),
    (3, 1, 32),
    (33, 5, 64),
    (64, 128, 128),
    (2, 16, 512),
    (100, 2, 96),      # two 64-row groups, the second ragged
    (32, 4, 160),
]


@pytest.mark.parametrize("case", range(len(ABSORB)))
def test_absorb_q(ctx, case):
    import torch

    import decode_attention_mla_amd as mla

    rows, H, dn = ABSORB[case]
    announce(f"absorb rows={rows} H={H} d_nope={dn}")
    si = wl.make_step_inputs(200 + case, rows, 1, H, d_nope=dn)
    q_out = torch.full((rows, H, 576), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    mla.mla_absorb_q(ctx, wl.bf16_tensor(si.q_nope), wl.bf16_tensor(si.q_rope),
                     wl.bf16_tensor(si.w_uk), q_out=q_out)
    check_absorb(bits_of(q_out), si)


def test_absorb_q_keeps_neighbouring_rows(ctx):
    """Rows past the last one are not written (the launch covers 16-row tiles)."""
    import torch

    import decode_attention_mla_amd as mla

    announce("absorb tail rows untouched")
    si = wl.make_step_inputs(220, 5, 1, 16)
    q_out = torch.full((16, 16, 576), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    mla.mla_absorb_q(ctx, wl.bf16_tensor(si.q_nope), wl.bf16_tensor(si.q_rope),
                     wl.bf16_tensor(si.w_uk), q_out=q_out[:5])
    got = bits_of(q_out)
    check_absorb(got[:5], si)
    assert np.all(got[5:] == 0x7FC0)


# ---------------------------------------------------------------- project

PROJECT = [
    # (rows, H, d_v)
    (1, 16, 128),
    (16, 16, 128),
    (17, 16, 128),
    (128, 16, 128),
    (3, 1, 64),
    (33, 5, 192),
    (64, 128, 128),
    (2, 16, 512),
    (5, 3, 16),
    (40, 2, 48),
    (100, 4, 32),
    (32, 2, 128),
]


@pytest.mark.parametrize("case", range(len(PROJECT)))
def test_project_out(ctx, case):
    import torch

    import decode_attention_mla_amd as mla

    rows, H, dv = PROJECT[case]
    announce(f"project rows={rows} H={H} d_v={dv}")
    si = wl.make_step_inputs(300 + case, rows, 1, H, d_v=dv)
    o = torch.from_numpy(si.o).to("cuda:0")
    out = torch.full((rows, H, dv), float("nan"), dtype=torch.float32, device="cuda:0")
    mla.mla_project_out(ctx, o, wl.bf16_tensor(si.w_uv), out=out)
    torch.cuda.synchronize()
    check_project(out.cpu().numpy(), si.o, si.w_uv)


def test_project_out_exact_cases(ctx):
    """Outputs the arithmetic fixes exactly: one-hot rows of o pick a weight
    column, and values with at most 16 significant bits survive the hi/lo
    split, so an identity weight returns them unchanged."""
    import torch

    import decode_attention_mla_amd as mla

    announce("project exact cases")
    H, dv = 2, 128
    si = wl.make_step_inputs(330, 1, 1, H, d_v=dv)
    o = np.zeros((64, H, 512), np.float32)
    chans = np.arange(64) * 8 + 3
    o[np.arange(64), :, chans] = 1.0
    out = mla.mla_project_out(ctx, torch.from_numpy(o).to("cuda:0"), wl.bf16_tensor(si.w_uv))
    torch.cuda.synchronize()
    want = steps.bf16_bits_to_f64(si.w_uv)[:, :, chans].transpose(2, 0, 1)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), want)
    eye = np.zeros((H, dv, 512), np.uint16)
    eye[:, np.arange(dv), np.arange(dv)] = 0x3F80
    x = np.random.default_rng(331).standard_normal((7, H, 512)).astype(np.float32)
    x = (x.view(np.uint32) & np.uint32(0xFFFF8000)).view(np.float32)  # 16 significant bits
    out = mla.mla_project_out(ctx, torch.from_numpy(x).to("cuda:0"), wl.bf16_tensor(eye))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), x[..., :dv])


# ---------------------------------------------------------------- append

APPEND = [
    # (lens, s_q, page_size, capacity)
    ([1], 1, 0, None),
    ([5, 64, 33], 1, 0, 80),
    ([5, 64, 33], 3, 0, None),
    ([16, 17, 31, 32, 33], 2, 16, None),   # new tokens across page boundaries
    ([200, 7, 64], 4, 64, None),
    ([4, 4], 4, 16, None),                 # the whole sequence is new
    ([129, 1000, 3], 1, 64, 1024),         # a sequence that fills its pages
]


def cache_case(case, lens, s_q, ps, cap):
    """A poisoned cache holding the old keys: the slots the append fills are
    NaN before it runs."""
    B = len(lens)
    w = wl.Workload("append", B, s_q, 16, int(max(lens)), ps, 400 + case)
    inp = wl.make_inputs(w, poison=True, seqlens=lens, capacity=cap)
    kv = inp.kv.copy()
    for b, L in enumerate(lens):
        for key in range(L - s_q, L):
            if inp.block_table is None:
                kv[b, key] = wl.BF16_NAN
            else:
                kv[inp.block_table[b, key // ps], key % ps] = wl.BF16_NAN
    return inp, kv


@pytest.mark.parametrize("host_lens", [True, False])
@pytest.mark.parametrize("case", range(len(APPEND)))
def test_append_kv(ctx, case, host_lens):
    import torch

    import decode_attention_mla_amd as mla

    lens, s_q, ps, cap = APPEND[case]
    announce(f"append lens={lens} s_q={s_q} page={ps} cap={cap} host_lens={host_lens}")
    inp, kv = cache_case(case, lens, s_q, ps, cap)
    si = wl.make_step_inputs(410 + case, len(lens), s_q, 1)
    kv_d = wl.bf16_tensor(kv)
    bt = None if inp.block_table is None else torch.from_numpy(inp.block_table).to("cuda:0")
    mla.mla_append_kv(ctx, wl.bf16_tensor(si.new_rows), kv_d, bt,
                      torch.from_numpy(inp.seqlens).to("cuda:0"),
                      seqlens_host=inp.seqlens if host_lens else None)
    got = bits_of(kv_d)
    want = steps.append_kv(kv, inp.block_table, inp.seqlens, si.new_rows)
    assert np.array_equal(got, want)


def test_append_clamps_device_lengths(ctx):
    """Without host lengths nothing is checked on the host: a device length
    past the capacity is clamped to it (the last s_q keys are written)."""
    import torch

    import decode_attention_mla_amd as mla

    announce("append clamp")
    inp, kv = cache_case(40, [10, 64], 2, 0, 64)
    si = wl.make_step_inputs(440, 2, 2, 1)
    kv_d = wl.bf16_tensor(kv)
    lens_dev = torch.tensor([10, 1000], dtype=torch.int32, device="cuda:0")
    mla.mla_append_kv(ctx, wl.bf16_tensor(si.new_rows), kv_d, None, lens_dev)
    want = steps.append_kv(kv, None, np.array([10, 64]), si.new_rows)
    assert np.array_equal(bits_of(kv_d), want)


def test_step_errors(ctx):
    import ctypes

    import torch

    import decode_attention_mla_amd as mla

    announce("step argument errors")
    lib = mla.load()
    si = wl.make_step_inputs(450, 2, 1, 16)
    qn, qr, wk = (wl.bf16_tensor(a) for a in (si.q_nope, si.q_rope, si.w_uk))
    q_out = torch.empty((2, 16, 576), dtype=torch.bfloat16, device="cuda:0")
    P = ctypes.c_void_p
    rc = lib.mla_absorb_q(ctx.handle, qn.data_ptr(), qr.data_ptr(), wk.data_ptr(), q_out.data_ptr(), 2, 16, 48)
    assert rc == mla.MLA_ERR_UNSUPPORTED and "d_nope" in mla.last_error(ctx.handle)
    rc = lib.mla_absorb_q(ctx.handle, qn.data_ptr() + 2, qr.data_ptr(), wk.data_ptr(), q_out.data_ptr(), 2, 16, 128)
    assert rc == mla.MLA_ERR_INVALID_ARG and "aligned" in mla.last_error(ctx.handle)
    rc = lib.mla_absorb_q(ctx.handle, None, qr.data_ptr(), wk.data_ptr(), q_out.data_ptr(), 2, 16, 128)
    assert rc == mla.MLA_ERR_INVALID_ARG
    rc = lib.mla_absorb_q(None, qn.data_ptr(), qr.data_ptr(), wk.data_ptr(), q_out.data_ptr(), 2, 16, 128)
    assert rc == mla.MLA_ERR_INVALID_ARG
    o = torch.zeros((2, 16, 512), dtype=torch.float32, device="cuda:0")
    wv = wl.bf16_tensor(si.w_uv)
    out = torch.empty((2, 16, 128), dtype=torch.float32, device="cuda:0")
    rc = lib.mla_project_out(ctx.handle, o.data_ptr(), wv.data_ptr(), out.data_ptr(), 2, 16, 100)
    assert rc == mla.MLA_ERR_UNSUPPORTED and "d_v" in mla.last_error(ctx.handle)
    rc = lib.mla_project_out(ctx.handle, o.data_ptr(), wv.data_ptr(), out.data_ptr(), 0, 16, 128)
    assert rc == mla.MLA_ERR_INVALID_ARG
    kv = torch.zeros((2, 8, 576), dtype=torch.bfloat16, device="cuda:0")
    rows = wl.bf16_tensor(si.new_rows)
    lens = torch.tensor([3, 9], dtype=torch.int32, device="cuda:0")
    with pytest.raises(mla.MlaError, match="seqlens\\[1\\]"):
        mla.mla_append_kv(ctx, rows, kv, None, lens, seqlens_host=np.array([3, 9], np.int32))
    with pytest.raises(mla.MlaError, match="block_table"):
        pr, keep = mla.make_problem(2, 1, 16, 16, 0, 4, 2, None)
        mla._check(lib.mla_append_kv(ctx.handle, rows.data_ptr(), kv.data_ptr(), None, lens.data_ptr(),
                                     ctypes.byref(pr)), ctx.handle)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- whole decode step

STEP = [
    # (lens, s_q, H, page_size)
    ([300, 17], 1, 16, 0),
    ([64, 1000, 5], 2, 16, 64),
    ([2000], 4, 32, 16),
]


@pytest.mark.parametrize("case", range(len(STEP)))
def test_decode_step_chain(ctx, case):
    """absorb -> append -> mla_decode -> project on the GPU, against the
    oracle's absorb -> append -> attention -> project on the same inputs."""
    import torch

    import decode_attention_mla_amd as mla

    lens, s_q, H, ps = STEP[case]
    announce(f"decode step lens={lens} s_q={s_q} H={H} page={ps}")
    inp, kv = cache_case(50 + case, lens, s_q, ps, None)
    B = len(lens)
    si = wl.make_step_inputs(500 + case, B, s_q, H)
    dev = "cuda:0"
    kv_d = wl.bf16_tensor(kv)
    bt = None if inp.block_table is None else torch.from_numpy(inp.block_table).to(dev)
    lens_d = torch.from_numpy(inp.seqlens).to(dev)
    q = mla.mla_absorb_q(ctx, wl.bf16_tensor(si.q_nope.reshape(B, s_q, H, -1)),
                         wl.bf16_tensor(si.q_rope.reshape(B, s_q, H, -1)), wl.bf16_tensor(si.w_uk))
    mla.mla_append_kv(ctx, wl.bf16_tensor(si.new_rows), kv_d, bt, lens_d, seqlens_host=inp.seqlens)
    o, lse = mla.mla_decode(ctx, q, kv_d, bt, lens_d, inp.scale, seqlens_host=inp.seqlens)
    out = mla.mla_project_out(ctx, o, wl.bf16_tensor(si.w_uv))
    torch.cuda.synchronize()

    kv_ref = steps.append_kv(kv, inp.block_table, inp.seqlens, si.new_rows)
    assert np.array_equal(bits_of(kv_d), kv_ref)
    _, q_ref = steps.absorb_q(si.q_nope, si.q_rope, si.w_uk)
    o_ref, lse_ref = oracle.mla_decode(q_ref.reshape(B, s_q, H, 576), kv_ref, inp.block_table,
                                       inp.seqlens, inp.scale)
    out_ref = steps.project_out(o_ref.reshape(B * s_q, H, 512), si.w_uv).reshape(B, s_q, H, -1)
    err = out.cpu().numpy().astype(np.float64) - out_ref
    assert np.isfinite(err).all()
    assert float(np.sqrt(np.mean(err ** 2))) <= 1e-4, float(np.sqrt(np.mean(err ** 2)))
    assert float(np.abs(err).max()) <= 1e-3, float(np.abs(err).max())
    assert float(np.abs(lse.cpu().numpy() - lse_ref).max()) <= 1e-4
