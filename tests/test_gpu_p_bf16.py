"""MLA_OPT_P_BF16: P enters P V as one bf16 value in the kernels whose row
blocks share key steps.

Bound (derived from the arithmetic): each weight p_j is rounded to bf16, so
p_j (1 + d_j) with |d_j| <= 2^-8 (8 significant bits, rounded to nearest), while the sum l and the LSE keep the fp32
weights.  Then O_c moves by sum_j p_j d_j v_jc / l, at most 2^-8 max_j |v_jc|
over the sequence's keys; the key-group merge and the split combine are
weighted averages and keep that bound.  The tests check every element
against the fp64 oracle within that bound (plus the default path's 1e-5),
the LSE within the default bar, and that 16-row problems (one row block,
where both halves of P share one MFMA) are unaffected bit for bit.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import LSE_MAXABS_MAX, compare, run_gpu, to_device

pytestmark = pytest.mark.gpu

ROUNDING = 2.0 ** -8  # unit roundoff of bf16
SLACK = 1e-5  # the default path's own error, far above its measured 1e-7


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mla():
    import torch

    import decode_attention_mla_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    return m


def v_max(inp):
    """max_j |V[j][c]| over each sequence's keys: [B, 512]."""
    out = np.zeros((inp.q.shape[0], wl.D_V))
    for b, n in enumerate(inp.seqlens):
        rows = wl.bf16_bits_to_f32(wl.sequence_rows(inp.workload.seed, b, int(n)))[:, : wl.D_V]
        out[b] = np.abs(rows).max(axis=0)
    return out


# (B, s_q, H, lengths, page size): one key group of four row blocks, two key
# groups, four plus two, four plus a lone block, and eight (two groups).
CASES = [
    (2, 4, 16, [3000, 700], 0),
    (3, 2, 16, [1000, 33, 2048], 64),
    (2, 2, 48, [1500, 100], 16),
    (2, 5, 16, [900, 2500], 0),
    (1, 1, 128, [4096], 32),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_within_the_rounding_bound(mla, case):
    B, s_q, H, lens, ps = CASES[case]
    announce(f"P as one bf16 {CASES[case]}")
    inp = wl.small("pbf", B, s_q, H, lens, page_size=ps, seed=700 + case)
    dev = to_device(inp)
    ctx = mla.Context()
    try:
        o_def, l_def = run_gpu(ctx, inp, dev)
        ctx.set_option(mla.MLA_OPT_P_BF16, 1)
        o, l = run_gpu(ctx, inp, dev)
    finally:
        ctx.close()
    ro, rl = oracle.mla_decode(inp.q, inp.kv, inp.block_table, inp.seqlens, inp.scale)
    bound = ROUNDING * v_max(inp)[:, None, None, :] + SLACK
    assert np.isfinite(o).all() and np.isfinite(l).all()
    excess = np.abs(o - ro) - bound
    assert excess.max() <= 0, f"{CASES[case]}: {int((excess > 0).sum())} elements past the bound"
    assert np.abs(l - rl).max() <= LSE_MAXABS_MAX
    # the option took effect
    assert not np.array_equal(o, o_def)


def test_one_row_block_is_unaffected(mla):
    announce("P as one bf16, 16 rows")
    inp = wl.small("pbf1", 3, 1, 16, [700, 4000, 33], page_size=64, seed=710)
    dev = to_device(inp)
    ctx = mla.Context()
    try:
        o_def, l_def = run_gpu(ctx, inp, dev)
        ctx.set_option(mla.MLA_OPT_P_BF16, 1)
        o, l = run_gpu(ctx, inp, dev)
    finally:
        ctx.close()
    assert np.array_equal(o, o_def) and np.array_equal(l, l_def)


def test_rmse_at_long_context(mla):
    """The pages' own measure (an RMSE against a double-precision reference)
    on N(0,1) inputs at 64 heads, 16K keys: within the default bar."""
    announce("P as one bf16, RMSE at 16K keys, 64 heads")
    inp = wl.small("pbfl", 2, 1, 64, [16384, 12000], seed=720)
    ctx = mla.Context()
    ctx.set_option(mla.MLA_OPT_P_BF16, 1)
    try:
        o, l = run_gpu(ctx, inp)
    finally:
        ctx.close()
    ro, rl = oracle.mla_decode(inp.q, inp.kv, inp.block_table, inp.seqlens, inp.scale)
    rmse, _, _ = compare(o, l, ro, rl, "P as one bf16 at 16K keys")
    assert rmse > 1e-7  # not the default path (its RMSE is about 2e-8 here)


def test_option_values(mla):
    ctx = mla.Context()
    try:
        with pytest.raises(mla.MlaError):
            ctx.set_option(mla.MLA_OPT_P_BF16, 2)
        ctx.set_option(mla.MLA_OPT_P_BF16, 0)
    finally:
        ctx.close()


N_FUZZ = 60


def test_random_shapes_within_the_bound(mla):
    """The seeded random shapes of the default fuzz (batch, lengths, tokens,
    heads, pages, forced splits, peaked queries), with the option on: every
    element within the rounding bound, the LSE within the default bar."""
    from test_gpu_fuzz import draw_case

    ctx = mla.Context()
    ctx.set_option(mla.MLA_OPT_P_BF16, 1)
    try:
        for i in range(N_FUZZ):
            c = draw_case(i)
            print(f"[p-bf16 fuzz {i}] {c}", flush=True)
            sys.stdout.flush()
            inp = wl.small("fz", c["B"], c["s_q"], c["H"], c["lens"], page_size=c["page"], seed=c["seed"])
            if c["q_scale"] != 1.0:
                inp.q[:] = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(inp.q) * np.float32(c["q_scale"]))
            ctx.set_option(mla.MLA_OPT_NUM_SPLITS, c["splits"])
            ctx.set_option(mla.MLA_OPT_MIN_CHUNK, c["min_chunk"])
            o, l = run_gpu(ctx, inp, host_lens=c["host_lens"])
            ro, rl = oracle.mla_decode(inp.q, inp.kv, inp.block_table, inp.seqlens, inp.scale)
            bound = ROUNDING * v_max(inp)[:, None, None, :] + SLACK
            assert np.isfinite(o).all() and np.isfinite(l).all(), f"case {i}"
            excess = np.abs(o - ro) - bound
            assert excess.max() <= 0, f"case {i} {c}: {int((excess > 0).sum())} elements past the bound"
            assert np.abs(l - rl).max() <= LSE_MAXABS_MAX, f"case {i} {c}: LSE"
    finally:
        ctx.close()
