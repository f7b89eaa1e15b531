"""Seeded random decode shapes against the fp64 oracle, through the C ABI.

One test walks a fixed, seeded list of shapes and stops at the first case
that misses the bar (O RMSE <= 1e-4, O max-abs <= 1e-3, LSE max-abs <= 1e-4,
every element of every row), naming it.  The draws cover what the fixed
shape lists do not: batch 1-8, lengths 1-5000 (log-uniform, ragged within a
batch), 1-8 query tokens (causal), 16-144 heads, contiguous and paged
layouts (pages of 16-128 keys), the default split plan and forced split
counts and smallest ranges, host lengths or device lengths only, and
queries scaled up for peaked softmaxes.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import compare, run_gpu

N_CASES = 600
MAX_ROW_KEYS = 3_000_000  # bounds the oracle's work per case (rows x keys)


def draw_case(i):
    rng = np.random.default_rng([4242, i])
    H = int(rng.choice([16, 32, 48, 64, 80, 96, 128, 144]))
    s_q = int(rng.integers(1, 9))
    while s_q * H > 288 and s_q > 1:
        s_q -= 1
    B = int(rng.integers(1, 9))
    l_max = int(np.exp(rng.uniform(0.0, np.log(5000.0))))
    l_max = max(l_max, s_q)
    lens = rng.integers(s_q, l_max + 1, size=B)
    while B > 1 and B * s_q * H * float(lens.mean()) > MAX_ROW_KEYS:
        B -= 1
        lens = lens[:B]
    page = int(rng.choice([0, 16, 32, 64, 128]))
    splits = int(rng.choice([0, 0, 1, 2, 5, 13, 64, 256, 300]))
    min_chunk = int(rng.choice([0, 0, 16, 48, 256, 1024]))
    host_lens = bool(rng.integers(0, 4) > 0)
    q_scale = float(rng.choice([1.0, 1.0, 3.0, 8.0]))
    return dict(B=B, s_q=s_q, H=H, lens=[int(x) for x in lens], page=page, splits=splits,
                min_chunk=min_chunk, host_lens=host_lens, q_scale=q_scale, seed=5000 + i)


def test_draws_are_within_the_bounds():
    for i in range(N_CASES):
        c = draw_case(i)
        assert 1 <= c["B"] <= 8 and 1 <= c["s_q"] <= 8 and c["H"] % 16 == 0
        assert all(c["s_q"] <= L <= 5000 for L in c["lens"])


@pytest.mark.gpu
def test_random_shapes_against_oracle():
    import torch

    import decode_attention_mla_amd as mla

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    ctx = mla.Context()
    try:
        for i in range(N_CASES):
            c = draw_case(i)
            print(f"[fuzz {i}] {c}", flush=True)
            sys.stdout.flush()
            inp = wl.small("fz", c["B"], c["s_q"], c["H"], c["lens"], page_size=c["page"], seed=c["seed"])
            if c["q_scale"] != 1.0:
                inp.q[:] = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(inp.q) * np.float32(c["q_scale"]))
            ctx.set_option(mla.MLA_OPT_NUM_SPLITS, c["splits"])
            ctx.set_option(mla.MLA_OPT_MIN_CHUNK, c["min_chunk"])
            o, l = run_gpu(ctx, inp, host_lens=c["host_lens"])
            ro, rl = oracle.mla_decode(inp.q, inp.kv, inp.block_table, inp.seqlens, inp.scale)
            compare(o, l, ro, rl, f"fuzz case {i} {c}")
    finally:
        ctx.set_option(mla.MLA_OPT_NUM_SPLITS, 0)
        ctx.set_option(mla.MLA_OPT_MIN_CHUNK, 0)
        ctx.close()


N_MANY = 40


def draw_many(i):
    """Larger batches of short sequences (65-200 of 1-300 keys): the plan and
    the combine walk the lengths 64 at a time, and most workgroups hold
    several segments."""
    rng = np.random.default_rng([4343, i])
    H = int(rng.choice([16, 32, 64]))
    s_q = int(rng.integers(1, 3))
    B = int(rng.integers(65, 201))
    lens = [int(x) for x in rng.integers(s_q, 301, size=B)]
    page = int(rng.choice([0, 16, 64]))
    splits = int(rng.choice([0, 0, 7, 100]))
    host_lens = bool(rng.integers(0, 2))
    return dict(B=B, s_q=s_q, H=H, lens=lens, page=page, splits=splits, host_lens=host_lens, seed=6000 + i)


@pytest.mark.gpu
def test_many_short_sequences_against_oracle():
    import torch

    import decode_attention_mla_amd as mla

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    ctx = mla.Context()
    try:
        for i in range(N_MANY):
            c = draw_many(i)
            print(f"[many {i}] B={c['B']} s_q={c['s_q']} H={c['H']} page={c['page']} splits={c['splits']} "
                  f"host_lens={c['host_lens']}", flush=True)
            inp = wl.small("mn", c["B"], c["s_q"], c["H"], c["lens"], page_size=c["page"], seed=c["seed"])
            ctx.set_option(mla.MLA_OPT_NUM_SPLITS, c["splits"])
            o, l = run_gpu(ctx, inp, host_lens=c["host_lens"])
            ro, rl = oracle.mla_decode(inp.q, inp.kv, inp.block_table, inp.seqlens, inp.scale)
            compare(o, l, ro, rl, f"many case {i}")
    finally:
        ctx.set_option(mla.MLA_OPT_NUM_SPLITS, 0)
        ctx.close()


def test_many_draws_are_within_the_bounds():
    for i in range(N_MANY):
        c = draw_many(i)
        assert 65 <= c["B"] <= 200 and c["H"] % 16 == 0
        assert all(c["s_q"] <= L <= 300 for L in c["lens"])
