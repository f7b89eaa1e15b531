"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Bar (fp32 outputs): O RMSE <= 1e-4, O max-abs <= 1e-3, LSE max-abs <= 1e-4.
Every case is checked element by element on every row, the full-size
workloads included (in the default launch configuration that bench.py
times).
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import compare, run_gpu, to_device

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


def oracle_of(inp, rows=None):
    if rows is None:
        return oracle.mla_decode(inp.q, inp.kv, inp.block_table, inp.seqlens, inp.scale)
    bt = None if inp.block_table is None else inp.block_table[rows]
    kv = inp.kv if inp.block_table is not None else inp.kv[rows]
    return oracle.mla_decode(inp.q[rows], kv, bt, inp.seqlens[rows], inp.scale)


SMALL = [
    # (B, s_q, H, lens, page_size)
    (1, 1, 16, [1], 0),
    (1, 1, 16, [2], 64),
    (3, 1, 16, [15, 16, 17], 0),
    (2, 1, 16, [63, 65], 16),
    (2, 1, 16, [127, 300], 64),
    (1, 1, 16, [4097], 0),
    (2, 2, 16, [5, 70], 0),
    (2, 3, 16, [3, 200], 16),
    (3, 4, 16, [4, 64, 1000], 64),
    (2, 1, 32, [100, 33], 0),
    (2, 1, 64, [257, 16], 16),
    (1, 4, 32, [129], 64),
    (4, 2, 48, [31, 32, 33, 500], 0),
    (2, 5, 16, [7, 150], 16),           # row blocks 4 + 1: two kernels
    (2, 1, 48, [300, 70], 16),          # three row blocks: one idle wave
    (1, 1, 128, [777], 64),             # eight row blocks: two groups of four
    (1, 2, 64, [1000], 0),              # eight row blocks over two tokens
    (1, 8, 16, [1000], 16),             # eight causal tokens
    (1, 1, 144, [600], 0),              # nine row blocks: two groups, then one
    (2, 3, 32, [50, 700], 64),          # six row blocks: a group, then two
]


@pytest.mark.parametrize("splits,min_chunk", [(0, 0), (3, 16), (7, 64), (256, 16)])
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_shapes_against_oracle(ctx, case, splits, min_chunk):
    import decode_attention_mla_amd as mla

    B, s_q, H, lens, ps = SMALL[case]
    announce(f"small {SMALL[case]} splits={splits} min_chunk={min_chunk}")
    inp = wl.small("s", B, s_q, H, lens, page_size=ps, seed=100 + case)
    ctx.set_option(mla.MLA_OPT_NUM_SPLITS, splits)
    ctx.set_option(mla.MLA_OPT_MIN_CHUNK, min_chunk)
    try:
        o, l = run_gpu(ctx, inp)
        ro, rl = oracle_of(inp)
        compare(o, l, ro, rl, str(SMALL[case]))
        # without host lengths the launch is sized blind: same bits
        o2, l2 = run_gpu(ctx, inp, host_lens=False)
        assert np.array_equal(o, o2) and np.array_equal(l, l2)
    finally:
        ctx.set_option(mla.MLA_OPT_NUM_SPLITS, 0)
        ctx.set_option(mla.MLA_OPT_MIN_CHUNK, 0)


# Device lengths outside [s_q, capacity] (the host does not see them): the
# kernels clamp them to [0, capacity], and a row whose causal window
# [0, L - s_q + t] holds no key is defined as O = 0, LSE = -inf.  The other
# rows are single-token attentions over the window, which the oracle gives.
OUT_OF_CONTRACT = [
    # (B, s_q, H, device lens, page_size, capacity)
    (4, 1, 16, [0, 5, 0, 40], 0, 48),
    (3, 4, 16, [0, 2, 300], 16, 320),
    (2, 4, 32, [1, 3], 64, 64),
    (3, 2, 16, [0, 0, 0], 0, 16),
    (2, 2, 16, [40, 1000], 0, 33),   # longer than the cache: clamped to 33
]


@pytest.mark.parametrize("case", range(len(OUT_OF_CONTRACT)))
def test_device_lengths_outside_the_contract(ctx, case):
    import torch

    B, s_q, H, lens, ps, cap = OUT_OF_CONTRACT[case]
    announce(f"device lengths {OUT_OF_CONTRACT[case]}")
    held = [min(n, cap) for n in lens]
    w = wl.Workload("e", B, s_q, H, max(max(held), 1), ps, 200 + case)
    inp = wl.make_inputs(w, poison=True, seqlens=held, capacity=cap)
    dev = list(to_device(inp))
    dev[3] = torch.tensor(lens, dtype=torch.int32, device="cuda")
    # outputs start as NaN: every row must be written
    out = torch.full((B, s_q, H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, s_q, H), float("nan"), dtype=torch.float32, device="cuda")
    o, l = run_gpu(ctx, inp, dev=dev, host_lens=False, out=out, lse=lse)
    n_empty = 0
    for b in range(B):
        for t in range(s_q):
            vis = held[b] - s_q + t + 1
            if vis <= 0:
                n_empty += 1
                assert np.all(np.isneginf(l[b, t])) and np.all(o[b, t] == 0.0), (b, t)
                continue
            bt = None if inp.block_table is None else inp.block_table[b:b + 1]
            kv = inp.kv if inp.block_table is not None else inp.kv[b:b + 1]
            ro, rl = oracle.mla_decode(inp.q[b:b + 1, t:t + 1], kv, bt,
                                       np.array([vis], np.int32), inp.scale)
            compare(o[b:b + 1, t:t + 1], l[b:b + 1, t:t + 1], ro, rl, f"{OUT_OF_CONTRACT[case]} b={b} t={t}")
    assert n_empty > 0 or case == len(OUT_OF_CONTRACT) - 1


# Medium decode shapes: many heads (several row-block groups), several
# query tokens, other page sizes, one long sequence; every row checked.
MEDIUM = [
    # (B, s_q, H, lens, page_size)
    (4, 1, 128, [3000, 1, 777, 4096], 64),
    (2, 2, 64, [5000, 300], 32),
    (3, 1, 16, [10000, 20000, 5], 128),
    (2, 3, 32, [4096, 4097], 256),
    (1, 4, 16, [65536], 0),
    (5, 1, 32, [1, 2, 3, 4, 5], 16),
    (2, 1, 80, [2000, 33], 0),          # row blocks 4 + 1
    (3, 3, 16, [1500, 3, 4000], 0),     # three row blocks sharing one key group
]


@pytest.mark.parametrize("case", range(len(MEDIUM)))
def test_medium_shapes_against_oracle(ctx, case):
    B, s_q, H, lens, ps = MEDIUM[case]
    announce(f"medium {MEDIUM[case]}")
    inp = wl.small("m", B, s_q, H, lens, page_size=ps, seed=300 + case)
    o, l = run_gpu(ctx, inp)
    ro, rl = oracle_of(inp)
    compare(o, l, ro, rl, str(MEDIUM[case]))
    o2, l2 = run_gpu(ctx, inp, host_lens=False)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


# More than 64 sequences: the plan and the combine walk the lengths 64 at a
# time, and a workgroup's segments can run across that boundary.
MANY = [
    # (B, s_q, H, page_size, seed)
    (70, 1, 16, 0, 21),
    (130, 1, 16, 16, 22),
    (100, 2, 32, 64, 23),
    (65, 4, 16, 0, 24),
]


@pytest.mark.parametrize("splits", [0, 7])
@pytest.mark.parametrize("case", range(len(MANY)))
def test_more_than_64_sequences(ctx, case, splits):
    import decode_attention_mla_amd as mla

    B, s_q, H, ps, seed = MANY[case]
    lens = [int(x) for x in np.random.default_rng(seed).integers(s_q, 400, size=B)]
    announce(f"many sequences {MANY[case]} splits={splits}")
    inp = wl.small("many", B, s_q, H, lens, page_size=ps, seed=seed)
    ctx.set_option(mla.MLA_OPT_NUM_SPLITS, splits)
    try:
        o, l = run_gpu(ctx, inp)
        ro, rl = oracle_of(inp)
        compare(o, l, ro, rl, str(MANY[case]))
        o2, l2 = run_gpu(ctx, inp, host_lens=False)
        assert np.array_equal(o, o2) and np.array_equal(l, l2)
    finally:
        ctx.set_option(mla.MLA_OPT_NUM_SPLITS, 0)


# Lengths whose plain line starts sequences inside key ranges, so that the
# plan follows every sequence with MLA_PLAN_SEQ_GAP line keys: short
# sequences several to a range, long ones across many, more than 64 of them,
# in every kernel mode.  (name, lens, s_q, H, page_size, key ranges)
_rng = np.random.default_rng(31)
GAPPED = [
    ("70 mixed, one row block", [int(x) for x in np.concatenate([_rng.integers(20, 300, size=64),
                                                                  _rng.integers(3000, 6000, size=6)])],
     1, 16, 16, 64),
    ("two key groups", [900, 33, 2500, 7, 1200], 2, 16, 0, 16),
    ("one key group", [100, 2000, 50, 3000, 70, 900], 4, 16, 64, 32),
    ("128 heads", [500, 4000, 90], 1, 128, 16, 8),
]


@pytest.mark.parametrize("case", range(len(GAPPED)))
def test_plan_with_sequence_gaps(ctx, case):
    """The plan with gaps: the host mirror reports the gap, and host-sized
    and blind launches (where every workgroup decides the gap itself) match
    the oracle and each other bit for bit."""
    import decode_attention_mla_amd as mla

    name, lens, s_q, H, ps, splits = GAPPED[case]
    announce(f"gapped plan: {name}, B={len(lens)} s_q={s_q} H={H} page={ps} ranges={splits}")
    _, info = mla.mla_plan(lens, splits, 64)
    assert info["seq_gap"] == 128, info
    inp = wl.small("gap", len(lens), s_q, H, lens, page_size=ps, seed=900 + case)
    ctx.set_option(mla.MLA_OPT_NUM_SPLITS, splits)
    try:
        o, l = run_gpu(ctx, inp)
        ro, rl = oracle_of(inp)
        compare(o, l, ro, rl, name)
        o2, l2 = run_gpu(ctx, inp, host_lens=False)
        assert np.array_equal(o, o2) and np.array_equal(l, l2), f"{name}: blind launch differs"
    finally:
        ctx.set_option(mla.MLA_OPT_NUM_SPLITS, 0)


def test_single_key_returns_value_row_exactly(ctx):
    announce("single key")
    inp = wl.small("one", 4, 1, 16, [1, 1, 1, 1], page_size=64, seed=5)
    o, l = run_gpu(ctx, inp)
    for b in range(4):
        row = wl.bf16_bits_to_f32(inp.kv[inp.block_table[b, 0], 0]).astype(np.float64)
        assert np.array_equal(o[b, 0], np.broadcast_to(row[:512], (16, 512)))
    ro, rl = oracle_of(inp)
    assert np.max(np.abs(l - rl)) <= 1e-5


def test_zero_query_gives_mean_of_values(ctx):
    announce("zero query")
    inp = wl.small("zq", 2, 4, 16, [77, 1500], seed=6)
    inp.q[:] = 0
    o, l = run_gpu(ctx, inp)
    ro, rl = oracle_of(inp)
    compare(o, l, ro, rl, "zero query")


def test_peaked_softmax_and_large_scores(ctx):
    """Scaled-up queries give peaked softmaxes and force reference-max moves."""
    announce("peaked")
    inp = wl.small("pk", 3, 2, 16, [50, 700, 3000], page_size=16, seed=7)
    q = wl.bf16_bits_to_f32(inp.q) * 6.0
    inp.q[:] = wl.f32_to_bf16_bits(q)
    o, l = run_gpu(ctx, inp)
    ro, rl = oracle_of(inp)
    compare(o, l, ro, rl, "peaked")


def test_increasing_scores_rescale_every_block(ctx):
    """Keys whose scores grow along the sequence move the running max in
    every block (the slow path of the online softmax)."""
    announce("increasing")
    inp = wl.small("inc", 1, 1, 16, [2048], seed=8)
    inp.q[0, 0, :, 520] = wl.f32_to_bf16_bits(np.array([8.0], np.float32))[0]
    ramp = np.linspace(0, 40, 2048, dtype=np.float32)
    inp.kv[0, :2048, 520] = wl.f32_to_bf16_bits(ramp)
    o, l = run_gpu(ctx, inp)
    ro, rl = oracle_of(inp)
    compare(o, l, ro, rl, "increasing")


def test_bitwise_repeatable(ctx):
    announce("repeatable")
    inp = wl.make_inputs(wl.WORKLOADS["mla_bs16_ctx4096"])
    dev = to_device(inp)
    o1, l1 = run_gpu(ctx, inp, dev)
    o2, l2 = run_gpu(ctx, inp, dev)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("name", sorted(wl.WORKLOADS))
def test_workload_full_size(ctx, name):
    """Each workload at its full size, in the launch configuration bench.py
    times: every output element of every row against the oracle."""
    import torch

    announce(f"workload {name}, every row")
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, poison=True)
    o, l = run_gpu(ctx, inp)
    torch.cuda.empty_cache()
    ro, rl = oracle_of(inp)
    compare(o, l, ro, rl, name)
    # and the LSE of an N(0,1) context lies near ln(L) + |scale q|^2 / 2
    # (the Gaussian tilt law of the inputs)
    a2 = (wl.bf16_bits_to_f32(inp.q).astype(np.float64) * inp.scale) ** 2
    vis = inp.seqlens[:, None].astype(np.float64) - w.s_q + 1 + np.arange(w.s_q)[None, :]
    law = np.log(vis)[:, :, None] + a2.sum(-1) / 2
    tol = 8 * np.sqrt((np.exp(a2.sum(-1)) - 1) / vis[:, :, None])
    assert np.all(np.abs(l - law) <= tol)


def test_long_single_sequence(ctx):
    """One sequence of 2,000,003 keys (2.3 GB of cache): key byte offsets
    past 2^31, 256 parts of one sequence merged in 16 batches, a ragged
    last block; every row against the oracle."""
    import torch

    announce("long single sequence L=2000003")
    inp = wl.small("long", 1, 1, 16, [2_000_003], page_size=0, seed=77)
    o, l = run_gpu(ctx, inp)
    torch.cuda.empty_cache()
    ro, rl = oracle_of(inp)
    compare(o, l, ro, rl, "long single sequence")
