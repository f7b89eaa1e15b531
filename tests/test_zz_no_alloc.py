"""mla_decode_noalloc (the entry point that allocates nothing) through the
C ABI: against mla_decode and against the fp64 oracle, on two calls in a
row, the second smaller, so that the second reads a scratch array that still
holds the first call's partials; then a problem whose partials need fewer
key ranges than the default plan, one too large for the array, and the call
captured in a HIP graph and replayed.

Bar: the O/LSE bar of the parity tests (O RMSE <= 1e-4, max-abs <= 1e-3,
LSE max-abs <= 1e-4) against the oracle, and equality with mla_decode's
output when both use the same split plan.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import compare, to_device

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def run_noalloc(mla, inp, host_lens=True):
    import torch

    q, kv, bt, lens = to_device(inp)
    B, s_q, H = inp.q.shape[:3]
    out = torch.full((B, s_q, H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, s_q, H), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_decode_noalloc(q, kv, bt, lens, inp.scale, out, lse,
                           seqlens_host=inp.seqlens if host_lens else None)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def run_ctx(mla, inp, splits=0):
    import torch

    ctx = mla.Context()
    try:
        ctx.set_option(mla.MLA_OPT_NUM_SPLITS, splits)
        o, l = mla.mla_decode(ctx, *to_device(inp), inp.scale, seqlens_host=inp.seqlens)
        torch.cuda.synchronize()
        return o.cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64)
    finally:
        ctx.close()


@pytest.fixture(scope="module")
def mla():
    import torch

    import decode_attention_mla_amd as m

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(0)
    return m


def test_two_calls_in_a_row_second_smaller(mla):
    big = wl.small("na1", 4, 4, 16, [3000, 17, 5000, 640], page_size=64, seed=700)
    small = wl.small("na2", 2, 1, 16, [900, 40], page_size=0, seed=701)
    for inp, what in ((big, "first, larger"), (small, "second, smaller")):
        announce(f"noalloc {what}: B={inp.q.shape[0]} s_q={inp.q.shape[1]}")
        o, l = run_noalloc(mla, inp)
        ro, rl = oracle.mla_decode(inp.q, inp.kv, inp.block_table, inp.seqlens, inp.scale)
        compare(o, l, ro, rl, f"noalloc {what}")
        oc, lc = run_ctx(mla, inp)
        assert np.array_equal(o, oc) and np.array_equal(l, lc), f"noalloc {what} differs from mla_decode"
    # device lengths only, after both
    announce("noalloc device lengths only")
    o, l = run_noalloc(mla, small, host_lens=False)
    ro, rl = oracle.mla_decode(small.q, small.kv, small.block_table, small.seqlens, small.scale)
    compare(o, l, ro, rl, "noalloc device lengths")


def test_fewer_key_ranges_when_the_default_plan_does_not_fit(mla):
    """80 heads at s_q = 1 (five row blocks) on a 256-CU device: the default
    plan needs 2560 partial row blocks, the array holds 2048, so the call
    uses 204 key ranges; mla_decode with that split count gives the same
    bits."""
    import torch

    announce("noalloc with fewer key ranges")
    inp = wl.small("na3", 3, 1, 80, [2000, 33, 4100], page_size=16, seed=702)
    o, l = run_noalloc(mla, inp)
    ro, rl = oracle.mla_decode(inp.q, inp.kv, inp.block_table, inp.seqlens, inp.scale)
    compare(o, l, ro, rl, "noalloc 80 heads")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_rb = 5
    default = cus  # one row-block group of four plus a last group of one: one group per launch
    splits = min(default, 2048 // (2 * n_rb))
    oc, lc = run_ctx(mla, inp, splits=splits)
    assert np.array_equal(o, oc) and np.array_equal(l, lc)


def test_too_large_is_refused_before_any_launch(mla):
    import torch

    announce("noalloc too large")
    assert mla.noalloc_scratch_bytes() == 2048 * 16 * 513 * 4 + 256
    B, s_q, H = 1, 2, 8256  # 16,512 query rows: one key range needs 2 x 1032 row blocks
    q = torch.zeros((B, s_q, H, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, 16, 576), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((B,), 16, dtype=torch.int32, device="cuda")
    out = torch.full((B, s_q, H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, s_q, H), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(mla.MlaError) as ei:
        mla.mla_decode_noalloc(q, kv, None, lens, 1 / 24, out, lse)
    assert ei.value.code == mla.MLA_ERR_WORKSPACE
    assert "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and torch.isnan(lse).all()


def test_graph_replays_of_the_noalloc_call(mla):
    """The call captured in a HIP graph (device lengths only, so nothing on
    the host reads them) and replayed with new lengths and queries written in
    place; between replays an eager call of another shape overwrites the
    scratch array.  Every replay and every eager call against the oracle."""
    import torch

    B, s_q, H = 3, 1, 16
    full = [700, 33, 2048]
    announce("noalloc graph capture")
    inp = wl.small("nag", B, s_q, H, full, page_size=16, seed=703)
    other = wl.small("nag2", 2, 2, 16, [1200, 90], page_size=0, seed=704)
    q, kv, bt, lens = to_device(inp)
    out = torch.full((B, s_q, H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, s_q, H), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        mla.mla_decode_noalloc(q, kv, bt, lens, inp.scale, out, lse, stream=stream)  # warm-up
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        mla.mla_decode_noalloc(q, kv, bt, lens, inp.scale, out, lse, stream=stream)

    rng = np.random.default_rng(705)
    for rep, new_lens in enumerate([full, [2, 33, 1500], [640, 17, 2047], [699, 2, 64]]):
        # Lengths only shrink, so every key read is a real cache row.
        inp.seqlens[:] = new_lens
        inp.q[:] = wl.f32_to_bf16_bits(rng.standard_normal(inp.q.shape).astype(np.float32))
        lens.copy_(torch.from_numpy(inp.seqlens))
        q.copy_(torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ro, rl = oracle.mla_decode(inp.q, inp.kv, inp.block_table, inp.seqlens, inp.scale)
        compare(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                ro, rl, f"noalloc replay {rep} lens={new_lens}")
        # An eager call of another shape between replays (same scratch array).
        oe, le = run_noalloc(mla, other)
        roe, rle = oracle.mla_decode(other.q, other.kv, other.block_table, other.seqlens, other.scale)
        compare(oe, le, roe, rle, f"noalloc eager {rep}")
