"""The split workspace at the C ABI: its size, a caller-owned buffer
(mla_workspace_size, mla_ctx_set_workspace), and the context's own buffer
growing without invalidating work captured earlier.

Results with a caller's workspace are checked against the fp64 oracle and,
bit for bit, against the same call on the library's own workspace.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import compare, run_gpu, to_device

pytestmark = pytest.mark.gpu


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


def expected_bytes(splits, s_q, heads):
    return 2 * splits * (s_q * heads // 16) * 16 * 513 * 4 + 256


def test_workspace_size_formula(mla):
    import torch

    announce("workspace size")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ctx = mla.Context()
    try:
        # one launch per group of four row blocks (and a last group of
        # three); a last group of one or two has a launch of its own
        for s_q, H, groups in [(1, 16, 1), (4, 16, 1), (1, 64, 1), (1, 128, 2), (2, 80, 2), (5, 16, 1),
                               (1, 144, 2), (3, 32, 1)]:
            assert ctx.workspace_size(s_q, H) == expected_bytes(cus // groups, s_q, H), (s_q, H)
        ctx.set_option(mla.MLA_OPT_NUM_SPLITS, 7)
        assert ctx.workspace_size(2, 32) == expected_bytes(7, 2, 32)
        with pytest.raises(mla.MlaError):
            ctx.workspace_size(1, 24)
    finally:
        ctx.close()


CASES = [
    # (B, s_q, H, lens, page_size)
    (3, 1, 16, [700, 33, 4000], 0),
    (2, 4, 16, [5000, 17], 64),
    (2, 1, 128, [3000, 900], 16),
    (4, 2, 48, [100, 2000, 64, 3], 0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_caller_workspace_matches_own_workspace(mla, case):
    import torch

    B, s_q, H, lens, ps = CASES[case]
    announce(f"caller workspace {CASES[case]}")
    inp = wl.small("ws", B, s_q, H, lens, page_size=ps, seed=600 + case)
    dev = to_device(inp)
    own = mla.Context()
    mine = mla.Context()
    try:
        o1, l1 = run_gpu(own, inp, dev)
        buf = mine.allocate_workspace(s_q, H)
        assert buf.numel() == mine.workspace_size(s_q, H)
        o2, l2 = run_gpu(mine, inp, dev)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        ro, rl = oracle.mla_decode(inp.q, inp.kv, inp.block_table, inp.seqlens, inp.scale)
        compare(o2, l2, ro, rl, f"caller workspace {CASES[case]}")
        # device lengths only: same bits
        o3, l3 = run_gpu(mine, inp, dev, host_lens=False)
        assert np.array_equal(o2, o3) and np.array_equal(l2, l3)
        torch.cuda.synchronize()
    finally:
        own.close()
        mine.close()


def test_too_small_workspace_is_refused_before_any_launch(mla):
    import torch

    announce("workspace too small")
    inp = wl.small("wsz", 2, 2, 32, [300, 1000], seed=610)
    q, kv, bt, lens = to_device(inp)
    ctx = mla.Context()
    try:
        need = ctx.workspace_size(2, 32)
        small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
        ctx.set_workspace(small)
        out = torch.full((2, 2, 32, 512), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((2, 2, 32), float("nan"), dtype=torch.float32, device="cuda")
        with pytest.raises(mla.MlaError) as ei:
            mla.mla_decode(ctx, q, kv, bt, lens, inp.scale, out=out, lse=lse)
        assert ei.value.code == mla.MLA_ERR_WORKSPACE
        with pytest.raises(mla.MlaError) as ei:
            ctx.reserve(2, 32)
        assert ei.value.code == mla.MLA_ERR_WORKSPACE
        torch.cuda.synchronize()
        assert torch.isnan(out).all() and torch.isnan(lse).all()
        # a smaller problem fits
        inp1 = wl.small("wsz1", 2, 1, 16, [300, 1000], seed=611)
        o, l = run_gpu(ctx, inp1)
        ro, rl = oracle.mla_decode(inp1.q, inp1.kv, inp1.block_table, inp1.seqlens, inp1.scale)
        compare(o, l, ro, rl, "smaller problem in a small workspace")
        # misaligned or empty buffers are refused
        with pytest.raises(mla.MlaError):
            ctx.set_workspace(small[16:])
        # back to the library's own workspace: the large problem runs
        ctx.set_workspace(None)
        o, l = run_gpu(ctx, inp)
        ro, rl = oracle.mla_decode(inp.q, inp.kv, inp.block_table, inp.seqlens, inp.scale)
        compare(o, l, ro, rl, "own workspace again")
    finally:
        ctx.close()


def test_graph_capture_with_caller_workspace(mla):
    """No reserve: the caller's buffer is the workspace, captured into the
    graph; replays with new lengths and queries match the oracle."""
    import torch

    announce("graph with caller workspace")
    B, s_q, H = 3, 2, 16
    full = [900, 40, 3000]
    inp = wl.small("wsg", B, s_q, H, full, page_size=32, seed=620)
    q, kv, bt, lens = to_device(inp)
    stream = torch.cuda.Stream()
    ctx = mla.Context(stream=stream)
    try:
        ws = ctx.allocate_workspace(s_q, H)
        out = torch.full((B, s_q, H, 512), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, s_q, H), float("nan"), dtype=torch.float32, device="cuda")
        stream.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            mla.mla_decode(ctx, q, kv, bt, lens, inp.scale, out=out, lse=lse)
        rng = np.random.default_rng(621)
        for rep, new_lens in enumerate([full, [2, 40, 2500], [899, 7, 3000]]):
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
            compare(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
                    f"replay {rep}")
        del graph
        assert ws.data_ptr() == ctx.workspace.data_ptr()
    finally:
        torch.cuda.synchronize()
        ctx.close()


def test_growth_is_refused_during_capture_and_keeps_earlier_graphs_valid(mla):
    import torch

    announce("workspace growth and capture")
    stream = torch.cuda.Stream()
    ctx = mla.Context(stream=stream)
    small_inp = wl.small("gr1", 2, 1, 16, [500, 1200], seed=630)
    big_inp = wl.small("gr4", 2, 4, 32, [500, 1200], seed=631)
    try:
        ctx.reserve(1, 16)
        q, kv, bt, lens = to_device(small_inp)
        out = torch.empty((2, 1, 16, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((2, 1, 16), dtype=torch.float32, device="cuda")
        stream.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            mla.mla_decode(ctx, q, kv, bt, lens, small_inp.scale, out=out, lse=lse)
        # a larger problem while capturing: refused, nothing allocated
        q4, kv4, bt4, lens4 = to_device(big_inp)
        g2 = torch.cuda.CUDAGraph()
        with pytest.raises(mla.MlaError) as ei:
            with torch.cuda.graph(g2, stream=stream):
                mla.mla_decode(ctx, q4, kv4, bt4, lens4, big_inp.scale)
        assert ei.value.code == mla.MLA_ERR_WORKSPACE
        del g2
        # eagerly it grows (a new, larger buffer) ...
        with torch.cuda.stream(stream):
            o4, l4 = mla.mla_decode(ctx, q4, kv4, bt4, lens4, big_inp.scale, seqlens_host=big_inp.seqlens)
        stream.synchronize()
        ro, rl = oracle.mla_decode(big_inp.q, big_inp.kv, big_inp.block_table, big_inp.seqlens, big_inp.scale)
        compare(o4.cpu().numpy().astype(np.float64), l4.cpu().numpy().astype(np.float64), ro, rl, "grown")
        # ... and the graph captured on the smaller buffer still replays right
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ro, rl = oracle.mla_decode(small_inp.q, small_inp.kv, small_inp.block_table, small_inp.seqlens,
                                   small_inp.scale)
        compare(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ro, rl,
                "graph after growth")
        del graph
    finally:
        torch.cuda.synchronize()
        ctx.close()


def test_two_contexts_on_two_streams_overlap(mla):
    """Two contexts, each on a stream of its own (default priority), called
    in turn with no synchronization between the calls, so that their kernels
    may run at the same time: one on the library's own workspace, one on a
    caller's torch buffer.  Each context's partials stay its own: every
    result against the oracle and, bit for bit, against the same call made
    alone."""
    import torch

    announce("two contexts on two streams")
    ia = wl.small("s2a", 4, 1, 16, [3000, 5000, 100, 64], page_size=0, seed=811)
    ib = wl.small("s2b", 2, 4, 16, [2000, 4100], page_size=64, seed=812)
    da, db = to_device(ia), to_device(ib)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    ca, cb = mla.Context(stream=sa), mla.Context(stream=sb)
    try:
        ca.reserve(1, 16)
        buf = cb.allocate_workspace(4, 16)
        torch.cuda.synchronize()
        outs = []
        for rep in range(3):
            oa = torch.full((4, 1, 16, 512), float("nan"), dtype=torch.float32, device="cuda")
            la = torch.full((4, 1, 16), float("nan"), dtype=torch.float32, device="cuda")
            ob = torch.full((2, 4, 16, 512), float("nan"), dtype=torch.float32, device="cuda")
            lb = torch.full((2, 4, 16), float("nan"), dtype=torch.float32, device="cuda")
            sa.wait_stream(torch.cuda.current_stream())
            sb.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(sa):
                mla.mla_decode(ca, *da, ia.scale, out=oa, lse=la, seqlens_host=ia.seqlens)
            with torch.cuda.stream(sb):
                mla.mla_decode(cb, *db, ib.scale, out=ob, lse=lb, seqlens_host=ib.seqlens)
            outs.append((oa, la, ob, lb))
        torch.cuda.synchronize()
        ra = oracle.mla_decode(ia.q, ia.kv, ia.block_table, ia.seqlens, ia.scale)
        rb = oracle.mla_decode(ib.q, ib.kv, ib.block_table, ib.seqlens, ib.scale)
        alone = mla.Context()
        try:
            aa = run_gpu(alone, ia, dev=da)
            ab = run_gpu(alone, ib, dev=db)
        finally:
            alone.close()
        for rep, (oa, la, ob, lb) in enumerate(outs):
            ga = (oa.cpu().numpy().astype(np.float64), la.cpu().numpy().astype(np.float64))
            gb = (ob.cpu().numpy().astype(np.float64), lb.cpu().numpy().astype(np.float64))
            compare(*ga, *ra, f"stream a, call {rep}")
            compare(*gb, *rb, f"stream b, call {rep}")
            assert np.array_equal(ga[0], aa[0]) and np.array_equal(ga[1], aa[1]), f"stream a, call {rep}"
            assert np.array_equal(gb[0], ab[0]) and np.array_equal(gb[1], ab[1]), f"stream b, call {rep}"
        del buf
    finally:
        torch.cuda.synchronize()
        ca.close()
        cb.close()
