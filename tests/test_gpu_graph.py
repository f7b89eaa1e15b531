"""mla_decode inside a captured HIP graph.

With device lengths only (no host copy) a call does no host synchronization,
allocation or memset once the context has reserved its workspace, so a
decode loop can capture it.  The graph is replayed several times with new
lengths and queries written in place between replays, eager work and
synchronizations in between, and every replay is checked against the fp64
oracle.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import compare, to_device

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


# s_q = 2: two row blocks (the two-key-group kernel); s_q = 1: one row block,
# launched blind with three sequences, so the kernel that sends a
# workgroup's next segment ahead of the merge.
@pytest.mark.parametrize("s_q", [2, 1])
@pytest.mark.parametrize("page_size", [0, 16])
def test_graph_replays_match_the_oracle(page_size, s_q):
    import torch

    import decode_attention_mla_amd as mla

    B, H = 3, 16
    full = [700, 33, 2048]
    announce(f"graph capture page_size={page_size} s_q={s_q}")
    inp = wl.small("g", B, s_q, H, full, page_size=page_size, seed=11)
    q, kv, bt, lens = to_device(inp)
    stream = torch.cuda.Stream()
    ctx = mla.Context(stream=stream)
    eager = mla.Context()
    try:
        ctx.reserve(s_q, H)
        out = torch.full((B, s_q, H, 512), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, s_q, H), float("nan"), dtype=torch.float32, device="cuda")
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            mla.mla_decode(ctx, q, kv, bt, lens, inp.scale, out=out, lse=lse)  # warm-up
        stream.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            mla.mla_decode(ctx, q, kv, bt, lens, inp.scale, out=out, lse=lse)

        rng = np.random.default_rng(12)
        for rep, new_lens in enumerate([full, [2, 33, 1500], [640, 17, 2047], [699, 2, 64]]):
            # Inputs change in place; the cache rows and pages stay (lengths
            # only shrink, so every key read is a real one).
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
                    ro, rl, f"replay {rep} lens={new_lens}")
            # eager work on the default stream between replays
            eo, el = mla.mla_decode(eager, q, kv, bt, lens, inp.scale, seqlens_host=inp.seqlens)
            torch.cuda.synchronize()
            compare(eo.cpu().numpy().astype(np.float64), el.cpu().numpy().astype(np.float64),
                    ro, rl, f"eager {rep}")
    finally:
        torch.cuda.synchronize()
        ctx.close()
        eager.close()
