"""Helpers for the GPU tests: move seeded inputs to the device, run the
library through its C ABI, compare against the oracle."""
from __future__ import annotations

import numpy as np

import workloads as wl

# Parity bar for fp32 outputs against the fp64 oracle.
O_RMSE_MAX = 1e-4
O_MAXABS_MAX = 1e-3
LSE_MAXABS_MAX = 1e-4


def to_device(inp: wl.Inputs):
    return wl.to_torch(inp, "cuda:0")


def run_gpu(ctx, inp: wl.Inputs, dev=None, host_lens=True, out=None, lse=None):
    import torch

    import decode_attention_mla_amd as mla

    q, kv, bt, lens = dev if dev is not None else to_device(inp)
    # Outputs start as NaN, so a row the library never writes fails the check.
    B, s_q, H = inp.q.shape[:3]
    if out is None:
        out = torch.full((B, s_q, H, 512), float("nan"), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.full((B, s_q, H), float("nan"), dtype=torch.float32, device=q.device)
    o, l = mla.mla_decode(ctx, q, kv, bt, lens, inp.scale, out=out, lse=lse,
                          seqlens_host=inp.seqlens if host_lens else None)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64)


def compare(o, l, ro, rl, what=""):
    err = o - ro
    rmse = float(np.sqrt(np.mean(err ** 2)))
    maxabs = float(np.max(np.abs(err)))
    lerr = float(np.max(np.abs(l - rl)))
    assert np.isfinite(o).all() and np.isfinite(l).all(), f"{what}: non-finite output"
    assert rmse <= O_RMSE_MAX, f"{what}: O rmse {rmse:.3g}"
    assert maxabs <= O_MAXABS_MAX, f"{what}: O max-abs {maxabs:.3g}"
    assert lerr <= LSE_MAXABS_MAX, f"{what}: LSE max-abs {lerr:.3g}"
    return rmse, maxabs, lerr
