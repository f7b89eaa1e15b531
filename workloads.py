"""Seeded synthetic inputs for MLA decode attention.

This module only draws random numbers and lays them out; it contains none of
the attention arithmetic.  Both the fp64 oracle (``oracle/``) and the HIP
library are fed from here, so they read the same bf16 bits.

The workloads are the decode shapes of "FlashMLA-ETAP" (gist.science technical
summary, Problem Statement and Results: DeepSeek-R1, 16 heads per GPU after the
128-head split over 8 GPUs, short query, contexts from 512 to 64K, batch 16
and 32; arxivlens page, Limitations: head dimension 576).  The latent KV row is
576 bf16 channels; keys use all of them and values use the first 512.

Recipe (per workload seed ``s``):

* ``rng = np.random.default_rng(s)``; ragged sequence lengths are drawn first
  as inclusive uniform integers, then Q as float32 standard normals.
* The KV rows of sequence ``b`` come from their own stream
  ``np.random.default_rng([s, 1, b])`` so one sequence can be regenerated
  without the rest (the oracle samples sequences at full size this way).
* Paged layouts assign pages through ``np.random.default_rng([s, 2])``'s
  permutation of all page ids, in sequence order.
* Every float32 draw is rounded to bfloat16 with round-to-nearest-even.

Unused cache slots (the tail of the last page, contiguous rows past the
sequence length) and unused block-table entries can be poisoned with NaN and
an out-of-range page id: a correct kernel never reads them.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple, Union

import numpy as np

D_QK = 576           # latent row width: 512 value channels + 64 rope channels
D_V = 512            # value channels = the first 512 channels of the row
BF16_NAN = 0x7FC0    # quiet NaN in bfloat16
POISON_PAGE = 0x3FFFFFFF  # block-table filler past a sequence's last page


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    s_q: int
    heads: int
    seqlen: Union[int, Tuple[int, int]]  # fixed, or inclusive uniform range
    page_size: int                       # 0 means contiguous [B, N, 576]
    seed: int

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(D_QK)))


# The shapes the bench, the counter runs and the parity tests use: the five
# decode shapes at 16 heads per GPU, then the headline context at 64 and 128
# heads (the 128-head model on two GPUs and on one; the same summary's
# Problem Statement).
WORKLOADS = {
    w.name: w
    for w in (
        Workload("mla_bs1_ctx512", 1, 1, 16, 512, 0, 1000),
        Workload("mla_bs16_ctx4096", 16, 1, 16, 4096, 0, 1001),
        Workload("mla_bs16_ctx65536", 16, 1, 16, 65536, 0, 1002),
        Workload("mla_bs64_ragged1k_32k_paged64", 64, 1, 16, (1024, 32768), 64, 1003),
        Workload("mla_bs32_sq4_ctx16384", 32, 4, 16, 16384, 0, 1004),
        Workload("mla_bs16_h64_ctx65536", 16, 1, 64, 65536, 0, 1005),
        Workload("mla_bs16_h128_ctx65536", 16, 1, 128, 65536, 0, 1006),
    )
}
HEADLINE = "mla_bs16_ctx65536"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_seqlens(w: Workload) -> np.ndarray:
    rng = np.random.default_rng(w.seed)
    if isinstance(w.seqlen, tuple):
        lo, hi = w.seqlen
        return rng.integers(lo, hi + 1, size=w.batch, dtype=np.int64).astype(np.int32)
    return np.full(w.batch, w.seqlen, dtype=np.int32)


def draw_q(w: Workload) -> np.ndarray:
    rng = np.random.default_rng(w.seed)
    if isinstance(w.seqlen, tuple):
        rng.integers(w.seqlen[0], w.seqlen[1] + 1, size=w.batch, dtype=np.int64)
    q = rng.standard_normal((w.batch, w.s_q, w.heads, D_QK), dtype=np.float32)
    return f32_to_bf16_bits(q)


def sequence_rows(seed: int, b: int, length: int) -> np.ndarray:
    """The logical latent rows [length, 576] (bf16 bits) of sequence b."""
    rng = np.random.default_rng([seed, 1, b])
    return f32_to_bf16_bits(rng.standard_normal((length, D_QK), dtype=np.float32))


@dataclasses.dataclass
class Inputs:
    workload: Workload
    q: np.ndarray                      # [B, s_q, H, 576] uint16 (bf16 bits)
    kv: np.ndarray                     # [B, cap, 576] or pool [P, page, 576] uint16
    block_table: Optional[np.ndarray]  # [B, max_pages] int32, or None
    seqlens: np.ndarray                # [B] int32
    scale: float

    @property
    def page_size(self) -> int:
        return self.workload.page_size

    @property
    def kv_bytes(self) -> int:
        """Bytes of latent rows that attention must read: sum of L_b rows."""
        return int(self.seqlens.astype(np.int64).sum()) * D_QK * 2


def make_inputs(
    w: Workload,
    poison: bool = False,
    seqlens: Optional[Sequence[int]] = None,
    capacity: Optional[int] = None,
) -> Inputs:
    """Build the full input set of a workload.

    ``seqlens`` overrides the drawn lengths (small test shapes);
    ``capacity`` pads the contiguous layout to more rows than the longest
    sequence.  With ``poison`` every slot no sequence owns holds NaN and
    every unused block-table entry an out-of-range page id.
    """
    lens = draw_seqlens(w) if seqlens is None else np.asarray(seqlens, dtype=np.int32)
    assert lens.shape == (w.batch,)
    q = draw_q(w)
    fill = BF16_NAN if poison else 0
    if w.page_size == 0:
        cap = int(lens.max()) if capacity is None else int(capacity)
        kv = np.full((w.batch, cap, D_QK), fill, dtype=np.uint16)
        for b in range(w.batch):
            kv[b, : lens[b]] = sequence_rows(w.seed, b, int(lens[b]))
        return Inputs(w, q, kv, None, lens, w.scale)

    ps = w.page_size
    npages = [(int(n) + ps - 1) // ps for n in lens]
    total = int(sum(npages))
    perm = np.random.default_rng([w.seed, 2]).permutation(total).astype(np.int32)
    max_pages = max(npages) if capacity is None else (int(capacity) + ps - 1) // ps
    table = np.full((w.batch, max_pages), POISON_PAGE if poison else 0, dtype=np.int32)
    pool = np.full((total, ps, D_QK), fill, dtype=np.uint16)
    off = 0
    for b in range(w.batch):
        n = int(lens[b])
        ids = perm[off : off + npages[b]]
        off += npages[b]
        table[b, : npages[b]] = ids
        rows = sequence_rows(w.seed, b, n)
        padded = np.full((npages[b] * ps, D_QK), fill, dtype=np.uint16)
        padded[:n] = rows
        pool[ids] = padded.reshape(npages[b], ps, D_QK)
    return Inputs(w, q, pool, table, lens, w.scale)


def to_torch(inp: Inputs, device="cuda:0"):
    """Upload the arrays as torch tensors (bf16 views of the bit patterns)."""
    import torch

    dev = torch.device(device)
    q = torch.from_numpy(inp.q.view(np.int16)).to(dev).view(torch.bfloat16)
    kv = torch.from_numpy(inp.kv.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = None if inp.block_table is None else torch.from_numpy(inp.block_table).to(dev)
    lens = torch.from_numpy(inp.seqlens).to(dev)
    return q, kv, bt, lens


def small(name: str, batch: int, s_q: int, heads: int, seqlens: Sequence[int],
          page_size: int = 0, seed: int = 7) -> Inputs:
    """A small test shape with explicit per-sequence lengths."""
    w = Workload(name, batch, s_q, heads, int(max(seqlens)), page_size, seed)
    return make_inputs(w, poison=True, seqlens=seqlens)


# ---------------------------------------------------------------------------
# Inputs of the MLA steps around the attention (query absorption, output
# up-projection, cache append).  The per-head widths are not fixed by the
# pages; DeepSeek-V3's 128 (query without rotary part) and 128 (value head)
# are the defaults.  Weights are standard normals scaled by 1/sqrt(fan-in),
# so the absorbed query has unit variance like the attention's query and
# the projected output the magnitude of the latent output.

D_NOPE = 128
D_VHEAD = 128
D_ROPE = D_QK - D_V


@dataclasses.dataclass
class StepInputs:
    q_nope: np.ndarray    # [rows, H, d_nope] uint16
    q_rope: np.ndarray    # [rows, H, 64] uint16
    w_uk: np.ndarray      # [H, 512, d_nope] uint16
    w_uv: np.ndarray      # [H, d_v, 512] uint16
    new_rows: np.ndarray  # [B, s_q, 576] uint16: latent rows of the new tokens
    o: np.ndarray         # [rows, H, 512] float32: stand-in latent attention output


def make_step_inputs(seed: int, batch: int, s_q: int, heads: int,
                     d_nope: int = D_NOPE, d_v: int = D_VHEAD) -> StepInputs:
    """Seeded step inputs; rows = batch * s_q.  Streams: ``[seed, 3, k]`` for
    the k-th array, so each is independent of the others' sizes."""
    rows = batch * s_q

    def normal(k, shape, scale=1.0):
        return np.random.default_rng([seed, 3, k]).standard_normal(shape, dtype=np.float32) * np.float32(scale)

    return StepInputs(
        q_nope=f32_to_bf16_bits(normal(0, (rows, heads, d_nope))),
        q_rope=f32_to_bf16_bits(normal(1, (rows, heads, D_ROPE))),
        w_uk=f32_to_bf16_bits(normal(2, (heads, D_V, d_nope), 1.0 / math.sqrt(d_nope))),
        w_uv=f32_to_bf16_bits(normal(3, (heads, d_v, D_V), 1.0 / math.sqrt(D_V))),
        new_rows=f32_to_bf16_bits(normal(4, (batch, s_q, D_QK))),
        o=normal(5, (rows, heads, D_V)),
    )


def bf16_tensor(bits: np.ndarray, device="cuda:0"):
    """Upload uint16 bf16 bit patterns as a torch bfloat16 tensor."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)
