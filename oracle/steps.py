"""fp64 CPU oracle for the MLA steps around the attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may use this module; the product library never does, and this module
imports nothing from it.

What MLA's low-rank joint compression implies ("FlashMLA-ETAP", gist.science
technical summary, Integration and Implementation: one latent KV row per
token, shared by all heads; arxivlens page, Limitations: head dimension 576):

* the latent row is read as 512 compressed-KV channels followed by 64
  rotary-key channels (the value part is the first 512 channels, as in the
  attention);
* the score of head h against key j is q_nope[h] . (W_UK[h] c_j) +
  q_rope[h] . k_rope_j, which equals [W_UK[h]^T q_nope[h], q_rope[h]] .
  [c_j, k_rope_j]: the absorbed query (``absorb_q``) dotted with the latent
  row;
* the head's output is W_UV[h] (sum_j p_j c_j) = W_UV[h] o[h]: the value
  up-projection applied to the latent attention output (``project_out``);
* each decode step appends the new tokens' latent rows to the cache
  (``append_kv``), as keys L_b - s_q .. L_b - 1.

These are the plain definitions, written out in float64 from the same bf16
bits the GPU reads.  The per-head sizes d_nope and d_v are arguments (the
pages do not fix them).  Parity status: pinned (``tests/test_oracle_steps.py``:
exact rational brute force on tiny shapes, identity and one-hot weights,
scaling, placement invariances, and the absorbed and explicit forms of MLA
attention agreeing).
"""
from __future__ import annotations

import numpy as np

LATENT = 512
ROPE = 64
ROW = LATENT + ROPE


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64, exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest bf16 (ties to even), as bit patterns.

    bf16 keeps 8 significant bits: write |x| = m 2^e with 1/2 <= m < 1; the
    result is rint(m 2^8) 2^(e-8) (rint rounds half to even), with the
    subnormal step 2^-133 below 2^-126 and infinity from the largest finite
    value plus half its last place on.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    m, e = np.frexp(x)
    normal = np.abs(x) >= 2.0 ** -126
    out[normal] = np.rint(m[normal] * 256.0) * np.exp2(e[normal] - 8.0)
    out[~normal] = np.rint(x[~normal] / 2.0 ** -133) * 2.0 ** -133
    big = np.abs(out) > 3.3895313892515355e38  # (2 - 2^-7) 2^127, the largest bf16
    out[big] = np.copysign(np.inf, x[big])
    out[np.isnan(x)] = np.nan
    return (out.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def append_kv(kv: np.ndarray, block_table, seqlens, new_rows: np.ndarray) -> np.ndarray:
    """The cache after appending: token t of sequence b becomes key
    L_b - s_q + t.  kv: uint16 [B][cap][576] (contiguous) or pool
    [P][page][576] (paged, with block_table [B][max_pages]); new_rows: uint16
    [B][s_q][576]; seqlens: the lengths including the new tokens.  Returns a
    new array; the input is not modified."""
    out = np.array(kv, copy=True)
    B, s_q = new_rows.shape[:2]
    for b in range(B):
        for t in range(s_q):
            key = int(seqlens[b]) - s_q + t
            if block_table is None:
                out[b, key] = new_rows[b, t]
            else:
                page_size = kv.shape[1]
                out[int(block_table[b][key // page_size]), key % page_size] = new_rows[b, t]
    return out


def absorb_q(q_nope: np.ndarray, q_rope: np.ndarray, w_uk: np.ndarray):
    """Absorbed query.  q_nope uint16 [rows][H][d_nope], q_rope uint16
    [rows][H][64], w_uk uint16 [H][512][d_nope] (row c: the weights of latent
    channel c).  Returns (q_lat, q_bits): q_lat float64 [rows][H][512] =
    sum_d q_nope[r][h][d] w_uk[h][c][d] exactly (each product of two bf16 is
    exact in float64), and q_bits uint16 [rows][H][576] = [bf16(q_lat),
    q_rope]."""
    qn = bf16_bits_to_f64(q_nope)
    w = bf16_bits_to_f64(w_uk)
    q_lat = np.einsum("rhd,hcd->rhc", qn, w)
    rows, H = q_nope.shape[:2]
    q_bits = np.empty((rows, H, ROW), dtype=np.uint16)
    q_bits[..., :LATENT] = f64_to_bf16_bits(q_lat)
    q_bits[..., LATENT:] = q_rope
    return q_lat, q_bits


def project_out(o: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """Output up-projection.  o float32 [rows][H][512], w_uv uint16
    [H][d_v][512] (row e: the weights of value channel e).  Returns float64
    [rows][H][d_v] = sum_c o[r][h][c] w_uv[h][e][c]."""
    return np.einsum("rhc,hec->rhe", np.asarray(o, dtype=np.float64), bf16_bits_to_f64(w_uv))


def project_out_abs(o: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """sum_c |o[r][h][c] w_uv[h][e][c]|: the scale of each output's rounding
    error."""
    return np.einsum("rhc,hec->rhe", np.abs(np.asarray(o, dtype=np.float64)), np.abs(bf16_bits_to_f64(w_uv)))
