"""Pins for the fp64 oracle (CPU only).

The pages print no worked example, so the oracle is tied to what the
mathematics fixes instead: exact special cases, closed forms, invariances, an
independent 50-digit brute force on tiny shapes, and the large-N law that the
synthetic N(0,1) inputs obey.  Each test names the property it relies on.
The two orders it checks against each other are the ones in "FlashMLA-ETAP"
(gist.science technical summary, Methodology, the ETAP bullet).
"""
import math

import mpmath
import numpy as np
import pytest

import oracle
import workloads as wl

D_QK, D_V = wl.D_QK, wl.D_V


def f32(bits):
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def rand_inputs(B, s_q, H, lens, page_size=0, seed=0, poison=True):
    return wl.small("t", B, s_q, H, lens, page_size=page_size, seed=seed)


def run(inp, **kw):
    return oracle.mla_decode(inp.q, inp.kv, inp.block_table, inp.seqlens, inp.scale, **kw)


def logical_rows(inp, b):
    """Rows of sequence b in key order, resolved through the block table by hand."""
    L = int(inp.seqlens[b])
    if inp.block_table is None:
        return inp.kv[b, :L]
    ps = inp.kv.shape[1]
    return np.stack([inp.kv[inp.block_table[b, j // ps], j % ps] for j in range(L)])


# --- 1. the two orders of the pages agree --------------------------------------

@pytest.mark.parametrize("B,s_q,H,lens,ps", [
    (1, 1, 16, [512], 0),
    (3, 1, 16, [1, 77, 300], 0),
    (2, 4, 16, [4, 129], 0),
    (3, 2, 32, [70, 64, 200], 64),
    (2, 4, 16, [1000, 333], 16),
])
def test_standard_and_transposed_orders_agree(B, s_q, H, lens, ps):
    inp = rand_inputs(B, s_q, H, lens, ps, seed=B * 10 + s_q)
    o1, l1 = run(inp)
    o2, l2 = oracle.mla_decode_transposed(inp.q, inp.kv, inp.block_table, inp.seqlens,
                                          inp.scale)
    assert np.isfinite(o1).all() and np.isfinite(l1).all()
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs(l1 - l2)) <= 1e-12


# --- 2. softmax rows sum to one; invisible keys get zero ---------------------

@pytest.mark.parametrize("s_q,ps", [(1, 0), (4, 64)])
def test_probability_rows_sum_to_one(s_q, ps):
    inp = rand_inputs(2, s_q, 16, [4096, 1500], ps, seed=3)
    _, _, p = run(inp, return_probs=True)
    for b in range(2):
        L = int(inp.seqlens[b])
        for t in range(s_q):
            vis = L - s_q + t + 1
            rows = p[b, t]
            assert np.all(np.abs(rows.sum(axis=-1) - 1.0) <= 1e-13)
            assert np.all(rows[:, vis:] == 0.0)
            assert np.all(rows[:, :vis] > 0.0)


# --- 3. a one-key context returns V exactly ----------------------------------

@pytest.mark.parametrize("ps", [0, 64])
def test_single_key_returns_value_row_exactly(ps):
    inp = rand_inputs(3, 1, 16, [1, 1, 1], ps, seed=11)
    o, lse = run(inp)
    for b in range(3):
        row = f32(logical_rows(inp, b)[0])
        for h in range(16):
            assert np.array_equal(o[b, 0, h], row[:D_V])
            qh = f32(inp.q[b, 0, h])
            s0 = float(np.float32(inp.scale)) * math.fsum(qh * row)
            assert abs(lse[b, 0, h] - s0) <= 1e-14 * max(1.0, abs(s0))


# --- 4. independent 50-digit brute force on tiny shapes ----------------------

def brute_force(inp, chans):
    mpmath.mp.dps = 50
    B, s_q, H, _ = inp.q.shape
    sc = mpmath.mpf(float(np.float32(inp.scale)))
    out = np.zeros((B, s_q, H, len(chans)))
    lse = np.zeros((B, s_q, H))
    for b in range(B):
        rows = f32(logical_rows(inp, b))
        L = rows.shape[0]
        for t in range(s_q):
            n = L - s_q + t + 1
            for h in range(H):
                qh = f32(inp.q[b, t, h])
                # bf16 x bf16 products are exact in double; fsum rounds once
                s = [sc * mpmath.mpf(math.fsum(qh * rows[j])) for j in range(n)]
                m = max(s)
                w = [mpmath.exp(x - m) for x in s]
                tot = mpmath.fsum(w)
                lse[b, t, h] = float(m + mpmath.log(tot))
                for ci, c in enumerate(chans):
                    out[b, t, h, ci] = float(
                        mpmath.fsum(w[j] * mpmath.mpf(rows[j, c]) for j in range(n)) / tot)
    return out, lse


@pytest.mark.parametrize("B,s_q,H,lens,ps", [
    (2, 1, 4, [1, 2], 0),
    (2, 1, 2, [3, 5], 16),
    (1, 4, 2, [64], 0),
    (2, 4, 2, [65, 130], 16),
    (1, 1, 16, [130], 64),
])
def test_brute_force_50_digits(B, s_q, H, lens, ps):
    inp = rand_inputs(B, s_q, H, lens, ps, seed=sum(lens))
    chans = [0, 1, 7, 100, 255, 256, 400, 511]
    o, lse = run(inp)
    bo, blse = brute_force(inp, chans)
    assert np.max(np.abs(o[..., chans] - bo)) <= 1e-13
    assert np.max(np.abs(lse - blse)) <= 1e-13


# --- 5. closed forms ---------------------------------------------------------

def test_zero_query_gives_mean_of_values():
    inp = rand_inputs(2, 4, 16, [37, 300], 16, seed=5)
    inp.q[:] = 0
    o, lse = run(inp)
    for b in range(2):
        rows = f32(logical_rows(inp, b))
        L = rows.shape[0]
        for t in range(4):
            n = L - 4 + t + 1
            mean = np.array([math.fsum(rows[:n, c]) for c in range(D_V)]) / n
            assert np.max(np.abs(o[b, t] - mean[None, :])) <= 1e-14
            assert np.max(np.abs(lse[b, t] - math.log(n))) <= 1e-14


def test_identical_keys_give_that_value_and_log_count():
    inp = rand_inputs(1, 1, 16, [999], 0, seed=6)
    inp.kv[0, :999] = inp.kv[0, 5]
    o, lse = run(inp)
    k = f32(inp.kv[0, 5])
    for h in range(16):
        s = float(np.float32(inp.scale)) * math.fsum(f32(inp.q[0, 0, h]) * k)
        assert np.max(np.abs(o[0, 0, h] - k[:D_V])) <= 1e-14 * 999
        assert abs(lse[0, 0, h] - (s + math.log(999))) <= 1e-12


def test_two_keys_logistic_weights():
    inp = rand_inputs(1, 1, 16, [2], 0, seed=8)
    o, lse = run(inp)
    k0, k1 = f32(inp.kv[0, 0]), f32(inp.kv[0, 1])
    sc = float(np.float32(inp.scale))
    for h in range(16):
        qh = f32(inp.q[0, 0, h])
        s0, s1 = sc * math.fsum(qh * k0), sc * math.fsum(qh * k1)
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        expect = w0 * k0[:D_V] + (1.0 - w0) * k1[:D_V]
        assert np.max(np.abs(o[0, 0, h] - expect)) <= 1e-14
        assert abs(lse[0, 0, h] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) <= 1e-14


def test_one_hot_design_reads_back_softmax_weights():
    """q = a_h * e_520 (a rope channel, outside V), key j holds a known score
    there and the one-hot value e_{10j+3}, so O[10j+3] is exactly the softmax
    weight of key j.  A swapped operand, a wrong sign or a lost scale changes
    every entry."""
    n = 6
    inp = rand_inputs(1, 1, 16, [n], 0, seed=9)
    inp.q[:] = 0
    inp.kv[:] = 0
    scores = np.array([1.0, -2.0, 0.5, 3.0, 0.0, -0.25])
    one = wl.f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    for j in range(n):
        inp.kv[0, j, 520] = wl.f32_to_bf16_bits(np.array([scores[j]], np.float32))[0]
        inp.kv[0, j, 10 * j + 3] = one       # value e_{10j+3}
    for h in range(16):
        inp.q[0, 0, h, 520] = wl.f32_to_bf16_bits(np.array([h + 1.0], np.float32))[0]
    o, lse = run(inp)
    sc = float(np.float32(inp.scale))
    for h in range(16):
        z = sc * (h + 1.0) * scores
        p = np.exp(z - z.max()) / np.exp(z - z.max()).sum()
        got = np.array([o[0, 0, h, 10 * j + 3] for j in range(n)])
        assert np.max(np.abs(got - p)) <= 1e-15
        mask = np.ones(D_V, bool)
        mask[[10 * j + 3 for j in range(n)]] = False
        assert np.all(o[0, 0, h, mask] == 0.0)
        assert abs(lse[0, 0, h] - (z.max() + math.log(np.exp(z - z.max()).sum()))) <= 1e-14


# --- 6. invariances ----------------------------------------------------------

def test_split_and_combine_equals_whole():
    rng = np.random.default_rng(0)
    inp = rand_inputs(3, 4, 16, [5000, 130, 64], 0, seed=12)
    full_o, full_l = run(inp)
    for trial in range(3):
        cuts = []
        for b in range(3):
            L = int(inp.seqlens[b])
            c = np.sort(rng.choice(np.arange(1, L), size=3, replace=False))
            cuts.append([0, *c.tolist(), L])
        parts_o, parts_l = [], []
        for s in range(4):
            wb = np.array([cuts[b][s] for b in range(3)], np.int32)
            we = np.array([cuts[b][s + 1] for b in range(3)], np.int32)
            po, pl = run(inp, window=(wb, we))
            parts_o.append(po)
            parts_l.append(pl)
        o, l = oracle.lse_combine(np.stack(parts_l), np.stack(parts_o))
        assert np.max(np.abs(o - full_o)) <= 1e-13
        assert np.max(np.abs(l - full_l)) <= 1e-13


def test_window_past_visible_keys_is_empty_and_weightless():
    inp = rand_inputs(1, 4, 16, [100], 0, seed=13)
    o, l = run(inp, window=(np.array([98], np.int32), np.array([100], np.int32)))
    assert np.all(np.isneginf(l[0, :2])) and np.all(o[0, :2] == 0.0)
    assert np.all(np.isfinite(l[0, 2:]))


def test_page_permutation_and_layout_do_not_change_bits():
    inp = rand_inputs(3, 2, 16, [700, 64, 129], 64, seed=14)
    o1, l1 = run(inp)
    # contiguous layout of the same logical rows
    cap = int(inp.seqlens.max())
    kv = np.zeros((3, cap, D_QK), np.uint16)
    for b in range(3):
        kv[b, : inp.seqlens[b]] = logical_rows(inp, b)
    o2, l2 = oracle.mla_decode(inp.q, kv, None, inp.seqlens, inp.scale)
    # another permutation of the pool
    perm = np.random.default_rng(1).permutation(inp.kv.shape[0])
    inv = np.argsort(perm)
    pool = inp.kv[perm]
    table = np.where(inp.block_table < inp.kv.shape[0],
                     inv[np.minimum(inp.block_table, inp.kv.shape[0] - 1)],
                     inp.block_table).astype(np.int32)
    o3, l3 = oracle.mla_decode(inp.q, pool, table, inp.seqlens, inp.scale)
    for o, l in ((o2, l2), (o3, l3)):
        assert np.array_equal(o, o1) and np.array_equal(l, l1)


def test_multi_token_row_equals_single_token_at_shorter_length():
    L = 333
    inp = rand_inputs(1, 4, 16, [L], 0, seed=15)
    o4, l4 = run(inp)
    for t in range(4):
        o1, l1 = oracle.mla_decode(inp.q[:, t:t + 1], inp.kv, None,
                                   np.array([L - 3 + t], np.int32), inp.scale)
        assert np.array_equal(o1[:, 0], o4[:, t]) and np.array_equal(l1[:, 0], l4[:, t])


def test_head_permutation_permutes_rows():
    inp = rand_inputs(2, 1, 16, [100, 50], 0, seed=16)
    o, l = run(inp)
    perm = np.random.default_rng(2).permutation(16)
    q2 = inp.q[:, :, perm].copy()
    o2, l2 = oracle.mla_decode(q2, inp.kv, None, inp.seqlens, inp.scale)
    assert np.array_equal(o2, o[:, :, perm]) and np.array_equal(l2, l[:, :, perm])


def test_common_score_shift_leaves_output_and_shifts_lse():
    """Adding the same amount to every score of a row (here through a rope
    channel where q = 1 and every key holds c) is a softmax invariance."""
    inp = rand_inputs(1, 1, 16, [200], 0, seed=17)
    inp.q[..., 575] = 0
    inp.kv[0, :, 575] = 0
    o1, l1 = run(inp)
    c = 8.0
    inp.q[..., 575] = wl.f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    inp.kv[0, :, 575] = wl.f32_to_bf16_bits(np.array([c], np.float32))[0]
    o2, l2 = run(inp)
    assert np.max(np.abs(o2 - o1)) <= 1e-14
    assert np.max(np.abs(l2 - l1 - float(np.float32(inp.scale)) * c)) <= 1e-13


# --- 7. the large-N law of the synthetic inputs ------------------------------

@pytest.mark.slow
def test_large_context_gaussian_tilt_law():
    """With k ~ N(0, I) and v = k[:512], s_j = a.k_j with a = scale*q, so
    E[e^s] = e^{|a|^2/2}: LSE -> ln N + |a|^2/2 (std ~ sqrt((e^{|a|^2}-1)/N)),
    and the tilted mean E[k e^s]/E[e^s] = a: O -> scale*q[:512] with residual
    rms ~ sqrt(e^{|a|^2}/N).  Gates at 6 sigma / 25 %."""
    N = 65536
    w = wl.Workload("law", 1, 1, 16, N, 0, 1002)
    inp = wl.make_inputs(w)
    o, lse = run(inp)
    sc = float(np.float32(inp.scale))
    a2 = np.array([sc * sc * float(np.sum(f32(inp.q[0, 0, h]) ** 2)) for h in range(16)])
    dev = lse[0, 0] - (math.log(N) + a2 / 2)
    assert np.all(np.abs(dev) <= 6 * np.sqrt((np.exp(a2) - 1) / N))
    resid = o[0, 0] - sc * f32(inp.q[0, 0])[:, :D_V]
    rms = np.sqrt(np.mean(resid ** 2, axis=1))
    pred = np.sqrt(np.exp(a2) / N)
    assert np.all(np.abs(rms / pred - 1.0) <= 0.25)
