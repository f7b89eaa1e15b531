"""Pins of the fp64 oracle for the MLA steps around the attention
(``oracle/steps.py``): exact rational arithmetic on sampled outputs, identity
and one-hot weights, exact scalings, placement invariances, a hand-worked
append, and the absorbed form of MLA attention agreeing with the explicit
one (keys and values up-projected per head).  CPU only."""
from fractions import Fraction

import numpy as np

import workloads as wl
from oracle import steps


def rand_bf16(rng, shape, scale=1.0):
    return wl.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def frac_bf16(bits):
    """Exact rational value of one bf16 bit pattern."""
    return Fraction(float(steps.bf16_bits_to_f64(np.array([bits], np.uint16))[0]))


# ---------------------------------------------------------------- rounding

def test_bf16_rounding_matches_the_fp32_bit_rule():
    # For float32 inputs, round-to-nearest-even to bf16 is the classic bit
    # rule: add 0x7FFF plus the lowest kept bit, drop the low 16 bits.
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-39).astype(np.float32),  # subnormal
                        np.float32([0.0, -0.0, 1.0, -3.5, 65504.0, 3.0e38])])
    bits = x.view(np.uint32).astype(np.uint64)
    rule = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(steps.f64_to_bf16_bits(x.astype(np.float64)), rule)


def test_bf16_rounding_ties_and_no_double_rounding():
    one = 1.0
    cases = {
        one + 2.0 ** -8: one,                          # tie -> even (1)
        one + 3 * 2.0 ** -8: one + 2.0 ** -6,          # tie -> even (mantissa 2)
        one + 2.0 ** -8 + 2.0 ** -40: one + 2.0 ** -7,  # above the tie: up (fp32 first would tie down)
        -(one + 2.0 ** -8 + 2.0 ** -40): -(one + 2.0 ** -7),
        3.3895313892515355e38 * (1 + 2.0 ** -9): 3.3895313892515355e38,  # under max + half a place
        3.3895313892515355e38 + 2.0 ** 119: np.inf,  # tie at the top: even is 2^128
        3.3895313892515355e38 * (1 + 2.0 ** -8): np.inf,
    }
    got = steps.f64_to_bf16_bits(np.array(list(cases.keys())))
    want = steps.f64_to_bf16_bits(np.array(list(cases.values())))
    assert np.array_equal(got, want)
    assert steps.bf16_bits_to_f64(got[2]) == one + 2.0 ** -7


# ---------------------------------------------------------------- absorb

def test_absorb_q_exact_on_sampled_outputs():
    rng = np.random.default_rng(7)
    rows, H, dn = 3, 2, 32
    qn, qr = rand_bf16(rng, (rows, H, dn)), rand_bf16(rng, (rows, H, 64))
    w = rand_bf16(rng, (H, 512, dn), 0.1)
    q_lat, q_bits = steps.absorb_q(qn, qr, w)
    for _ in range(40):
        r, h, c = int(rng.integers(rows)), int(rng.integers(H)), int(rng.integers(512))
        exact = sum(frac_bf16(qn[r, h, d]) * frac_bf16(w[h, c, d]) for d in range(dn))
        assert q_lat[r, h, c] == float(exact)  # the products are exact and the sum short
    assert np.array_equal(q_bits[..., 512:], qr)


def test_absorb_q_identity_weights_copy_the_query():
    rng = np.random.default_rng(8)
    rows, H, dn = 5, 3, 64
    qn, qr = rand_bf16(rng, (rows, H, dn)), rand_bf16(rng, (rows, H, 64))
    w = np.zeros((H, 512, dn), np.uint16)
    one = wl.f32_to_bf16_bits(np.float32([1.0]))[0]
    for h in range(H):
        w[h, np.arange(dn), np.arange(dn)] = one
    q_lat, q_bits = steps.absorb_q(qn, qr, w)
    assert np.array_equal(q_bits[..., :dn], qn)
    assert not q_lat[..., dn:].any()
    assert np.array_equal(q_bits[..., 512:], qr)


def test_absorb_q_scales_exactly():
    rng = np.random.default_rng(9)
    qn, qr = rand_bf16(rng, (4, 2, 32)), rand_bf16(rng, (4, 2, 64))
    w = rand_bf16(rng, (2, 512, 32))
    a, _ = steps.absorb_q(qn, qr, w)
    qn4 = wl.f32_to_bf16_bits(steps.bf16_bits_to_f64(qn).astype(np.float32) * 4)
    b, _ = steps.absorb_q(qn4, qr, w)
    assert np.array_equal(b, 4 * a)


# ---------------------------------------------------------------- project

def test_project_out_exact_on_sampled_outputs():
    rng = np.random.default_rng(10)
    rows, H, dv = 2, 2, 64
    o = rng.standard_normal((rows, H, 512)).astype(np.float32)
    w = rand_bf16(rng, (H, dv, 512), 0.05)
    out = steps.project_out(o, w)
    for _ in range(30):
        r, h, e = int(rng.integers(rows)), int(rng.integers(H)), int(rng.integers(dv))
        exact = sum(Fraction(float(o[r, h, c])) * frac_bf16(w[h, e, c]) for c in range(512))
        assert abs(out[r, h, e] - float(exact)) <= 1e-15 * float(sum(
            abs(Fraction(float(o[r, h, c])) * frac_bf16(w[h, e, c])) for c in range(512)))


def test_project_out_abs_exact_on_sampled_outputs():
    """sum_c |o w| (the scale of each projected output's rounding error)
    equals the exact rational sum of the absolute products; inputs of both
    signs, so a missing absolute value, a wrong head or a wrong axis shows."""
    rng = np.random.default_rng(14)
    rows, H, dv = 3, 3, 48
    o = rng.standard_normal((rows, H, 512)).astype(np.float32)
    w = rand_bf16(rng, (H, dv, 512), 0.05)
    mag = steps.project_out_abs(o, w)
    assert mag.shape == (rows, H, dv)
    for _ in range(30):
        r, h, e = int(rng.integers(rows)), int(rng.integers(H)), int(rng.integers(dv))
        exact = sum(abs(Fraction(float(o[r, h, c])) * frac_bf16(w[h, e, c])) for c in range(512))
        # 512 nonnegative terms: the float64 sum is within 512 ulps of it
        assert abs(mag[r, h, e] - float(exact)) <= 512 * 2.0 ** -52 * float(exact)


def test_project_out_abs_bounds_the_projection():
    """|sum o w| <= sum |o w| (triangle inequality), with equality exactly
    where every product has one sign: nonnegative o and w, or o negated."""
    rng = np.random.default_rng(15)
    o = rng.standard_normal((4, 2, 512)).astype(np.float32)
    w = rand_bf16(rng, (2, 32, 512))
    assert np.all(np.abs(steps.project_out(o, w)) <= steps.project_out_abs(o, w) * (1 + 1e-12))
    wpos = w & np.uint16(0x7FFF)  # clear the sign bit: |w| in bf16
    opos = np.abs(o)
    assert np.allclose(steps.project_out(opos, wpos), steps.project_out_abs(o, w), rtol=1e-13, atol=0)
    assert np.allclose(-steps.project_out(-opos, wpos), steps.project_out_abs(-o, w), rtol=1e-13, atol=0)


def test_project_out_one_hot_and_identity():
    rng = np.random.default_rng(11)
    H, dv = 2, 128
    w = rand_bf16(rng, (H, dv, 512))
    o = np.zeros((512, H, 512), np.float32)
    o[np.arange(512), :, np.arange(512)] = 1.0  # row r: one-hot at channel r
    out = steps.project_out(o, w)
    assert np.array_equal(out, steps.bf16_bits_to_f64(w).transpose(2, 0, 1))
    eye = np.zeros((H, dv, 512), np.uint16)
    one = wl.f32_to_bf16_bits(np.float32([1.0]))[0]
    eye[:, np.arange(dv), np.arange(dv)] = one
    o2 = rng.standard_normal((3, H, 512)).astype(np.float32)
    assert np.array_equal(steps.project_out(o2, eye), o2[..., :dv].astype(np.float64))


# ---------------------------------------------------------------- append

def test_append_hand_worked_example():
    # Two sequences, contiguous capacity 4, one 576-wide row per key; the
    # rows are tagged by their first channel.  Lengths after the append are
    # 3 and 2 with s_q = 2: sequence 0 gets keys 1 and 2, sequence 1 keys 0
    # and 1; key 0 of sequence 0 and keys 3 stay as they were.
    kv = np.zeros((2, 4, 576), np.uint16)
    kv[:, :, 0] = [[10, 11, 12, 13], [20, 21, 22, 23]]
    new = np.zeros((2, 2, 576), np.uint16)
    new[:, :, 0] = [[100, 101], [200, 201]]
    out = steps.append_kv(kv, None, np.array([3, 2]), new)
    assert out[:, :, 0].tolist() == [[10, 100, 101, 13], [200, 201, 22, 23]]
    assert kv[:, :, 0].tolist() == [[10, 11, 12, 13], [20, 21, 22, 23]]  # input untouched


def test_append_paged_matches_contiguous_and_touches_only_new_rows():
    rng = np.random.default_rng(12)
    B, s_q, cap, page = 3, 3, 64, 16
    lens = np.array([5, 64, 33])
    kv_c = rng.integers(0, 1 << 16, (B, cap, 576), dtype=np.uint16)
    perm = rng.permutation(B * cap // page)
    table = perm.reshape(B, cap // page).astype(np.int32)
    pool = np.empty((B * cap // page, page, 576), np.uint16)
    for b in range(B):
        for j in range(cap // page):
            pool[table[b, j]] = kv_c[b, j * page:(j + 1) * page]
    new = rng.integers(0, 1 << 16, (B, s_q, 576), dtype=np.uint16)
    out_c = steps.append_kv(kv_c, None, lens, new)
    out_p = steps.append_kv(pool, table, lens, new)
    for b in range(B):
        logical = np.concatenate([out_p[table[b, j]] for j in range(cap // page)])
        assert np.array_equal(logical, out_c[b])
        changed = np.flatnonzero((out_c[b] != kv_c[b]).any(axis=1))
        assert set(changed) <= set(range(lens[b] - s_q, lens[b]))
        assert np.array_equal(out_c[b, lens[b] - s_q:lens[b]], new[b])
    # appending the same rows again changes nothing more
    assert np.array_equal(steps.append_kv(out_c, None, lens, new), out_c)


# ---------------------------------------------------------------- MLA equivalence

def test_absorbed_attention_equals_explicit_mla():
    """Scores against the up-projected keys and values up-projected per key
    (explicit MLA) equal the absorbed form: the absorbed query against the
    latent rows, and the value projection applied once to the latent output."""
    rng = np.random.default_rng(13)
    L, H, dn, dv = 40, 2, 32, 64
    c_kv = steps.bf16_bits_to_f64(rand_bf16(rng, (L, 512)))
    k_rope = steps.bf16_bits_to_f64(rand_bf16(rng, (L, 64)))
    qn_bits, qr_bits = rand_bf16(rng, (1, H, dn)), rand_bf16(rng, (1, H, 64))
    w_uk, w_uv = rand_bf16(rng, (H, 512, dn), 0.05), rand_bf16(rng, (H, dv, 512), 0.05)
    scale = 1.0 / np.sqrt(dn + 64)
    qn, qr = steps.bf16_bits_to_f64(qn_bits)[0], steps.bf16_bits_to_f64(qr_bits)[0]
    wk, wv = steps.bf16_bits_to_f64(w_uk), steps.bf16_bits_to_f64(w_uv)
    # explicit: per-head keys k_nope[j][d] = sum_c w_uk[h][c][d] c_kv[j][c], values v[j][e]
    out_explicit = np.zeros((H, dv))
    for h in range(H):
        k_nope = c_kv @ wk[h]                       # [L][dn]
        v = c_kv @ wv[h].T                          # [L][dv]
        s = scale * (k_nope @ qn[h] + k_rope @ qr[h])
        p = np.exp(s - s.max())
        out_explicit[h] = (p / p.sum()) @ v
    # absorbed: latent query, attention over the latent rows, then project
    q_lat, _ = steps.absorb_q(qn_bits, qr_bits, w_uk)
    o = np.zeros((1, H, 512))
    for h in range(H):
        s = scale * (c_kv @ q_lat[0, h] + k_rope @ qr[h])
        p = np.exp(s - s.max())
        o[0, h] = (p / p.sum()) @ c_kv
    out_absorbed = np.einsum("rhc,hec->rhe", o, wv)[0]
    assert np.max(np.abs(out_absorbed - out_explicit)) <= 1e-12 * np.max(np.abs(out_explicit))
