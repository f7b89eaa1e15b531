"""CPU-only checks of the C ABI: symbols, argument validation, split plan.

No GPU is touched: mla_validate and mla_plan are host code, and the library
loads without a device.
"""
import ctypes
import re

import numpy as np
import pytest

import decode_attention_mla_amd as mla


@pytest.fixture(scope="module")
def lib():
    return mla.load()


def declared_functions():
    text = open(mla.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(mla_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("mla_decode", "mla_ctx_create", "mla_ctx_destroy", "mla_validate", "mla_plan"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in mla_decode.h but not exported"


def declared_constants():
    """Every `MLA_NAME = value` of the header's enums and defines."""
    text = open(mla.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    found = dict(re.findall(r"\b(MLA_[A-Z0-9_]+)\s*=\s*(-?\d+)", text))
    found.update(re.findall(r"#define\s+(MLA_[A-Z0-9_]+)\s+(-?\d+)\b", text))
    return {k: int(v) for k, v in found.items()}


def test_binding_constants_match_the_header():
    """The binding's status codes and option ids are the header's values."""
    consts = declared_constants()
    for name in ("MLA_OK", "MLA_ERR_INVALID_ARG", "MLA_ERR_UNSUPPORTED", "MLA_ERR_WORKSPACE", "MLA_ERR_HIP",
                 "MLA_OPT_NUM_SPLITS", "MLA_OPT_MIN_CHUNK", "MLA_OPT_KERNEL_TIMING", "MLA_OPT_P_BF16"):
        assert name in consts, f"{name} missing from mla_decode.h"
        assert getattr(mla, name) == consts[name], name


def test_version(lib):
    assert "gfx950" in mla.version()


# --- argument validation ------------------------------------------------------

A = 0x10000  # stand-in device addresses: never dereferenced by mla_validate


def validate(q=A, kv=A, bt=None, seqlens=A, scale=1 / 24, out=A, lse=A, **kw):
    args = dict(batch=2, s_q=1, num_heads=16, page_size=0, kv_capacity=128, num_pages=0,
                max_pages=0, seqlens_host=None)
    dims = {k: kw.pop(k) for k in ("head_dim_qk", "head_dim_v") if k in kw}
    args.update(kw)
    pr, keep = mla.make_problem(**args)
    for k, v in dims.items():
        setattr(pr, k, v)
    rc = mla.load().mla_validate(q, kv, bt, seqlens, ctypes.c_float(scale), out, lse,
                                 ctypes.byref(pr))
    return rc, mla.last_error()


def test_valid_contiguous_and_paged():
    assert validate()[0] == mla.MLA_OK
    assert validate(bt=A, page_size=64, num_pages=10, max_pages=4)[0] == mla.MLA_OK
    lens = np.array([5, 128], np.int32)
    assert validate(seqlens_host=lens)[0] == mla.MLA_OK


@pytest.mark.parametrize("kw,code,needle", [
    (dict(q=None), mla.MLA_ERR_INVALID_ARG, "non-NULL"),
    (dict(out=None), mla.MLA_ERR_INVALID_ARG, "non-NULL"),
    (dict(batch=0), mla.MLA_ERR_INVALID_ARG, "batch"),
    (dict(s_q=0), mla.MLA_ERR_INVALID_ARG, "s_q"),
    (dict(num_heads=24), mla.MLA_ERR_UNSUPPORTED, "multiple of 16"),
    (dict(head_dim_qk=128), mla.MLA_ERR_UNSUPPORTED, "head dims"),
    (dict(head_dim_v=576), mla.MLA_ERR_UNSUPPORTED, "head dims"),
    (dict(scale=float("nan")), mla.MLA_ERR_INVALID_ARG, "finite"),
    (dict(q=A + 8), mla.MLA_ERR_INVALID_ARG, "aligned"),
    (dict(out=A + 4), mla.MLA_ERR_INVALID_ARG, "aligned"),
    (dict(kv_capacity=0), mla.MLA_ERR_INVALID_ARG, "kv_capacity"),
    (dict(bt=A), mla.MLA_ERR_INVALID_ARG, "block_table"),
    (dict(page_size=40, bt=A, num_pages=4, max_pages=4), mla.MLA_ERR_UNSUPPORTED, "page_size"),
    (dict(page_size=64, num_pages=4, max_pages=4), mla.MLA_ERR_INVALID_ARG, "block_table"),
    (dict(page_size=64, bt=A, num_pages=0, max_pages=4), mla.MLA_ERR_INVALID_ARG, "num_pages"),
    (dict(seqlens_host=np.array([0, 5], np.int32)), mla.MLA_ERR_INVALID_ARG, "seqlens[0]"),
    (dict(seqlens_host=np.array([5, 129], np.int32)), mla.MLA_ERR_INVALID_ARG, "seqlens[1]"),
    (dict(s_q=4, seqlens_host=np.array([3, 9], np.int32)), mla.MLA_ERR_INVALID_ARG, "seqlens[0]"),
    (dict(page_size=64, bt=A, num_pages=9, max_pages=2,
          seqlens_host=np.array([128, 129], np.int32)), mla.MLA_ERR_INVALID_ARG, "seqlens[1]"),
])
def test_validation_errors(kw, code, needle):
    rc, msg = validate(**kw)
    assert rc == code, msg
    assert needle in msg


# --- the split plan -------------------------------------------------------------

def range_keys(total, splits, min_chunk):
    """Keys per range for a line of `total` keys: an equal share rounded up
    to a block, at least min_chunk."""
    c = max(-(-total // splits), min_chunk)
    return max(16, -(-c // 16) * 16)


def expected_line(padded, splits, min_chunk):
    """(line keys, keys per range, gap): the plain line of padded lengths,
    or, when it starts a sequence with keys inside a range, the line with
    MLA_PLAN_SEQ_GAP keys after every sequence with keys."""
    total = sum(padded)
    chunk = range_keys(total, splits, min_chunk)
    starts = np.concatenate([[0], np.cumsum(padded)[:-1]])
    if not any(p > 0 and st % chunk != 0 for p, st in zip(padded, starts)):
        return total, chunk, 0
    gap = declared_constants()["MLA_PLAN_SEQ_GAP"]
    total += gap * sum(1 for p in padded if p > 0)
    return total, range_keys(total, splits, min_chunk), gap


def check_plan(lens, splits, min_chunk):
    segs, info = mla.mla_plan(lens, splits, min_chunk)
    chunk = info["chunk"]
    assert chunk % 16 == 0 and chunk >= min_chunk
    padded = [(int(L) + 15) // 16 * 16 for L in lens]
    total, want_chunk, gap = expected_line(padded, splits, min_chunk)
    assert (info["total_keys"], chunk, info["seq_gap"]) == (total, want_chunk, gap)
    assert info["active_groups"] <= splits
    # every real key covered exactly once, segments inside one sequence
    cover = [np.zeros(int(L), np.int32) for L in lens]
    load = {}
    slots = set()
    for s in segs:
        b, kb, ke = s["seq"], s["key_begin"], s["key_end"]
        assert 0 <= kb < max(ke, kb + 1) and ke <= lens[b]
        assert kb % 16 == 0
        cover[b][kb:ke] += 1
        load[s["group"]] = load.get(s["group"], 0) + (min(ke + 15, padded[b]) // 16 * 16 - kb)
        if s["slot"] >= 0:
            assert s["slot"] not in slots
            slots.add(s["slot"])
            assert s["slot"] // 2 == s["group"]
    for b, c in enumerate(cover):
        assert np.all(c == 1), f"sequence {b} not covered exactly once"
    # a sequence is whole (slot -1) exactly when it has one segment
    per_seq = {}
    for s in segs:
        per_seq.setdefault(s["seq"], []).append(s)
    for b, ss in per_seq.items():
        assert (len(ss) == 1) == (ss[0]["slot"] == -1)
        groups = [x["group"] for x in ss]
        assert groups == list(range(groups[0], groups[0] + len(groups)))
    assert info["split_sequences"] == sum(1 for ss in per_seq.values() if len(ss) > 1)
    # balance: no group holds more than one chunk of padded keys
    assert max(load.values()) <= chunk
    # every segment where the line puts it: sequence b starts after the
    # padded keys and gaps of the sequences before it
    line_starts = np.concatenate([[0], np.cumsum([p + (gap if p > 0 else 0) for p in padded])[:-1]])
    for s in segs:
        st = int(line_starts[s["seq"]])
        assert s["group"] * chunk <= st + s["key_begin"] < (s["group"] + 1) * chunk
    # some group holds several segments only where a sequence with keys
    # starts inside a range, and without gaps exactly there (the launcher
    # picks the kernel that sends the next segment's first block ahead by
    # this rule)
    off_boundary = any(p > 0 and st % chunk != 0 for p, st in zip(padded, line_starts))
    per_group = {}
    for s in segs:
        per_group[s["group"]] = per_group.get(s["group"], 0) + 1
    several = max(per_group.values()) > 1
    assert off_boundary if several else True
    if gap == 0:
        assert several == off_boundary
    return segs, info


@pytest.mark.parametrize("lens,splits,min_chunk", [
    ([512], 256, 256),
    ([4096] * 16, 256, 256),
    ([65536] * 16, 256, 256),
    ([16384] * 32, 256, 256),
    ([1, 2, 17, 64, 65, 1000], 7, 64),
    ([3] * 100, 256, 256),
])
def test_plan_properties(lens, splits, min_chunk):
    check_plan(lens, splits, min_chunk)


def test_plan_headline_is_even():
    segs, info = check_plan([65536] * 16, 256, 256)
    assert info["chunk"] == 4096 and info["active_groups"] == 256
    assert all(s["key_end"] - s["key_begin"] == 4096 for s in segs)


def test_plan_ragged_workload_balanced():
    import workloads as wl
    lens = wl.draw_seqlens(wl.WORKLOADS["mla_bs64_ragged1k_32k_paged64"])
    segs, info = check_plan(lens, 256, 256)
    assert info["active_groups"] == 256


def test_plan_random_fuzz():
    rng = np.random.default_rng(0)
    for _ in range(200):
        B = int(rng.integers(1, 80))
        lens = rng.integers(1, 5000, size=B)
        check_plan(lens, int(rng.integers(1, 300)), int(rng.choice([64, 128, 256, 1024])))


def test_smoke_case_passes_host_validation():
    """The smoke check's inputs satisfy the library's own argument checks
    (s_q <= L_b <= capacity, page geometry), so smoke() cannot fail on them."""
    import __graft_entry__ as entry

    inp = entry.smoke_inputs()
    B, s_q, H = inp.q.shape[:3]
    rc, msg = validate(batch=B, s_q=s_q, num_heads=H, page_size=inp.kv.shape[1], kv_capacity=0,
                       num_pages=inp.kv.shape[0], max_pages=inp.block_table.shape[1], bt=A,
                       seqlens_host=inp.seqlens)
    assert rc == mla.MLA_OK, msg
