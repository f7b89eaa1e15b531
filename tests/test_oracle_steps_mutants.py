"""The pins of ``oracle/steps.py`` must reject plausible mistakes.

Each case swaps one function of the oracle for a copy with one planted
mistake (a wrong head, a dropped channel, a shifted key, another rounding)
and runs every pin of ``tests/test_oracle_steps.py`` against it: at least
one must fail.  CPU only.
"""
import inspect

import numpy as np
import pytest

import test_oracle_steps as pins
from oracle import steps

ORIG = {name: getattr(steps, name)
        for name in ("absorb_q", "project_out", "project_out_abs", "append_kv", "f64_to_bf16_bits")}


def absorb_wrong_head(q_nope, q_rope, w_uk):
    q_lat, q_bits = ORIG["absorb_q"](q_nope, q_rope, np.roll(w_uk, 1, axis=0))
    return q_lat, q_bits


def absorb_rope_dropped(q_nope, q_rope, w_uk):
    q_lat, q_bits = ORIG["absorb_q"](q_nope, q_rope, w_uk)
    q_bits = q_bits.copy()
    q_bits[..., 512:] = 0
    return q_lat, q_bits


def absorb_last_channel_dropped(q_nope, q_rope, w_uk):
    w = np.array(w_uk, copy=True)
    w[..., -1] = 0
    return ORIG["absorb_q"](q_nope, q_rope, w)


def project_wrong_head(o, w_uv):
    return ORIG["project_out"](o, np.roll(w_uv, 1, axis=0))


def project_channel_dropped(o, w_uv):
    o2 = np.array(o, copy=True)
    o2[..., 511] = 0
    return ORIG["project_out"](o2, w_uv)


def project_in_fp32(o, w_uv):
    return ORIG["project_out"](o, w_uv).astype(np.float32).astype(np.float64)


def project_abs_signed_weights(o, w_uv):
    # the absolute value taken of o only
    return np.einsum("rhc,hec->rhe", np.abs(np.asarray(o, dtype=np.float64)), steps.bf16_bits_to_f64(w_uv))


def project_abs_of_sum(o, w_uv):
    # |sum o w| instead of sum |o w|
    return np.abs(ORIG["project_out"](o, w_uv))


def project_abs_wrong_head(o, w_uv):
    return ORIG["project_out_abs"](o, np.roll(w_uv, 1, axis=0))


def append_shifted(kv, block_table, seqlens, new_rows):
    return ORIG["append_kv"](kv, block_table, np.asarray(seqlens) - 1, new_rows)


def append_tokens_reversed(kv, block_table, seqlens, new_rows):
    return ORIG["append_kv"](kv, block_table, seqlens, np.asarray(new_rows)[:, ::-1])


def round_truncating(x):
    x = np.asarray(x, dtype=np.float64)
    return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def round_half_away(x):
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    out = np.trunc(m * 256.0 + np.copysign(0.5, m)) * np.exp2(e - 8.0)
    with np.errstate(over="ignore"):
        return (out.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


MUTANTS = {
    "absorb_wrong_head": ("absorb_q", absorb_wrong_head),
    "absorb_rope_dropped": ("absorb_q", absorb_rope_dropped),
    "absorb_last_channel_dropped": ("absorb_q", absorb_last_channel_dropped),
    "project_wrong_head": ("project_out", project_wrong_head),
    "project_channel_dropped": ("project_out", project_channel_dropped),
    "project_in_fp32": ("project_out", project_in_fp32),
    "project_abs_signed_weights": ("project_out_abs", project_abs_signed_weights),
    "project_abs_of_sum": ("project_out_abs", project_abs_of_sum),
    "project_abs_wrong_head": ("project_out_abs", project_abs_wrong_head),
    "append_shifted": ("append_kv", append_shifted),
    "append_tokens_reversed": ("append_kv", append_tokens_reversed),
    "round_truncating": ("f64_to_bf16_bits", round_truncating),
    "round_half_away": ("f64_to_bf16_bits", round_half_away),
}

PINS = [f for name, f in inspect.getmembers(pins, inspect.isfunction) if name.startswith("test_")]


def test_pins_pass_on_the_oracle():
    for pin in PINS:
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, monkeypatch):
    target, fn = MUTANTS[name]
    monkeypatch.setattr(steps, target, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except Exception:  # an assertion, or a mistake that breaks a shape or an index
            failed.append(pin.__name__)
    assert failed, f"no pin rejects {name}"
