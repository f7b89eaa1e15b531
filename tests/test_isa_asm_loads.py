"""The split kernel issues some LDS reads from inline assembly and waits for
them in a later statement.  The compiler treats an asm output as written
when the statement ends, so the kernel is only correct if no instruction
reads, writes or copies those registers before the wait.  This test builds
the gfx950 assembly with the library's own flags and checks exactly that
(CPU only: hipcc cross-compiles)."""
import os
import re
import subprocess

import pytest

from decode_attention_mla_amd import build as libbuild

pytestmark = pytest.mark.slow


def vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "mla.s"
    flags = [f for f in libbuild.FLAGS if f not in ("-fPIC", "-shared")]
    subprocess.run([libbuild.HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(out),
                    libbuild.SRC], check=True, capture_output=True)
    return out.read_text().split("\n")


def test_in_flight_transposed_reads_are_never_touched(asm):
    issued = 0
    pending = set()
    for line in asm:
        t = line.strip()
        if t.startswith(".LBB") or t.startswith("s_endpgm") or t.startswith("s_branch") \
                or t.startswith("s_cbranch"):
            assert not pending, f"transposed read still in flight at block boundary: {t}"
        if t.startswith("ds_read_b64_tr_b16"):
            pending |= vregs(t.split()[1].rstrip(","))
            issued += 1
            continue
        if t.startswith("s_waitcnt") and "lgkmcnt(0)" in t:
            pending = set()
            continue
        if not t or t.startswith(";") or t.startswith("."):
            continue
        ops = re.findall(r"v\[\d+:\d+\]|v\d+\b", t)
        touched = set().union(*[vregs(o) for o in ops]) if ops else set()
        assert not (touched & pending), f"in-flight register touched: {t}"
    assert issued > 0, "no transposed reads found: the check is vacuous"


def test_no_scratch_in_the_split_kernel(asm):
    text = "\n".join(asm)
    body = text[text.index("_ZN3mla16mla_split_kernelENS_6ParamsE:"):]
    body = body[: body.index("s_endpgm")]
    assert "scratch_" not in body, "the split kernel spills to scratch"
    assert "v_pk_mul_f32" not in body and "v_pk_add_f32" not in body and "v_pk_fma_f32" not in body
