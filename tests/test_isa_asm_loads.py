"""The split kernel issues some loads from inline assembly (transposing LDS
reads, the query loads into accumulation registers).  The compiler takes an
asm statement's outputs as written when the statement ends, so every such
statement must wait for its own loads before it ends.  This test builds the
gfx950 assembly with the library's own flags and checks exactly that, for
every inline-asm block of the split kernel (CPU only: hipcc cross-compiles).
"""
import re
import subprocess

import pytest

from decode_attention_mla_amd import build as libbuild

pytestmark = pytest.mark.slow

LDS_LOAD = re.compile(r"^ds_read")
VMEM_LOAD = re.compile(r"^(global_load|buffer_load|flat_load)")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "mla.s"
    flags = [f for f in libbuild.FLAGS if f not in ("-fPIC", "-shared")]
    subprocess.run([libbuild.HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(out),
                    libbuild.SRC], check=True, capture_output=True)
    return out.read_text().split("\n")


# Every instance of the split kernel: one row block per workgroup, two key
# groups, one key group.
SPLIT_KERNELS = tuple(f"_ZN3mla16mla_split_kernelILi{m}EEEvNS_6ParamsE" for m in range(3))


def kernel_body(asm, name):
    start = next(i for i, l in enumerate(asm) if l.startswith(name + ":"))
    end = next(i for i in range(start, len(asm)) if asm[i].strip().startswith("s_endpgm"))
    return asm[start:end + 1]


def asm_blocks(lines):
    """Instructions of each inline-asm statement, in order."""
    blocks, cur = [], None
    for line in lines:
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            cur = []
        elif t.startswith(";;#ASMEND"):
            blocks.append(cur)
            cur = None
        elif cur is not None and t and not t.startswith(";"):
            cur.append(t)
    return blocks


@pytest.mark.parametrize("name", SPLIT_KERNELS)
def test_inline_asm_loads_wait_in_their_own_statement(asm, name):
    blocks = asm_blocks(kernel_body(asm, name))
    checked = 0
    for ins in blocks:
        lds = [i for i in ins if LDS_LOAD.match(i)]
        vmem = [i for i in ins if VMEM_LOAD.match(i)]
        if not lds and not vmem:
            continue
        checked += 1
        last = ins[-1]
        assert last.startswith("s_waitcnt"), f"asm loads without a closing wait: {ins}"
        if lds:
            assert "lgkmcnt(0)" in last, f"LDS loads not waited for in their statement: {ins}"
        if vmem:
            assert "vmcnt(0)" in last, f"global loads not waited for in their statement: {ins}"
        # nothing but the loads themselves before the closing wait
        for i in ins[:-1]:
            assert LDS_LOAD.match(i) or VMEM_LOAD.match(i), f"other work between asm loads and wait: {i}"
    assert checked > 0, "no inline-asm loads found: the check is vacuous"


@pytest.mark.parametrize("name", SPLIT_KERNELS)
def test_no_scratch_in_the_split_kernel(asm, name):
    body = "\n".join(kernel_body(asm, name))
    assert "scratch_" not in body, "the split kernel spills to scratch"
    assert "v_pk_mul_f32" not in body and "v_pk_add_f32" not in body and "v_pk_fma_f32" not in body
