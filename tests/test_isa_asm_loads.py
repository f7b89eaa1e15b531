"""The split kernel issues some loads from inline assembly (transposing LDS
reads, the query loads into accumulation registers).  The compiler takes an
asm statement's outputs as written when the statement ends, so every such
statement must wait for its own loads before it ends.  This test builds the
gfx950 assembly with the library's own flags and checks exactly that, for
every inline-asm block of the split kernels and of the MLA steps' kernels,
and that no kernel of either source spills to scratch or uses packed fp32
arithmetic (CPU only: hipcc cross-compiles).
"""
import re
import subprocess

import pytest

from decode_attention_mla_amd import build as libbuild

pytestmark = pytest.mark.slow

LDS_LOAD = re.compile(r"^ds_read")
VMEM_LOAD = re.compile(r"^(global_load|buffer_load|flat_load)")


def device_asm(tmp_path_factory, src, name):
    out = tmp_path_factory.mktemp("isa") / name
    flags = [f for f in libbuild.FLAGS if f not in ("-fPIC", "-shared")]
    subprocess.run([libbuild.HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(out), src],
                   check=True, capture_output=True)
    return out.read_text().split("\n")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    return device_asm(tmp_path_factory, libbuild.SRC, "mla.s")


@pytest.fixture(scope="module")
def steps_asm(tmp_path_factory):
    return device_asm(tmp_path_factory, libbuild.STEPS_SRC, "steps.s")


# Every instance of the split kernel: one row block per workgroup (also the
# one that sends the next segment's first blocks before the merge), two key
# groups, one key group; the shared-step ones also with P as one bf16
# (MLA_OPT_P_BF16).
SPLIT_KERNELS = tuple(f"_ZN3mla16mla_split_kernelILi{m}ELb{h}EEEvNS_6ParamsE"
                      for m, h in ((0, 0), (3, 0), (1, 0), (1, 1), (2, 0), (2, 1)))


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


def kernel_names(asm):
    names = []
    for line in asm:
        m = re.match(r"^(_Z\w+):", line)
        if m:
            names.append(m.group(1))
    return names


def check_clean(body, name):
    text = "\n".join(body)
    assert "scratch_" not in text, f"{name} spills to scratch"
    for op in ("v_pk_mul_f32", "v_pk_add_f32", "v_pk_fma_f32"):
        assert op not in text, f"{name} uses {op}"


@pytest.mark.parametrize("name", SPLIT_KERNELS)
def test_no_scratch_in_the_split_kernel(asm, name):
    check_clean(kernel_body(asm, name), name)


def test_every_device_function_is_clean(asm, steps_asm):
    """No scratch and no packed fp32 arithmetic anywhere in the device code
    of either source: the attention kernels (combine included) and the MLA
    steps' kernels."""
    names = 0
    for code in (asm, steps_asm):
        for name in kernel_names(code):
            check_clean(kernel_body(code, name), name)
            names += 1
    assert names >= len(SPLIT_KERNELS) + 2 + 3, "kernels missing from the assembly"
    assert any("mla_combine_kernel" in n for n in kernel_names(asm))
    assert sum("absorb" in n or "project" in n or "append" in n for n in kernel_names(steps_asm)) >= 3


def test_inline_asm_loads_wait_in_the_steps_kernels(steps_asm):
    for name in kernel_names(steps_asm):
        for ins in asm_blocks(kernel_body(steps_asm, name)):
            if any(LDS_LOAD.match(i) or VMEM_LOAD.match(i) for i in ins):
                assert ins[-1].startswith("s_waitcnt"), f"{name}: asm loads without a closing wait: {ins}"
