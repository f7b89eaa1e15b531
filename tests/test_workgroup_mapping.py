"""CPU check of the split kernel's workgroup-id mapping, compiled from the
kernel source itself.

`range_and_group` turns a workgroup id into (key range, row-block group).
The test cuts that function out of `mla_kernels.hip`, compiles it for the
host with g++ and checks, for every range count up to 700 and 1 to 4
groups:
- every id maps to one (range, group) pair, and every pair has one id;
- the groups of one range in the full blocks of eight ranges have ids 8
  apart, so ids that go round-robin over 8 XCDs put them on one XCD;
- with one group the mapping is the identity.
"""
import re
import subprocess

import pytest

from decode_attention_mla_amd import build

SRC = build.SRC  # the attention kernels' source


def cut_function(text, name):
    """The text of the function `name`, from its signature to its closing brace."""
    m = re.search(r"__device__\s+inline\s+void\s+" + name + r"\s*\(", text)
    assert m, f"{name} not found in the kernel source"
    i = text.index("{", m.end())
    depth = 0
    for j in range(i, len(text)):
        if text[j] == "{":
            depth += 1
        elif text[j] == "}":
            depth -= 1
            if depth == 0:
                return text[m.start():j + 1]
    raise AssertionError(f"unbalanced braces in {name}")


CHECKER = r"""
#include <cstdio>
#include <vector>

%s

int main() {
    for (int n_groups = 1; n_groups <= 4; ++n_groups) {
        for (int ranges = 1; ranges <= 700; ++ranges) {
            const int n = ranges * n_groups;
            std::vector<int> owner(n, -1);
            std::vector<int> first_id(ranges, -1);
            for (int id = 0; id < n; ++id) {
                int g = -1, grp = -1;
                range_and_group(id, n_groups, ranges, g, grp);
                if (g < 0 || g >= ranges || grp < 0 || grp >= n_groups) {
                    std::printf("out of range: ranges=%%d groups=%%d id=%%d -> (%%d, %%d)\n", ranges, n_groups, id, g, grp);
                    return 1;
                }
                int &o = owner[g * n_groups + grp];
                if (o != -1) {
                    std::printf("two ids: ranges=%%d groups=%%d ids %%d and %%d -> (%%d, %%d)\n", ranges, n_groups, o, id, g, grp);
                    return 1;
                }
                o = id;
                if (n_groups == 1 && g != id) {
                    std::printf("one group, not the identity: ranges=%%d id=%%d -> %%d\n", ranges, id, g);
                    return 1;
                }
                const int full8 = ranges / 8 * 8;
                if (g < full8) {
                    if (first_id[g] == -1) first_id[g] = id;
                    const int d = id - first_id[g];
                    if (d %% 8 != 0 || d >= 8 * n_groups) {
                        std::printf("groups of range %%d not 8 apart in one block: ranges=%%d groups=%%d ids %%d, %%d\n",
                                    g, ranges, n_groups, first_id[g], id);
                        return 1;
                    }
                }
            }
        }
    }
    std::printf("ok\n");
    return 0;
}
"""


def run_checker(tmp_path, fn):
    fn = fn.replace("__device__ inline", "static inline", 1)
    src = tmp_path / "mapping.cpp"
    src.write_text(CHECKER % fn)
    exe = tmp_path / "mapping"
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-o", str(exe), str(src)])
    return subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)


def test_range_and_group_is_a_bijection_with_groups_on_one_xcd(tmp_path):
    r = run_checker(tmp_path, cut_function(open(SRC).read(), "range_and_group"))
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


# Plausible slips in the mapping, each of which the checker must catch.
MUTANTS = [
    ("grp = w / 8;", "grp = w % n_groups;"),              # groups adjacent, not 8 apart
    ("g = full8 + t % rem;", "g = full8 + t / n_groups;"),  # tail ranges mis-split
    ("w % 8;", "w / n_groups;"),                          # range index from the wrong digit
    ("id < full8 * n_groups", "id < full8"),              # tail taken too early
]


@pytest.mark.parametrize("old,new", MUTANTS)
def test_checker_catches_a_slip(tmp_path, old, new):
    fn = cut_function(open(SRC).read(), "range_and_group")
    assert old in fn, f"mutant anchor {old!r} not in the function"
    r = run_checker(tmp_path, fn.replace(old, new, 1))
    assert r.returncode != 0, f"mutant {old!r} -> {new!r} passed the checker"
