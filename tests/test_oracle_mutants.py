"""The oracle's pins must reject plausible mistakes.

Each case copies ``oracle/mla_oracle.c``, plants one mistake by a textual
substitution, builds the copy with gcc into a temporary directory and runs the
pin suite (``tests/test_oracle.py``) against it in a subprocess.  The suite
must fail for every mutant.  Nothing here touches the GPU or the HIP library.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mla_oracle.c")

MUTANTS = {
    "exp_sign_flipped": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "scale_dropped": ("s[j] = sc * acc;", "s[j] = acc;"),
    "causal_off_by_one": ("hi = L - s_q + t + 1;", "hi = L - s_q + t;"),
    "page_slot_shifted": ("j % page_size) * d_qk", "(j + 1) % page_size) * d_qk"),
    "value_from_last_channels": ("o[c] += p * bf16_to_double(vr[c]);",
                                 "o[c] += p * bf16_to_double(vr[c + (d_qk - d_v)]);"),
    "lse_without_max": ("lse[r] = m + log(l);", "lse[r] = log(l);"),
    "token_index_swapped": ("const int t = (int)((r / H) % s_q);",
                            "const int t = (int)(r % s_q);"),
    "query_channel_transposed": ("acc += bf16_to_double(qr[c]) * bf16_to_double(kr[c]);",
                                 "acc += bf16_to_double(qr[(c * 7) % d_qk]) * bf16_to_double(kr[c]);"),
    "combine_weight_unnormalised": ("const double w = exp(lse_parts[(int64_t)s * rows + r] - tot);",
                                    "const double w = exp(lse_parts[(int64_t)s * rows + r] - m);"),
}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation site for {name} not unique"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(before, after))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                           "-o", str(lib), str(mutant), "-lm"])
    env = dict(os.environ, MLA_ORACLE_LIB=str(lib), OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py"), "-k", "not large_context"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins accepted mutant {name}:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout
