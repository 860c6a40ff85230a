"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies oracle/kvp_oracle.c, applies one plausible mistake (a dropped term, a
wrong index, a wrong sign, a transposed operand), builds it into a temporary library and
runs the pin suites against it in a subprocess.  The suites must fail for every mutant.
The real oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvp_oracle.c")

# (name, original text, replacement, occurrence index or None for all)
MUTANTS = [
    ("mask_off_by_one", "for (int j = i + 1; j < n; ++j)", "for (int j = i + 2; j < n; ++j)", None),
    ("mask_hides_self", "for (int j = i + 1; j < n; ++j)", "for (int j = i; j < n; ++j)", None),
    ("gqa_modulo_map", "return h / (Hq / Hkv);", "return h % Hkv;", None),
    ("scale_dropped_row", "s[j] = scale * acc;\n        if (s[j] > m)\n            m = s[j];\n    }\n    double Z",
     "s[j] = acc;\n        if (s[j] > m)\n            m = s[j];\n    }\n    double Z", None),
    ("no_normalisation", "s[j] = s[j] / Z;", "s[j] = s[j];", None),
    ("merge_no_rescale_numerator", "acc += o[(long)i * d + c] * exp(m[i] - M);",
     "acc += o[(long)i * d + c];", None),
    ("merge_wrong_sign", "L += l[i] * exp(m[i] - M);", "L += l[i] * exp(M - m[i]);", None),
    ("partial_sum_count", "l += s[j];", "l += 1.0;", None),
    ("varlen_drops_self", "int nk = causal ? i + 1 : n;", "int nk = causal ? (i > 0 ? i : 1) : n;", None),
    ("varlen_ignores_segment_start", "k + ((long)a * Hkv + g) * d", "k + ((long)g) * d", None),
    ("decode_swaps_k_v", "K + base, d, V + base, d,", "V + base, d, K + base, d,", None),
    ("full_value_head_zero", "acc += row[j] * v[((long)j * Hkv + g) * d + c];",
     "acc += row[j] * v[((long)j * Hkv + 0) * d + c];", None),
    ("kv_bytes_missing_two", "return 2LL * L * Hkv * d * elem_bytes;", "return 1LL * L * Hkv * d * elem_bytes;", None),
    ("decode_ctx_minus_one", "orc_attention_row(d, ctx[b],", "orc_attention_row(d, ctx[b] > 1 ? ctx[b] - 1 : 1,", None),
    ("chunk_mask_from_cache_start", "orc_attention_row(d, first + i + 1,", "orc_attention_row(d, i + 1,", None),
    ("chunk_drops_own_position", "orc_attention_row(d, first + i + 1,", "orc_attention_row(d, first + i > 0 ? first + i : 1,", None),
    ("chunk_rows_of_first_request", "long row = (long)cu[b] + i;", "long row = (long)i;", None),
    ("score_transposed_index", "acc += q[c] * K[(long)j * kstride + c];\n        s[j] = scale * acc;\n        if (s[j] > m)\n            m = s[j];\n    }\n    double Z",
     "acc += q[c] * K[(long)c * kstride + (j % d)];\n        s[j] = scale * acc;\n        if (s[j] > m)\n            m = s[j];\n    }\n    double Z", None),
]

SUITES = ["tests/test_oracle_pins.py", "tests/test_oracle_brute.py", "tests/test_oracle_chunk.py"]


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new, occ):
    src = open(SRC).read()
    assert old in src, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new)
    assert mutated != src
    csrc = tmp_path / "mutant.c"
    csrc.write_text(mutated)
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-o",
                    str(lib), str(csrc), "-lm"], check=True)
    env = dict(os.environ, KVP_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + SUITES,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
