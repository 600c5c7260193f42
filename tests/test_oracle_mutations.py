"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of the oracle's C source (a flipped
comparison, a different summation order, a dropped term or token, a wrong
tie rule, ...), builds it with gcc in a temporary directory and runs the pin
suite and the hand-derived golden cases against that library in a child
process: at least one of them must fail.
The oracle itself is never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "tsv_oracle.c")

# (name, text in the oracle, replacement): each a mistake an implementation
# of the method could plausibly make
MUTATIONS = [
    ("term takes the min of the two products",
     "t[d] = a > c ? a : c;", "t[d] = a < c ? a : c;"),
    ("channel terms summed left to right",
     "float sg = tree_sum(t, D);",
     "float sg = 0.0f; for (int d = 0; d < D; ++d) sg += t[d];"),
    ("first query head of the group only",
     "else if (gi == 0 || sg > best)", "else if (gi == 0)"),
    ("group sum taken as the max",
     "best = gi == 0 ? sg : best + sg;", "best = gi == 0 || sg > best ? sg : best;"),
    ("group heads visited in decreasing order",
     "const int g = gi;", "const int g = G - 1 - gi;"),
    ("score uses the box max for every channel",
     "float a = qv[d] * mn;", "float a = qv[d] * mx;"),
    ("ties go to the higher page",
     "return (a->page > b->page) - (a->page < b->page);",
     "return (a->page < b->page) - (a->page > b->page);"),
    ("sink pages not forced",
     "for (int64_t p = 0; p < f; ++p) chosen[p] = 1; /* forced sink pages */",
     "f = 0;"),
    ("one page short of the budget",
     "for (int64_t i = 0; i < keff - f - r; ++i) chosen[cand[i].page] = 1;",
     "for (int64_t i = 0; i + 1 < keff - f - r; ++i) chosen[cand[i].page] = 1;"),
    ("recent window shifted one page back",
     "for (int64_t p = n - r; p < n; ++p) chosen[p] = 1;",
     "for (int64_t p = n - r - 1; p < n - 1; ++p) if (p >= 0) chosen[p] = 1;"),
    ("recent pages not forced",
     "for (int64_t p = n - r; p < n; ++p) chosen[p] = 1; /* forced recent pages */", ""),
    ("box ignores the last valid token",
     "for (int64_t t = 1; t < v; ++t) {", "for (int64_t t = 1; t < v - 1; ++t) {"),
    ("append never opens a new box",
     "if (slot == 0) { /* first token of a fresh page: the box is the point */",
     "if (0) { /* first token of a fresh page: the box is the point */"),
    ("attention logit without the scale",
     "z[i] = (double)scale * dot;", "z[i] = dot;"),
    ("attention drops the last token of a page",
     "for (int64_t t = 0; t < v; ++t) tok[nt++]", "for (int64_t t = 0; t + 1 < v; ++t) tok[nt++]"),
    ("values read from the key pool",
     "acc[d] += w * (double)kv_get(v_pool,", "acc[d] += w * (double)kv_get(k_pool,"),
    ("fp8 exponent bias 8 (the FNUZ variant)",
     "v = ldexp((double)(8 + m), e - 10);", "v = ldexp((double)(8 + m), e - 11);"),
    ("fp8 subnormals scaled like normals",
     "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    ("E5M2 exponent bias 16 (the FNUZ variant)",
     "v = ldexp((double)(4 + m), e - 17);", "v = ldexp((double)(4 + m), e - 18);"),
    ("E5M2 decoded with the E4M3 table",
     "return dtype == TSVO_FP8 ? fp8_table[b] : e5m2_table[b];", "return fp8_table[b];"),
    ("selection output in score order",
     "for (int64_t p = 0; p < n; ++p)\n        if (chosen[p]) out[c++] = (int32_t)p;",
     "for (int64_t i = 0; i < keff - f; ++i) out[c++] = cand[i].page;\n"
     "      for (int64_t p = 0; p < f; ++p) out[c++] = (int32_t)p;"),
]


def _pins_against(source_text, tmp_path):
    """Build `source_text` as the oracle library and run the pins and the
    golden cases (CPU) against it."""
    mutated = tmp_path / "tsv_oracle_mut.c"
    mutated.write_text(source_text)
    lib = tmp_path / "libtsv_oracle_mut.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-I", os.path.join(ROOT, "oracle"), "-o", str(lib), str(mutated),
                    "-lm"], check=True)
    env = dict(os.environ, TSV_ORACLE_LIB=str(lib))
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           "-m", "not gpu",
                           os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                           os.path.join(ROOT, "tests", "test_golden.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


def test_unmutated_copy_passes(tmp_path):
    """Control: the same build of the unchanged source passes every pin."""
    r = _pins_against(open(SRC).read(), tmp_path)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    r = _pins_against(src.replace(old, new), tmp_path)
    assert r.returncode == 1, f"no pin failed for: {name}\n{r.stdout[-2000:]}"
