"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of ``oracle/bcq_oracle.c`` (on the CPU,
in a temporary directory), builds it, and runs ``tests/test_oracle.py`` against
that build in a subprocess.  The pin suite must fail for every mutant.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "bcq_oracle.c")

MUTANTS = {
    "sign_mapping_flipped": ("? +1 : -1;", "? -1 : +1;"),
    "bit_order_msb_first": ("(word >> (k % 32))", "(word >> (31 - k % 32))"),
    "offset_term_dropped": ("acc += zero[(size_t)m * G + j] * group_sum;", ""),
    "group_sum_over_all_columns": ("for (int k = j * g; k < (j + 1) * g; ++k)\n                group_sum",
                                   "for (int k = 0; k < K; ++k)\n                group_sum"),
    "alpha_plane_row_transposed": ("acc += alpha[((size_t)i * M + m) * G + j]",
                                   "acc += alpha[((size_t)m * p + i) * G + j]"),
    "alpha_group_index_dropped": ("acc += alpha[((size_t)i * M + m) * G + j]",
                                  "acc += alpha[((size_t)i * M + m) * G + 0]"),
    "last_plane_dropped": ("for (int i = 0; i < p; ++i) {\n                double plane_sum",
                           "for (int i = 0; i < p - 1; ++i) {\n                double plane_sum"),
    "subtract_becomes_add": ("plane_sum -= x[k];", "plane_sum += x[k];"),
    "zero_index_transposed": ("acc += zero[(size_t)m * G + j]", "acc += zero[(size_t)j * M + m]"),
    "dequant_offset_dropped": ("double v = zero[(size_t)m * G + j];", "double v = 0.0;"),
    "word_index_wrong_row_stride": ("((size_t)i * (size_t)M + (size_t)m) * W",
                                    "((size_t)m * (size_t)M + (size_t)i) * W"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, "mutation anchor must match exactly once"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(before, after))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-std=c99", "-shared", "-fPIC", "-o", str(so), str(mutant_c)],
                   check=True)
    env = dict(os.environ, BCQ_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "mutant %s passed every pin:\n%s" % (name, r.stdout[-2000:])
