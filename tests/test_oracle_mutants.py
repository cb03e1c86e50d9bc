"""How strong the oracle's pins are: each mutant below is the oracle's C source
with one plausible mistake planted in it (a flipped sign, a dropped term, a
wrong index or bit position, another rounding rule). A child process builds the
mutant into a temporary directory, loads it in place of the oracle's own
library and runs the pin tests (test_oracle_pins.py) against it; at least one
pin must fail. The oracle's source and library are only read.

The mistakes target each step the oracle takes: the weight decoding of the
PQ2_0 format, the per-group activation quantisation and its plane order, the
exact group dot with its -sum(q) offset folded in, the float epilogue and its
error scale, and the binary16 weight-scale decoding."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pq2_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in the oracle's source, the mistaken text put in its place)
MUTANTS = [
    ("weight_sign", "return c - 1;", "return 1 - c;"),
    ("weight_offset", "return c - 1;", "return c - 2;"),
    ("code_order_in_byte", "(2 * (int)(k % 4))", "(2 * (int)(3 - k % 4))"),
    ("scale_divisor", "amax / 127.0f", "amax / 128.0f"),
    ("round_ties_away", "rintf(xg[i] / sc)", "roundf(xg[i] / sc)"),
    ("round_truncate", "rintf(xg[i] / sc)", "truncf(xg[i] / sc)"),
    ("reciprocal_multiply", "rintf(xg[i] / sc)", "rintf(xg[i] * (1.0f / sc))"),
    ("amax_signed", "float a = fabsf(xg[i]);", "float a = xg[i];"),
    ("t_sums_magnitudes", "sum += v;", "sum += v < 0 ? -v : v;"),
    ("plane_order_skipped", "q[m * K + g * 128 + 4 * b + s]", "q[m * K + g * 128 + 32 * s + b]"),
    ("plane_order_transposed", "qp[m * K + g * 128 + 32 * s + b]", "qp[m * K + g * 128 + 4 * b + s]"),
    ("dot_drops_last_weight", "k < (g + 1) * PQ2_ORACLE_GROUP;",
     "k < (g + 1) * PQ2_ORACLE_GROUP - 1;"),
    ("dot_wrong_row", "oracle_weight(codes, K, n, k)", "oracle_weight(codes, K, 0, k)"),
    ("act_scale_index", "(double)s[m * G + g]", "(double)s[m * G]"),
    ("weight_scale_index", "ws[n * G + g]", "ws[n * G]"),
    ("half_exponent_bias", "e - 25", "e - 24"),
    ("half_subnormal", "(double)f, -24", "(double)f, -23"),
    ("half_sign_dropped", "return sign ? -v : v;", "return v;"),
    ("epilogue_drops_first_group", "for (int64_t g = 0; g < G; ++g) {\n        double term",
     "for (int64_t g = 1; g < G; ++g) {\n        double term"),
    ("error_scale_signed", "mag += fabs(term);", "mag += term;"),
]

CHILD = (
    "import sys, oracle\n"
    "oracle.SRC, oracle.LIB, oracle._lib = sys.argv[1], sys.argv[2], None\n"
    "import pytest\n"
    "sys.exit(pytest.main(['-x', '-q', '-p', 'no:cacheprovider', sys.argv[3]]))\n"
)


def _run_pins(tmp, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"{name}: the text to mutate must occur once"
    d = os.path.join(tmp, name)
    os.makedirs(d)
    msrc = os.path.join(d, "pq2_oracle.c")
    with open(msrc, "w") as f:
        f.write(src.replace(old, new))
    r = subprocess.run([sys.executable, "-c", CHILD, msrc, os.path.join(d, "liboracle_pq2.so"), PINS],
                       cwd=ROOT, capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout[-2000:] + r.stderr[-2000:]


def test_unmutated_source_passes_the_pins(tmp_path):
    """The child set-up itself is sound: a copy of the unchanged source passes."""
    rc, out = _run_pins(str(tmp_path), "unchanged", "return c - 1;", "return c - 1;")
    assert rc == 0, out


def test_every_mutant_fails_a_pin(tmp_path):
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda m: (m[0],) + _run_pins(str(tmp_path), *m), MUTANTS))
    survivors = [name for name, rc, _ in results if rc == 0]
    # a kill is a failed pin (exit status 1) of a mutant that built and loaded
    broken = [(name, out) for name, rc, out in results
              if rc not in (0, 1) or "CalledProcessError" in out or "OSError" in out]
    assert not broken, broken
    assert not survivors, f"mutants no pin catches: {survivors}"
