"""The pins catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of oracle/nvfp4_oracle.c (a textual
change, compiled on the CPU with the oracle's own flags), then runs the pin
files that guard that part of the method against the mutated build (a
separate pytest process that loads it through NVFP4_ORACLE_LIB) and requires
that at least one pin fails.  The unchanged source, built the same way, passes
the same files.  The mistakes are the kinds a reader could make from the
pages: a field width, bias or sign bit of a scale format, a wrong E2M1 value,
a dropped term or a sign in the error that decides Four-Over-Six, the tie
rule, the stochastic-rounding threshold and index, a transposed operand, the
outer-scale formula and the straight-through gradients of scale learning."""
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
T = "tests/"

FORMATS = [T + "test_oracle_formats.py"]
QUANT = [T + "test_oracle_quantize.py", T + "test_oracle_select.py"]
FAKEQ = [T + "test_oracle_fakequant.py"]
COLUMN = [T + "test_oracle_quantize.py", T + "test_oracle_next.py", T + "test_oracle_requant.py"]

# (name, text in the oracle, planted text, pin files that must catch it)
MUTANTS = [
    ("ue5m3 exponent bias 16 instead of 15",
     "ldexp((double)(8 + m), e - 18)", "ldexp((double)(8 + m), e - 19)", FORMATS),
    ("ue5m3 with 2 mantissa bits",
     "int e = code >> 3, m = code & 7;\n  return e == 0 ? ldexp((double)m, -17) : ldexp((double)(8 + m), e - 18);",
     "int e = code >> 2, m = code & 3;\n  return e == 0 ? ldexp((double)m, -16) : ldexp((double)(4 + m), e - 17);",
     FORMATS),
    ("ue5m3 read as signed (bit 7 a sign bit)",
     "if (code == 0xFF) return NAN;",
     "if (code == 0xFF) return NAN;\n  if (code & 0x80) return -ldexp((double)(8 + (code & 7)), ((code & 0x7F) >> 3) - 18);",
     FORMATS),
    ("e2m1 grid with 5 in place of 6",
     "{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}", "{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.0}", FORMATS),
    ("scale encode ties to the odd code",
     "(d == best_d && (c & 1) == 0)", "(d == best_d && (c & 1) == 1)", FORMATS),
    ("fmix32 multiplier off by one",
     "h *= 0x85ebca6bu;", "h *= 0x85ebca6cu;", FORMATS),
    ("four-over-six keeps max->4 on a tie",
     "if (e4 < e6) {", "if (e4 <= e6) {", QUANT),
    ("block error drops a partial sum",
     "return (P[0] + P[1]) + (P[2] + P[3]);", "return (P[0] + P[1]) + P[2];", QUANT),
    ("residual with the wrong sign",
     "d[i] = fmaf(-q, S, xb[i]);", "d[i] = fmaf(q, S, xb[i]);", QUANT),
    ("outer scale from 4 instead of 6",
     "return amax / (6.0f * sg);", "return amax / (4.0f * sg);", QUANT),
    ("stochastic rounding needs a strict carry",
     "(u + F >= (1u << 22))", "(u + F > (1u << 22))", QUANT),
    ("stochastic rounding indexed by block, not element",
     "(uint64_t)(row0 + r) * (uint64_t)cols + (uint64_t)(b * 16);",
     "(uint64_t)(row0 + r) * (uint64_t)cols + (uint64_t)b;", QUANT),
    ("column-wise blocks without the transpose",
     "t[c * rows + r] = x[r * cols + c];", "t[r * cols + c] = x[r * cols + c];", COLUMN),
    ("straight-through scale gradient with the wrong sign",
     "double d = in ? q - (double)y : (y < -6.0f ? -6.0 : 6.0);",
     "double d = in ? (double)y - q : (y < -6.0f ? -6.0 : 6.0);", FAKEQ),
    ("dual pre-scale gradient with the wrong sign",
     "(-((double)s_post[blk] * acc_t)", "(((double)s_post[blk] * acc_t)", FAKEQ),
]


def _build_copy(tmp_path, old=None, new=None):
    with open(oracle_build.SRC) as f:
        src = f.read()
    if old is not None:
        assert src.count(old) == 1, f"the planted change must have one place: {old!r}"
        src = src.replace(old, new)
    path = tmp_path / "oracle_copy.c"
    path.write_text(src)
    return oracle_build.build(src=str(path), lib=str(tmp_path / "liboracle_copy.so"))


def _run_pins(lib, files):
    env = dict(os.environ, NVFP4_ORACLE_LIB=lib)
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                           "-p", "no:cacheprovider", *files],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_unchanged_copy_passes_the_pins(tmp_path):
    lib = _build_copy(tmp_path)
    files = sorted(set(FORMATS + QUANT + FAKEQ + COLUMN))
    r = _run_pins(lib, files)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


@pytest.mark.parametrize("name,old,new,files", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, files):
    lib = _build_copy(tmp_path, old, new)
    r = _run_pins(lib, files)
    # 1: a pin failed (0 would mean every pin passed; other codes are errors
    # of the run itself, not a caught mistake)
    assert r.returncode == 1, (name, r.returncode, r.stdout[-3000:] + r.stderr[-3000:])
    assert " failed" in r.stdout, (name, r.stdout[-2000:])
