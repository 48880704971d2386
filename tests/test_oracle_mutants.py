"""The oracle's pins catch plausible mistakes in the oracle.

Each case below plants one mistake in a copy of ``oracle/lora_oracle.c`` (a
dropped term, a wrong scale, a transposed operand, a wrong rounding rule, ...),
builds the copy with the oracle's own flags, and runs the pin suite
``tests/test_oracle_pins.py`` against it in a child process.  The suite must
fail on every mutant, and fail as a test failure (pytest exit status 1), not a
crash.  The real oracle is never modified; the mutants live in a temporary
directory.  CPU only.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in lora_oracle.c, replacement, occurrence to replace: 1 = first)
MUTANTS = [
    ("rslora scale uses r", "return lora_alpha / sqrt((double)r);",
     "return lora_alpha / (double)r;", 1),
    ("plain scale uses sqrt(r)", "return lora_alpha / (double)r;",
     "return lora_alpha / sqrt((double)r);", 1),
    ("scale dropped", "store_elem(y, dtype, o, yv + s * acc);",
     "store_elem(y, dtype, o, yv + acc);", 1),
    ("base output dropped", "store_elem(y, dtype, o, yv + s * acc);",
     "store_elem(y, dtype, o, s * acc);", 1),
    ("A read transposed", "load_elem(At[k], dtype, (int64_t)j * d_in + i)",
     "load_elem(At[k], dtype, (int64_t)i * r + j)", 1),
    ("B read transposed", "acc = acc + h[j] * load_elem(B[k], dtype, (int64_t)j * d_out + n);",
     "acc = acc + h[j] * load_elem(B[k], dtype, (int64_t)n * r + j);", 1),
    ("last rank dropped", "for (int32_t j = 0; j < r; ++j)\n                acc = acc + h[j]",
     "for (int32_t j = 0; j + 1 < r; ++j)\n                acc = acc + h[j]", 1),
    ("last input feature dropped",
     "for (int32_t i = 0; i < d_in; ++i)\n                acc = acc + load_elem(x, dtype, (int64_t)t * d_in + i) *\n"
     "                                load_elem(At[k]",
     "for (int32_t i = 0; i + 1 < d_in; ++i)\n                acc = acc + load_elem(x, dtype, (int64_t)t * d_in + i) *\n"
     "                                load_elem(At[k]", 1),
    ("bf16 rounded twice (through fp32)", "((uint16_t *)base)[i] = double_to_bf16_rne(v);",
     "((uint16_t *)base)[i] = double_to_bf16_rne((double)(float)v);", 1),
    ("bf16 ties away from zero", "double r = nearbyint(v / q) * q;",
     "double r = round(v / q) * q;", 1),
    ("bf16 truncated", "double r = nearbyint(v / q) * q;",
     "double r = trunc(v / q) * q;", 1),
    ("negative slot applied as slot 0", "if (k < 0 || k >= n_slots || rank[k] <= 0)\n            continue;",
     "if (k < 0)\n            k = 0;\n        if (k >= n_slots || rank[k] <= 0)\n            continue;", 1),
    ("DoRA factor applied after the bias",
     "            if (dora && dora[k])\n                v = dora[k][n] * v;\n"
     "            if (bias && bias[k])\n                v = v + load_elem(bias[k], dtype, n);\n",
     "            if (bias && bias[k])\n                v = v + load_elem(bias[k], dtype, n);\n"
     "            if (dora && dora[k])\n                v = dora[k][n] * v;\n", 1),
    ("saved module read transposed", "load_elem(W[k], dtype, (int64_t)n * d_in + i)",
     "load_elem(W[k], dtype, (int64_t)i * d_out + n)", 1),
    ("saved module bias dropped", "                acc = acc + load_elem(bias[k], dtype, n);\n"
     "            store_elem(y, dtype, (int64_t)t * d_out + n, acc);",
     "                acc = acc + 0.0;\n"
     "            store_elem(y, dtype, (int64_t)t * d_out + n, acc);", 1),
    ("saved module added to the base output",
     "            store_elem(y, dtype, (int64_t)t * d_out + n, acc);",
     "            store_elem(y, dtype, (int64_t)t * d_out + n,\n"
     "                       acc + load_elem(y, dtype, (int64_t)t * d_out + n));", 1),
    ("adapter size counts d_in only", "total += ((int64_t)d_in[m] + d_out[m]) * r * bytes_per_param;",
     "total += (int64_t)d_in[m] * r * bytes_per_param;", 1),
]


def _mutate(src: str, old: str, new: str, nth: int) -> str:
    assert src.count(old) >= nth, f"mutation site not found: {old[:60]!r}"
    pos = -1
    for _ in range(nth):
        pos = src.index(old, pos + 1)
    return src[:pos] + new + src[pos + len(old):]


def _run_pins_against(lib: str) -> subprocess.CompletedProcess:
    # The child imports the oracle package, points it at the mutant library,
    # then runs the pin suite in the same interpreter.
    code = ("import sys; sys.path.insert(0, %r); import oracle; "
            "oracle._LIB_PATH = %r; oracle._lib = None; import pytest; "
            "sys.exit(pytest.main([%r, '-x', '-q', '-p', 'no:cacheprovider']))") % (ROOT, lib, PINS)
    env = dict(os.environ, OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=600, cwd=ROOT, env=env)


def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = open(os.path.join(ROOT, "oracle", "lora_oracle.c")).read()
    libs = []
    for i, (name, old, new, nth) in enumerate(MUTANTS):
        c = tmp_path / f"mutant_{i}.c"
        c.write_text(_mutate(src, old, new, nth))
        so = str(tmp_path / f"mutant_{i}.so")
        subprocess.run(["gcc", *oracle.CFLAGS, "-o", so, str(c), "-lm"], check=True)
        libs.append((name, so))
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda nl: (nl[0], _run_pins_against(nl[1])), libs))
    survivors = [name for name, r in results if r.returncode == 0]
    crashed = [(name, r.returncode) for name, r in results if r.returncode not in (0, 1)]
    assert not survivors, f"mutants no pin catches: {survivors}"
    assert not crashed, f"mutants that crashed the pin run instead of failing a pin: {crashed}"


def test_unmutated_copy_passes_the_pins(tmp_path):
    """The harness itself: a copy of the oracle built the same way passes."""
    c = tmp_path / "same.c"
    c.write_text(open(os.path.join(ROOT, "oracle", "lora_oracle.c")).read())
    so = str(tmp_path / "same.so")
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", so, str(c), "-lm"], check=True)
    r = _run_pins_against(so)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
