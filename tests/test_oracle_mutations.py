"""CPU: the oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (a dropped
weight, an off-by-one divisor, a wrong sign or index, a lost base, a wrong
rounding tie, an unfused product, clients taken out of order, ...), builds
the copy, and runs the pin suite against it in a separate process: the pins
must fail.  The copy lives in a temporary directory; the oracle itself is
never modified."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, exact text in oracle/fedavg_oracle.c, replacement); the text must
# occur exactly once
MUTATIONS = [
    # fp64 definition (orc_weighted_average, resolve)
    ("o1 weight dropped", "            s += (double)n[k] * v;\n            m += (double)n[k] * fabs(v);\n"
                          "            W += (uint64_t)n[k];\n            c += 1;\n        }\n        int rc",
     "            s += v;\n            m += (double)n[k] * fabs(v);\n"
     "            W += (uint64_t)n[k];\n            c += 1;\n        }\n        int rc"),
    ("o1 divisor W + 1", "    const double D = (mode == ORC_DELTAS_ZERO_FILL) ? (double)S : (double)W;",
     "    const double D = (mode == ORC_DELTAS_ZERO_FILL) ? (double)S : (double)(W + 1);"),
    ("o1 base subtracted", "    double r = (mode == ORC_WEIGHTS) ? mean : b + mean;",
     "    double r = (mode == ORC_WEIGHTS) ? mean : b - mean;"),
    ("o1 sent mask of client 0", "            if (sent && !sent[k][i])\n                continue;",
     "            if (sent && !sent[0][i])\n                continue;"),
    ("o1 zero weight not skipped", "            if (n[k] == 0)\n                continue;\n            if (sent",
     "            if (n[k] < 0)\n                continue;\n            if (sent"),
    ("o1 unsent loses base", "        *ref32 = (float)b;", "        *ref32 = (float)0.0;"),
    ("o1 client counted twice", "            W += (uint64_t)n[k];\n            c += 1;\n        }\n        int rc",
     "            W += (uint64_t)n[k];\n            c += 2;\n        }\n        int rc"),
    ("bf16 rounds half up", "    if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))", "    if (lo >= 0x8000u)"),
    ("sparse value of the previous entry",
     "                double v = (double)val[k][j];\n                s[i] += (double)n[k] * v;",
     "                double v = (double)val[k][j > 0 ? j - 1 : 0];\n                s[i] += (double)n[k] * v;"),
    ("sparse weight of client 0", "                s[i] += (double)n[k] * v;", "                s[i] += (double)n[0] * v;"),
    # fixed-point value sum (orc_sum)
    ("sum exponent offset", "        int p = e ? (int)e - 1 : 0;", "        int p = e ? (int)e : 0;"),
    ("sum ties not to even", "    if (round && (sticky || (mant & 1u))) {", "    if (round) {"),
    ("sum upper digit sign lost", "        d[p / 32 + 1] += neg ? -hi : hi;", "        d[p / 32 + 1] += hi;"),
    ("sum subnormal implicit bit", "        uint64_t m = e ? (f | 0x800000u) : f;", "        uint64_t m = f | 0x800000u;"),
    # fp32 mirror (orc_mirror_f32)
    ("mirror unfused product", "            acc = fmaf((float)n[k], (float)value_at(x[k], x_dtype, i), acc);",
     "            acc = (float)n[k] * (float)value_at(x[k], x_dtype, i) + acc;"),
    ("mirror divides by W in zero fill", "            const float D = (float)(mode == ORC_DELTAS_ZERO_FILL ? S : W);",
     "            const float D = (float)W;"),
    ("mirror base subtracted", "            r = (mode == ORC_WEIGHTS) ? q : (float)value_at(base, base_dtype, i) + q;",
     "            r = (mode == ORC_WEIGHTS) ? q : (float)value_at(base, base_dtype, i) - q;"),
    ("mirror clients reversed", "        for (int k = 0; k < K; ++k) {\n            if (n[k] == 0 || (sent && !sent[k][i]))",
     "        for (int k = K - 1; k >= 0; --k) {\n            if (n[k] == 0 || (sent && !sent[k][i]))"),
    # fp32 mirror of sparse lists (orc_sparse_mirror_f32)
    ("sparse mirror unfused product", "                acc[i] = fmaf((float)n[k], val[k][j], acc[i]);",
     "                acc[i] = (float)n[k] * val[k][j] + acc[i];"),
    ("sparse mirror divides by W in zero fill",
     "            const float D = (float)(mode == ORC_DELTAS_ZERO_FILL ? S : W[i]);",
     "            const float D = (float)W[i];"),
    ("sparse mirror unsent loses base", "            r = base[i];", "            r = 0.0f;"),
    ("sparse mirror client counted twice", "                c[i] += 1;\n            }\n        }\n    }\n#pragma omp parallel for schedule(static)\n    for (int64_t i = 0; i < len; ++i) {",
     "                c[i] += 2;\n            }\n        }\n    }\n#pragma omp parallel for schedule(static)\n    for (int64_t i = 0; i < len; ++i) {"),
    # checksum, top-k
    ("checksum ignores the index", "        h += fmix64((i * 0x9E3779B97F4A7C15ULL) ^ bits);", "        h += fmix64(bits);"),
    ("top-k ties to the higher index", "    return (x->index > y->index) - (x->index < y->index);",
     "    return (x->index < y->index) - (x->index > y->index);"),
]


def test_every_mutation_is_specific():
    with open(os.path.join(ROOT, "oracle", "fedavg_oracle.c")) as f:
        src = f.read()
    for name, old, new in MUTATIONS:
        assert src.count(old) == 1, name
        assert old != new, name


def _copy_tree(dst):
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("*.so", "*.so.tmp", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "synth"), os.path.join(dst, "synth"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(dst, "tests"))
    for name in ("test_oracle_pins.py", "parity.py", "conftest.py"):
        shutil.copy(os.path.join(ROOT, "tests", name), os.path.join(dst, "tests", name))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_the_mistake(name, old, new, tmp_path):
    dst = str(tmp_path)
    _copy_tree(dst)
    path = os.path.join(dst, "oracle", "fedavg_oracle.c")
    with open(path) as f:
        src = f.read()
    assert src.count(old) == 1
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    env = dict(os.environ, PYTHONPATH=dst, OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join("tests", "test_oracle_pins.py")],
                         cwd=dst, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 1, f"{name}: the pins did not fail (rc {res.returncode})\n{res.stdout[-2000:]}"
    assert "failed" in res.stdout, res.stdout[-2000:]
