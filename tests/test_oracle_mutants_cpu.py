"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of oracle/csa2_oracle.c
(an off-by-one, a reversed tie, a dropped term, a wrong stride or index), builds
it into its own library, and runs tests/test_oracle_pins.py against that build
(CSA2_ORACLE_LIB); the pins must fail for every mutant.  The working tree's
oracle is never touched.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "csa2_oracle.c")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("reachability off by one in the top-K", "if (p < 0 || p >= n_valid) continue;", "if (p < 0 || p > n_valid) continue;"),
    ("ties go to the higher row", "return (x->pos < y->pos) ? -1 : (x->pos > y->pos);\n}\nstatic int by_pos",
     "return (x->pos > y->pos) ? -1 : (x->pos < y->pos);\n}\nstatic int by_pos"),
    ("selection not emitted in row order", "qsort(c, (size_t)take, sizeof(cand_t), by_pos);", ""),
    ("window rows dropped", "for (j = 0; j < win_len; ++j, ++e)", "for (j = 0; j < 0; ++j, ++e)"),
    ("sink left out of the denominator", "if (sink) l += exp(sink[hh] - mx);", ""),
    ("softmax scale ignored", "s[j] = scale * acc;", "s[j] = acc;"),
    ("ReLU dropped", "f32 = relu ? (acc > 0.0f ? acc : 0.0f) : acc;", "f32 = acc;"),
    ("index weights dropped", "float f32, wh = w ? w[h] : 1.0f;", "float f32, wh = 1.0f;"),
    ("fp8 block scale ignored", "out[i] = code * scale;", "out[i] = code;"),
    ("bf16 exponent bias", "v = ldexp(1.0 + (double)m / 128.0, e - 127);", "v = ldexp(1.0 + (double)m / 128.0, e - 126);"),
    ("e4m3 subnormal step", "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    ("V read transposed", "oh[i] += p * vmat[(size_t)j * (size_t)d + (size_t)i];",
     "oh[i] += p * vmat[(size_t)i * (size_t)e + (size_t)j];"),
    ("window replay cut ignored", "if (a < replay_start) a = replay_start;", ""),
    ("score chain summed backwards", "for (i = 0; i < d_i; ++i) {\n      acc = fmaf", "for (i = d_i - 1; i >= 0; --i) {\n      acc = fmaf"),
    ("empty row's lse 0 instead of -inf", "if (lse) lse[hh] = -INFINITY;", "if (lse) lse[hh] = 0;"),
    ("every head reads head 0's query", "const double *qh = q + (size_t)hh * (size_t)d;", "const double *qh = q;"),
    ("compressor emits at the group's first token", "if (u != m - 1) {\n        emit_idx[b] = -1;",
     "if (u != 0) {\n        emit_idx[b] = -1;"),
    ("compressor entry index off by one", "emit_idx[b] = (int32_t)((p + 1) / m - 1);", "emit_idx[b] = (int32_t)((p + 1) / m);"),
    ("RMSNorm without the mean", "r = 1.0 / sqrt(ss / (double)d + eps);", "r = 1.0 / sqrt(ss + eps);"),
    ("de-rotation turns the wrong way", "p[0] = (float)(x * cs + y * sn);", "p[0] = (float)(x * cs - y * sn);"),
]


def _mutant_kills(tmp, i, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutant {i}: text not found"
    lib = os.path.join(tmp, f"liboracle_m{i}.so")
    cfile = os.path.join(tmp, f"m{i}.c")
    open(cfile, "w").write(src.replace(old, new, 1))
    subprocess.run(["gcc", "-O2", "-std=c99", "-D_DEFAULT_SOURCE", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                    "-fPIC", "-shared", "-w", "-o", lib, cfile, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, CSA2_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-x", "-q",
                        "-p", "no:cacheprovider"], env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    return r.returncode != 0


def test_every_planted_mistake_fails_a_pin(tmp_path):
    # control: the same build of the unchanged source passes the pins
    assert not _mutant_kills(str(tmp_path), "ctl", "/*", "/*"), "the unchanged oracle fails its pins"
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        futs = [ex.submit(_mutant_kills, str(tmp_path), i, old, new) for i, (_, old, new) in enumerate(MUTANTS)]
        killed = [f.result() for f in futs]
    survivors = [MUTANTS[i][0] for i, k in enumerate(killed) if not k]
    assert not survivors, f"mutants the pins miss: {survivors}"
