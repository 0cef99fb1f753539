"""Planted mistakes in the oracle. Each mutant below is a copy of oracle/dq_ref.c with one
plausible slip (a dropped term, a wrong sign, a wrong or transposed index, the wrong tie rule
or constant, a skipped step of the iteration), built in a scratch directory. The oracle's pins
(the CPU test files that hold it to brute force, closed forms, library routines, the pages'
printed values and invariants) must fail on every one of them: they constrain each step of
the oracle rather than let it agree with itself. Every mutant stays within its arrays, so a
failure is a failed check, not a crash."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "dq_ref.c")
PIN_FILES = ["tests/test_oracle_codecs.py", "tests/test_oracle_solver.py", "tests/test_golden.py",
             "tests/test_oracle_act.py", "tests/test_oracle_gemm.py", "tests/test_oracle_pass_g.py",
             "tests/test_oracle_diag.py"]

# (what the slip is, text in dq_ref.c that occurs exactly once, what it becomes)
MUTANTS = [
    ("integer rounding ties away from zero",
     "if (frac > 0.5) return f + 1.0;", "if (frac >= 0.5) return f + 1.0;"),
    ("E2M1 ties to the odd index",
     "(dd == bd && (k % 2) == 0)", "(dd == bd && (k % 2) == 1)"),
    ("E2M1 grid with 5 in place of 6",
     "{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}", "{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.0}"),
    ("bf16 rounding truncates",
     "  return ldexp(rne_int(ldexp(f, 8)), e - 8);", "  return ldexp(floor(ldexp(f, 8)), e - 8);"),
    ("E4M3 with two mantissa bits",
     "    r = ldexp(rne_int(ldexp(f, 4)), e - 4);", "    r = ldexp(rne_int(ldexp(f, 3)), e - 3);"),
    ("E8M0 projection tie goes down",
     "if (v >= 1.5 * p) k += 1;", "if (v > 1.5 * p) k += 1;"),
    ("INT4 scale from absmax / 8",
     "fl32_div(m, 7.0f)", "fl32_div(m, 8.0f)"),
    ("MX shared exponent one too large",
     "e = (ex - 1) - 2;", "e = (ex - 1) - 1;"),
    ("MXINT4 clamp lets -8 through",
     "if (q < -7) q = -7;", "if (q < -8) q = -8;"),
    ("NVFP4 block scale without the 6",
     "float u = fl32_div(m, c->sixg);", "float u = fl32_div(m, c->g);"),
    ("NVFP4 tensor scale from 4 * 448",
     "float g = fl32_div(A, 2688.0f);", "float g = fl32_div(A, 1792.0f);"),
    ("row scale applied before the column scale",
     "x[k] = fl32_mul(fl32_mul(w_at(c, i, j), rb[j]), ra[i]);",
     "x[k] = fl32_mul(fl32_mul(w_at(c, i, j), ra[i]), rb[j]);"),
    ("row update drops b from R",
     "(0.5 * qA[i * n + j]) * (double)b[j];", "(0.5 * qA[i * n + j]);"),
    ("row update: D sums |R| instead of R^2",
     "        D += R * R;", "        D += fabs(R);"),
    ("no re-quantization before the column update",
     "dB[i * c.ng + j / group] * (0.5 * qB[i * n + j]);", "dA[i * c.ng + j / group] * (0.5 * qA[i * n + j]);"),
    ("column update reads the neighbouring column of W",
     "Nc[j] += (double)w_at(&c, i, j) * S;", "Nc[j] += (double)w_at(&c, i, (j + 1) % n) * S;"),
    ("inner row copy not re-synced after the row update",
     "    fill_reciprocals(a, ra, m);\n\n    /* 4: re-quantize", "\n\n    /* 4: re-quantize"),
    ("all-zero code slice gets scale 1/2",
     "a[i] = 1.0f; /* all-zero code slice: scale 1 */", "a[i] = 0.5f; /* all-zero code slice */"),
    ("mse adds the reconstruction",
     "double r = (double)w_at(c, i, j) - rec;", "double r = (double)w_at(c, i, j) + rec;"),
    ("mse drops a",
     "double rec = (double)a[i] * dv[i * ng + j / G]", "double rec = dv[i * ng + j / G]"),
    ("mse divided by rows only",
     "return tot / ((double)m * (double)n);", "return tot / (double)m;"),
    ("codes packed high nibble first",
     "(uint8_t)(nib[0] | (nib[1] << 4));", "(uint8_t)(nib[1] | (nib[0] << 4));"),
    ("E2M1 code loses its sign bit",
     "nib[h] = (uint8_t)((v2 < 0 ? 8 : 0) | idx);", "nib[h] = (uint8_t)idx;"),
    ("activations divided by b",
     "fl32_mul(w_at(&c, t, j), b ? b[j] : 1.0f)", "fl32_div(w_at(&c, t, j), b ? b[j] : 1.0f)"),
    ("product uses the first activation block scale throughout",
     "e8m0_value(act_scales[t * kb + k / 32])", "e8m0_value(act_scales[t * kb])"),
    ("product divides by a",
     "Y[t * out + i] = acc * (a ? (double)a[i] : 1.0);", "Y[t * out + i] = acc / (a ? (double)a[i] : 1.0);"),
    ("NVFP4 block scale without its 2^-9 floor",
     "if (s < ldexp(1.0, -9)) s = ldexp(1.0, -9);", "if (s < 0.0) s = 0.0;"),
    ("INT4 scale without its 2^-133 floor",
     "if (s < ldexp(1.0, -133)) s = ldexp(1.0, -133);", "if (s < 0.0) s = 0.0;"),
    ("E4M3 scale bits with the exponent bias off by one",
     "int ef = (e - 1) + 7;", "int ef = (e - 1) + 8;"),
    ("per-pass tensor scale never recomputed",
     "c->g = tensor_scale(c, ra, rb);", "c->g = c->g;"),
    ("projection margin measured to the wrong upper neighbour of a bf16 value",
     "next = p + ldexp(1.0, e - 7);", "next = p + ldexp(1.0, e - 8);"),
    ("projection margin relative to the projected value instead of v",
     "if (has_next) m = fmin(m, fabs(v - 0.5 * (p + next)) / v);",
     "if (has_next) m = fmin(m, fabs(v - 0.5 * (p + next)) / p);"),
    ("row-update change counts compare the wrong pair of passes",
     "changes[4 * t + 0] = count_diff_i8(qA, qB, m * n);",
     "changes[4 * t + 0] = count_diff_i8(qB, qB, m * n);"),
    ("column-update scale changes counted on the codes' buffer",
     "changes[4 * (t - 1) + 3] = count_diff_u16(sB, sA, m * c.ng);\n    }\n\n    /* 3",
     "changes[4 * (t - 1) + 3] = count_diff_u16(sB, sB, m * c.ng);\n    }\n\n    /* 3"),
    ("all-zero column gets scale 2",
     "if (Dc[j] == 0.0) {\n        b[j] = 1.0f;", "if (Dc[j] == 0.0) {\n        b[j] = 2.0f;"),
]


def test_every_mutation_site_is_in_the_source():
    src = open(SRC).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) == 1, name


def _survives(tmp_dir, name, old, new, gcc_flags):
    """Build the mutant and run the pins on it; True if every pin passes."""
    src = open(SRC).read()
    os.makedirs(tmp_dir, exist_ok=True)
    with open(os.path.join(tmp_dir, "dq_ref.c"), "w") as f:
        f.write(src.replace(old, new))
    shutil.copy(os.path.join(ROOT, "oracle", "dq_ref.h"), os.path.join(tmp_dir, "dq_ref.h"))
    lib = os.path.join(tmp_dir, "libdq_ref_mutant.so")
    subprocess.run(["gcc", *gcc_flags, os.path.join(tmp_dir, "dq_ref.c"), "-o", lib, "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ, DQ_REF_LIB=lib, OMP_NUM_THREADS="1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          "-m", "not gpu", *PIN_FILES],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    # exit status 1: the pins ran and one failed; 0: all passed; anything else is an error
    assert res.returncode in (0, 1), (name, res.stdout[-2000:], res.stderr[-2000:])
    return res.returncode == 0


def test_pins_catch_every_planted_mistake(tmp_path):
    import oracle
    from concurrent.futures import ThreadPoolExecutor

    workers = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = {name: ex.submit(_survives, str(tmp_path / f"m{k}"), name, old, new, oracle.GCC_FLAGS)
                for k, (name, old, new) in enumerate(MUTANTS)}
        survivors = [name for name, f in futs.items() if f.result()]
    assert not survivors, f"mutants no pin catches: {survivors}"
