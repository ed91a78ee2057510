"""Planted mistakes in the oracle (CPU only): the pins must catch each one.

Every mutant below is a copy of ``oracle/hs2_oracle.c`` with one plausible error
written in (a dropped term, a wrong sign, index or operand, an off-by-one edge, a
wrong rounding rule). It is compiled like the oracle itself into a library of its
own, and the oracle pins (``tests/test_oracle_pins.py``) are run against it in a
child process through ``HS2_ORACLE_LIB``. Each mutant must make at least one pin
fail; the unchanged copy, built the same way, must pass them all. The mistakes
live only in these temporary copies, never in the oracle's own source.
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hs2_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in the oracle, replacement): each text occurs exactly once.
MUTANTS = [
    # group score (per-head softmax probabilities summed over the group)
    ("group score without the row sum l",
     "double p = exp(zr[j] - m) / l;", "double p = exp(zr[j] - m);"),
    ("row sum with the sign of m flipped",
     "l += exp(zr[j] - m);", "l += exp(zr[j] + m);"),
    ("query heads of a group interleaved across groups",
     "const int h = g * G + hh;", "const int h = hh * D->Hkv + g;"),
    ("key rows read from group 0",
     "const size_t off = ((size_t)(base + j) * D->Hkv + g) * d;",
     "const size_t off = ((size_t)(base + j) * D->Hkv) * d;"),
    # ranking, candidates and window
    ("scores ranked ascending",
     "if (x->s > y->s) return -1;", "if (x->s < y->s) return -1;"),
    ("ties taken highest position first",
     "if (x->j < y->j) return -1; /* then lower position */\n  if (x->j > y->j) return 1;",
     "if (x->j < y->j) return 1; /* then lower position */\n  if (x->j > y->j) return -1;"),
    ("last candidate t - W left out",
     "const int64_t n_cand = t - W + 1 > 0 ? t - W + 1 : 0;",
     "const int64_t n_cand = t - W > 0 ? t - W : 0;"),
    ("forced window one token short",
     "for (int64_t j = (t - W + 1 > 0 ? t - W + 1 : 0); j <= t; j++) mark[j] = 1;",
     "for (int64_t j = (t - W + 2 > 0 ? t - W + 2 : 0); j <= t; j++) mark[j] = 1;"),
    ("decaying budget running the wrong way",
     "return D->K - (int)(((int64_t)(D->K - D->k_end) * t) / (L - 1));",
     "return D->K - (int)(((int64_t)(D->K - D->k_end) * (L - 1 - t)) / (L - 1));"),
    ("key rows taken from the start of the packed batch, not of the sequence",
     "const size_t off = ((size_t)(base + j) * D->Hkv + g) * d;",
     "const size_t off = ((size_t)j * D->Hkv + g) * d;"),
    # sparse and full attention
    ("sparse logits without the softmax scale",
     "y[a] = D->scale * dot;", "y[a] = dot;"),
    ("sparse layer weighting K rows instead of V rows",
     "kv_row(J, 1, ((size_t)(base + ir[a]) * D->Hkv + g) * d, d, rd);",
     "kv_row(J, 0, ((size_t)(base + ir[a]) * D->Hkv + g) * d, d, rd);"),
    ("sparse layer dropping the query's own position",
     "if (j < 0 || j > t) { y[a] = -INFINITY; continue; }",
     "if (j < 0 || j >= t) { y[a] = -INFINITY; continue; }"),
    ("sparse layer mapping heads to KV groups round-robin",
     "const int g = h / G;\n        const int32_t* ir",
     "const int g = h % D->Hkv;\n        const int32_t* ir"),
    ("full attention without the softmax denominator",
     "double val = acc[c] / den;", "double val = acc[c];"),
    # rounding rules
    ("bf16 ties rounded down instead of to even",
     "uint32_t m = (uint32_t)fl; /* 128..255 */\n  if (rem > 0.5 || (rem == 0.5 && (m & 1u))) m++;",
     "uint32_t m = (uint32_t)fl; /* 128..255 */\n  if (rem > 0.5) m++;"),
    ("E4M3 ties rounded up instead of to even",
     "if (rem > 0.5 || (rem == 0.5 && (n & 1u))) n++;", "if (rem >= 0.5) n++;"),
]


def _build(text, path):
    c_path = path + ".c"
    with open(c_path, "w") as f:
        f.write(text)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", c_path,
                           "-o", path, "-lm"])


def _run_pins(lib):
    env = dict(os.environ, HS2_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout + r.stderr


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


def test_every_mutant_text_occurs_once(source):
    for name, old, new in MUTANTS:
        assert source.count(old) == 1, name
        assert old != new, name


def test_pins_catch_every_planted_mistake(source, tmp_path):
    jobs = [("unchanged copy", source)] + [(n, source.replace(o, w)) for n, o, w in MUTANTS]
    libs = []
    for i, (name, text) in enumerate(jobs):
        lib = str(tmp_path / f"mutant{i}.so")
        _build(text, lib)
        libs.append(lib)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_run_pins, libs))
    rc0, out0 = results[0]
    assert rc0 == 0, "the unchanged copy must pass the pins:\n" + out0[-3000:]
    missed = []
    for (name, _), (rc, out) in zip(jobs[1:], results[1:]):
        # a pin failed (not a crash or a collection error)
        caught = rc == 1 and " failed" in out
        if not caught:
            missed.append(f"{name} (exit {rc}): {out[-400:]}")
        else:
            first = next((ln.split("::")[-1].split(" ")[0] for ln in out.splitlines()
                          if ln.startswith("FAILED")), "?")
            print(f"  {name}: caught by {first}", flush=True)
    assert not missed, "mutants the pins did not catch:\n" + "\n".join(missed)
