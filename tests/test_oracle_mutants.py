"""The oracle's pins catch plausible mistakes.

Each mutant plants one mistake (a dropped term, a wrong sign, a transposed
index, a wrong rounding rule or range) in a copy of oracle/sq_oracle.c, builds
it with the oracle's own flags into a temporary directory, and runs the pin
suites (tests/test_oracle_format.py, tests/test_oracle_step.py) against it in
a child process (SQ_ORACLE_LIB points the oracle wrapper at the mutated
build).  Every mutant must fail at least one pin; the unmodified source must
pass them all.  All of this runs on the CPU."""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sq_oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_format.py"),
        os.path.join(ROOT, "tests", "test_oracle_step.py")]

# (what the mistake is, text in sq_oracle.c, replacement)
MUTANTS = [
    ("update: gate dropped from the key correction",
     "((double)v[j] - a * u[j])", "((double)v[j] - u[j])"),
    ("update: correction added with the wrong sign",
     "a * S[(long)i * dv + j] + b * (double)k[i]", "a * S[(long)i * dv + j] - b * (double)k[i]"),
    ("update: decay applied to the correction only",
     "S[(long)i * dv + j] = a * S[(long)i * dv + j] + b", "S[(long)i * dv + j] = S[(long)i * dv + j] + b"),
    ("key reduction over the transposed state",
     "for (int i = 0; i < dk; i++) acc += (double)k[i] * S[(long)i * dv + j];\n        u[j] = acc;\n    }\n    double a = alpha",
     "for (int i = 0; i < dk; i++) acc += (double)k[i] * S[(long)(i % dv) * dv + (j % dk)];\n        u[j] = acc;\n    }\n    double a = alpha"),
    ("readout with the key instead of the query",
     "            for (int i = 0; i < dk; i++) acc += (double)q[i] * S[(long)i * dv + j];\n            o[j] = (float)acc;\n        }\n    }\n    int bad = orc_encode_tile(bits, dk, dv, S, r, c, tile);\n    free(u);\n    free(S);\n    return bad;\n}\n\n/* Readout without update",
     "            for (int i = 0; i < dk; i++) acc += (double)k[i] * S[(long)i * dv + j];\n            o[j] = (float)acc;\n        }\n    }\n    int bad = orc_encode_tile(bits, dk, dv, S, r, c, tile);\n    free(u);\n    free(S);\n    return bad;\n}\n\n/* Readout without update"),
    ("rounding: ties away from zero instead of to even",
     "if (frac > 0.5) return fl + 1.0;", "if (frac >= 0.5) return fl + 1.0;"),
    ("range: saturation one code too wide",
     "if (r > Q) r = Q;", "if (r > Q + 1) r = Q + 1;"),
    ("step size not rounded to fp32",
     "return (double)(float)((double)r * (double)c);", "return (double)r * (double)c;"),
    ("layout: rows and columns swapped inside a block",
     "return 16 * B + 4 * (j % 4) + (i % 4);", "return 16 * B + 4 * (i % 4) + (j % 4);"),
    ("packing: fields read most significant bit first",
     "if ((tile[pos >> 3] >> (pos & 7)) & 1) v |= (uint32_t)1 << b;",
     "if ((tile[pos >> 3] >> (pos & 7)) & 1) v |= (uint32_t)1 << (w - 1 - b);"),
    ("binary16: subnormal quantum off by one binade",
     "v = ldexp((double)m, -24); /* zero or subnormal", "v = ldexp((double)m, -25); /* zero or subnormal"),
    ("code offset: excess 2^(b-1) - 1 instead of 2^(b-1)",
     "int q = (int)f - (1 << (bits - 1));", "int q = (int)f - ((1 << (bits - 1)) - 1);"),
    ("non-finite quotient mapped to +Q instead of 0",
     "if (isnan(z)) return 0;", "if (isnan(z)) return Q;"),
    ("pool: slot indirection ignored",
     "uint8_t *tile = J->pool + (long)J->slot_ids[n] * J->slab + J->off[h];",
     "uint8_t *tile = J->pool + (long)n * J->slab + J->off[h];"),
    ("per-channel gate applied to the wrong channel",
     "*= (double)alpha[i]; /* T */", "*= (double)alpha[dk - 1 - i]; /* T */"),
    ("bfloat16: one mantissa bit too many",
     "double ulp = ldexp(1.0, ex - 7);", "double ulp = ldexp(1.0, ex - 8);"),
    ("per-slot factors: the slot's own set ignored",
     "return base + ((long)slot * stride + h) * (long)d;", "return base + (long)h * (long)d;"),
    ("non-finite report: taken on the value, not on the quotient a code is decided on",
     "? (float)(x / s) : (float)x;", "? (float)x : (float)x;"),
    ("non-finite report: never raised",
     "bad |= orc_nonfinite_field(bits, x, s);", "bad |= 0 * orc_nonfinite_field(bits, x, s);"),
]


def _run_pins(lib: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, SQ_ORACLE_LIB=lib, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-p", "no:cacheprovider",
                           "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=600)


def _build(tmp_path, name: str, text: str) -> str:
    sys.path.insert(0, ROOT)
    from oracle import build as ob
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    return ob.build(src=str(src), out=str(tmp_path / f"{name}.so"))


def test_every_mutant_fails_a_pin(tmp_path):
    text = open(SRC).read()
    libs = [_build(tmp_path, "unmodified", text)]
    for n, (what, old, new) in enumerate(MUTANTS):
        assert text.count(old) == 1, f"mutation site not unique or missing: {what}"
        libs.append(_build(tmp_path, f"mutant{n}", text.replace(old, new)))
    with cf.ThreadPoolExecutor(4) as ex:
        runs = list(ex.map(_run_pins, libs))
    assert runs[0].returncode == 0, "unmodified oracle fails its pins:\n" + runs[0].stdout[-2000:]
    survivors = [what for (what, _, _), r in zip(MUTANTS, runs[1:]) if r.returncode == 0]
    assert not survivors, f"mutants no pin catches: {survivors}"
