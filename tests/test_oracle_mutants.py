"""The oracle's pins have teeth. Each plausible mistake below is planted in a copy of the
oracle's C source: a flipped sign, a dropped term, a wrong index or bound, a swapped operand, or
a wrong rounding or tie rule. The copy is built with the oracle's own flags, and the pin tests
it concerns run against it in a subprocess (NQ_ORACLE_LIB points the wrapper at the mutant).
Every mutant must make them fail. The unmodified source, built the same way, must pass them.
Nothing here touches a GPU or the GPU library's arithmetic.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from oracle import build as oracle_build  # noqa: E402

NUM = "tests/test_oracle_numeric.py"
E8 = "tests/test_oracle_e8.py"
PATH = "tests/test_oracle_path.py"

# (what the mistake is, exact text in nq_oracle.c, replacement, pin files that must catch it)
MUTANTS = [
    ("fp16 rounding: ties away from zero",
     "double m = nearbyint(ldexp(a, 10 - E));", "double m = round(ldexp(a, 10 - E));", [NUM]),
    ("rotary table: frequencies base^(-i/128)",
     "pow(base, -(double)i / 64.0)", "pow(base, -(double)i / 128.0)", [NUM]),
    ("RoPE removal: + instead of - in the upper half",
     "x[i + 64] = bc - as;", "x[i + 64] = bc + as;", [NUM]),
    ("RoPE removal: a in place of b in the sine product",
     "float ac = a * C[i], bs = b * S[i];", "float ac = a * C[i], bs = a * S[i];", [NUM]),
    ("Hadamard: the normalisation dropped",
     "for (int i = 0; i < HD; i++) x[i] = x[i] * INV_SQRT128_F32;", "", [NUM]),
    ("Hadamard: the difference taken the other way",
     "float a = x[j], b = x[j + h];\n                x[j] = a + b;\n                x[j + h] = a - b;",
     "float a = x[j], b = x[j + h];\n                x[j] = a + b;\n                x[j + h] = b - a;",
     [NUM]),
    ("scores: the window sum one row short",
     "int32_t w0 = T - W < 0 ? 0 : T - W;", "int32_t w0 = T - W + 1 < 0 ? 0 : T - W + 1;", [NUM]),
    ("scores: only the last head summed",
     "        double acc = 0.0;\n        for (int32_t h = 0; h < H; h++)",
     "        double acc = 0.0;\n        for (int32_t h = H - 1; h < H; h++)", [NUM]),
    ("selection: equal scores keep the higher position",
     "return (a->t > b->t) - (a->t < b->t);", "return (a->t < b->t) - (a->t > b->t);", [PATH]),
    ("keep count: the evicted count rounded up",
     "int64_t n_evict = (int64_t)evict_permille * T / 1000;",
     "int64_t n_evict = ((int64_t)evict_permille * T + 999) / 1000;", [PATH]),
    ("E8: the odd-parity fix moves away from u",
     "if (v[j] > f[j]) f[j] += 1.0;\n        else if (v[j] < f[j]) f[j] -= 1.0;",
     "if (v[j] > f[j]) f[j] -= 1.0;\n        else if (v[j] < f[j]) f[j] += 1.0;", [E8]),
    ("E8: the fix re-rounds the coordinate of smallest error",
     "if (e > best) { best = e; j = i; }", "if (best < 0.0 || e < best) { best = e; j = i; }",
     [E8]),
    ("E8: the half-integer coset's offset not added back",
     "y1[i] += 0.5;", "y1[i] += 0.0;", [E8]),
    ("group scale: rounded to nearest instead of up",
     "uint16_t h = nqo_f2h_ceil(v);", "uint16_t h = nqo_f2h_rne(v);", [PATH]),
    ("group scale: radius 2^b - 1 instead of 2^(b-1) - 1",
     "float rho = (float)((1 << (bits - 1)) - 1);", "float rho = (float)((1 << bits) - 1);",
     [PATH]),
    ("delta coding: previous minus current",
     "cur[i] = (int8_t)(uint8_t)(((int)cur[i] - (int)prev[i]) & 0xff);",
     "cur[i] = (int8_t)(uint8_t)(((int)prev[i] - (int)cur[i]) & 0xff);", [PATH]),
    ("decode: the code not halved",
     "x[i] = s * (0.5 * (double)c[i]);", "x[i] = s * (double)c[i];", [PATH]),
    ("decode: RoPE restored with the wrong sign",
     "dst[i] = x[i] * cc - x[i + 64] * ss;", "dst[i] = x[i] * cc + x[i + 64] * ss;", [PATH]),
    ("attention: no 1/sqrt(128) scale",
     "double scale = 1.0 / sqrt(128.0);", "double scale = 1.0;", [PATH]),
    ("attention: query head j reads kv head j mod H",
     "int32_t h = j / grp;", "int32_t h = j % H;", [PATH]),
]


def _build(src_text: str, out: str) -> None:
    c = out[:-3] + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *oracle_build.CFLAGS, c, "-o", out, "-lm"], check=True,
                   capture_output=True)


def _pins(lib: str, files) -> int:
    env = dict(os.environ, NQ_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", *files, "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    return r.returncode


def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = open(oracle_build.SRC).read()
    for name, old, new, _ in MUTANTS:
        assert src.count(old) == 1, f"mutation site not unique or missing: {name}"
    clean = str(tmp_path / "clean.so")
    _build(src, clean)
    assert _pins(clean, [NUM, E8, PATH]) == 0, "the pins fail on the unmodified oracle"

    def one(k):
        name, old, new, files = MUTANTS[k]
        lib = str(tmp_path / f"mutant{k}.so")
        _build(src.replace(old, new), lib)
        return name, _pins(lib, files)

    with ThreadPoolExecutor(4) as ex:
        results = list(ex.map(one, range(len(MUTANTS))))
    # 1: a pin failed; negative: the mutant crashed the test process (also caught)
    survivors = [name for name, rc in results if not (rc == 1 or rc < 0)]
    assert not survivors, f"mistakes no pin catches: {survivors}"
