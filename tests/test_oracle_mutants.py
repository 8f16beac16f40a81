"""The oracle's pins have teeth. Each plausible mistake below is planted in a copy of the
oracle's source: a flipped sign, a dropped term, a wrong index or bound, a swapped operand, or a
wrong rounding or tie rule. The pin tests it concerns then run against the copy in a subprocess,
and every mutant must make them fail. The unmodified source, run the same way, must pass them.
- C oracle: the copy is built with the oracle's own flags, and NQ_ORACLE_LIB points the wrapper
  at it.
- numpy oracles (the attention-weight scorer, the Lloyd-Max baseline): the pins run from a copy
  of the tests and oracle packages with the mutated module.
Nothing here touches a GPU or the GPU library's arithmetic.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import shutil

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from oracle import build as oracle_build  # noqa: E402

NUM = "tests/test_oracle_numeric.py"
E8 = "tests/test_oracle_e8.py"
PATH = "tests/test_oracle_path.py"
NT = "tests/test_oracle_near_ties.py"

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
     "return (float)((1 << (bits - 1)) - 1);", "return (float)((1 << bits) - 1);",
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
    ("group scale: no clamp at +rho", "if (q > rho) q = rho;", "", [PATH]),
    ("group scale: no clamp at -rho", "if (q < -rho) q = -rho;", "", [PATH]),
    ("group scale: the absmax skips the first coordinate",
     "for (int i = 0; i < 8; i++) a = fabsf(xg[i]) > a ? fabsf(xg[i]) : a;",
     "for (int i = 1; i < 8; i++) a = fabsf(xg[i]) > a ? fabsf(xg[i]) : a;", [PATH]),
    ("selection: the window starts one token late",
     "keep[t] = (t == 0 || t >= c_end) ? 1 : 0;", "keep[t] = (t == 0 || t > c_end) ? 1 : 0;",
     [PATH]),
    ("selection: BOS not protected",
     "keep[t] = (t == 0 || t >= c_end) ? 1 : 0;", "keep[t] = (t >= c_end) ? 1 : 0;", [PATH]),
    ("selection: one candidate too many",
     "for (int32_t i = 0; i < m; i++) keep[c[i].t] = 1;",
     "for (int32_t i = 0; i <= m && i < n_cand; i++) keep[c[i].t] = 1;", [PATH]),
    ("keep count: BOS not counted among the protected",
     "int64_t prot = (int64_t)W + 1 < T ? (int64_t)W + 1 : T;",
     "int64_t prot = (int64_t)W < T ? (int64_t)W : T;", [PATH]),
    ("rotary table: angles in fp32",
     "double phi = (double)p * theta[i];", "double phi = (double)((float)p * (float)theta[i]);",
     [NUM]),
    ("fp16 round-up: rounds to nearest",
     "uint16_t nqo_f2h_ceil(float v)\n{", "uint16_t nqo_f2h_ceil(float v)\n{\n    return nqo_f2h_rne(v);",
     [NUM]),
    ("fp16 to fp32: subnormals flushed to zero",
     "float nqo_h2f(uint16_t h)\n{",
     "float nqo_h2f(uint16_t h)\n{\n    if (((h >> 10) & 0x1f) == 0) return (h & 0x8000) ? -0.0f : 0.0f;",
     [NUM]),
    ("E8: a distance tie goes to the half-integer coset",
     "const double *y = (d0 <= d1) ? y0 : y1;", "const double *y = (d0 < d1) ? y0 : y1;", [E8]),
    ("E8: rint ties away from zero",
     "f[i] = nearbyint(v[i]); sum += f[i];", "f[i] = round(v[i]); sum += f[i];", [E8]),
    ("E8: a zero-error coordinate moves away from zero",
     "else f[j] += (f[j] > 0.0) ? -1.0 : 1.0;", "else f[j] += (f[j] > 0.0) ? 1.0 : -1.0;", [E8]),
    ("decode: the running sum not taken mod 256",
     "c[i] = (int)(int8_t)(uint8_t)((c[i] + d[o * HD + i]) & 0xff);",
     "c[i] = c[i] + d[o * HD + i];", [PATH]),
    ("decode: the scale of the wrong group",
     "double s = (double)nqo_h2f(scales[o * NG + i / 8]);",
     "double s = (double)nqo_h2f(scales[o * NG + i % 16]);", [PATH]),
    ("attention: softmax without the maximum subtracted",
     "for (int32_t t = 0; t < n; t++) { z[t] = exp(z[t] - mx); den += z[t]; }",
     "for (int32_t t = 0; t < n; t++) { z[t] = exp(z[t]); den += z[t]; }", [PATH]),
    ("nominal ratio: one scale per group instead of two",
     "2.0 * 16.0 * 16.0", "16.0 * 16.0", [PATH]),
    ("encode: keys not rotated back",
     "            if (is_key)\n                nqo_rope_undo(", "            if (0)\n                nqo_rope_undo(",
     [PATH]),
    ("encode: values rotated back too",
     "            if (is_key)\n                nqo_rope_undo(", "            if (1)\n                nqo_rope_undo(",
     [PATH]),
    # the near-tie classification: it decides which GPU results may differ from the oracle's
    ("Voronoi near-tie: every group flagged",
     "return nqo_e8_margin(u, c) < lim;", "return 1;", [NT]),
    ("Voronoi near-tie: no group flagged",
     "return nqo_e8_margin(u, c) < lim;", "return 0;", [NT]),
    ("Voronoi near-tie: band 1000x too wide",
     "double lim = 1e-6 * (umax", "double lim = 1e-3 * (umax", [NT]),
    ("Voronoi near-tie: band not scaled by the largest coordinate",
     "double lim = 1e-6 * (umax > 1.0f ? (double)umax : 1.0);", "double lim = 1e-6;", [NT]),
    ("scale near-tie: every group flagged",
     "return near_lo || near_hi;", "return 1;", [NT]),
    ("scale near-tie: no group flagged",
     "return near_lo || near_hi;", "return 0;", [NT]),
    ("scale near-tie: lower band 1000x too wide",
     "int near_lo = dv - lo <= 1e-6 * dv;", "int near_lo = dv - lo <= 1e-3 * dv;", [NT]),
    ("scale near-tie: upper band 1000x too wide",
     "int near_hi = h != 0x7bff && hi - dv <= 1e-6 * dv;",
     "int near_hi = h != 0x7bff && hi - dv <= 1e-3 * dv;", [NT]),
    ("scale near-tie: a saturated scale taken to have an upper step",
     "int near_hi = h != 0x7bff && hi - dv <= 1e-6 * dv;",
     "int near_hi = hi - dv <= 1e-6 * dv;", [NT]),
    ("scale near-tie: the step below a saturated scale ignored",
     "int near_lo = dv - lo <= 1e-6 * dv;", "int near_lo = h != 0x7bff && dv - lo <= 1e-6 * dv;",
     [NT]),
    ("eviction near-tie: every candidate flagged",
     "if (fabs(c[i].s - th) <= 1e-6 * fabs(th)) near[c[i].t] = 1;", "near[c[i].t] = 1;", [NT]),
    ("eviction near-tie: no candidate flagged",
     "if (fabs(c[i].s - th) <= 1e-6 * fabs(th)) near[c[i].t] = 1;", ";", [NT]),
    ("eviction near-tie: band 1000x too wide",
     "if (fabs(c[i].s - th) <= 1e-6 * fabs(th))", "if (fabs(c[i].s - th) <= 1e-3 * fabs(th))",
     [NT]),
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
    assert _pins(clean, [NUM, E8, PATH, NT]) == 0, "the pins fail on the unmodified oracle"

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


ATT = "tests/test_oracle_attn_scorer.py"
LM = "tests/test_oracle_lloyd_max.py"

# (what the mistake is, module file, exact text, replacement, pin file that must catch it)
PY_MUTANTS = [
    ("attention scorer: logits scaled by 1/128", "attn_scorer.py",
     "/ np.sqrt(float(D))", "/ float(D)", ATT),
    ("attention scorer: query head j reads kv head j mod H", "attn_scorer.py",
     "K[j // G].T", "K[j % H].T", ATT),
    ("attention scorer: a query does not see its own position", "attn_scorer.py",
     "z = Z[w, :P + 1]", "z = Z[w, :P]", ATT),
    ("attention scorer: window positions shifted by one", "attn_scorer.py",
     "P = T - W + w ", "P = T - W + w - 1 ", ATT),
    ("Lloyd-Max: centroid with the wrong sign", "lloyd_max.py",
     "y_new = np.array([(_phi(a) - _phi(b))", "y_new = np.array([(_phi(b) - _phi(a))", LM),
    ("Lloyd-Max: thresholds not at the midpoints", "lloyd_max.py",
     "        t = 0.5 * (y[:-1] + y[1:])\n", "        t = 0.45 * (y[:-1] + y[1:])\n", LM),
    ("Lloyd-Max: RMS over 4 instead of 8 values", "lloyd_max.py",
     "ss * np.float32(0.125)", "ss * np.float32(0.25)", LM),
    ("Lloyd-Max: a value on a threshold takes the upper cell", "lloyd_max.py",
     "int(np.sum(t32 < ui))", "int(np.sum(t32 <= ui))", LM),
    ("Lloyd-Max: all-zero group indexed 0", "lloyd_max.py",
     "np.full(8, 1 << (bits - 1), np.uint8)", "np.zeros(8, np.uint8)", LM),
    ("Lloyd-Max: scale not saturated at 65504", "lloyd_max.py",
     "s16 = min(f2h_rne(float(s32)), 0x7BFF)", "s16 = f2h_rne(float(s32))", LM),
    ("Lloyd-Max: decode without the 1/sqrt(128)", "lloyd_max.py",
     "        x = x / math.sqrt(128.0)\n", "", LM),
    ("Lloyd-Max: decode restores RoPE with the wrong sign", "lloyd_max.py",
     "x[..., 64:] = hi * C + lo * S", "x[..., 64:] = hi * C - lo * S", LM),
    ("Lloyd-Max scale near-tie: every group flagged", "lloyd_max.py",
     "near |= abs(float(s32) - b) <= 1e-6 * float(s32)", "near |= True", NT),
    ("Lloyd-Max scale near-tie: no group flagged", "lloyd_max.py",
     "near |= abs(float(s32) - b) <= 1e-6 * float(s32)", "near |= False", NT),
    ("Lloyd-Max scale near-tie: band 1000x too wide", "lloyd_max.py",
     "near |= abs(float(s32) - b) <= 1e-6 * float(s32)",
     "near |= abs(float(s32) - b) <= 1e-3 * float(s32)", NT),
    ("Lloyd-Max threshold near-tie: every group flagged", "lloyd_max.py",
     "near |= bool(np.any(np.abs(ui - t32) <= 1e-6 * np.maximum(1.0, np.abs(t32))))",
     "near |= True", NT),
    ("Lloyd-Max threshold near-tie: no group flagged", "lloyd_max.py",
     "near |= bool(np.any(np.abs(ui - t32) <= 1e-6 * np.maximum(1.0, np.abs(t32))))",
     "near |= False", NT),
    ("Lloyd-Max threshold near-tie: band 1000x too wide", "lloyd_max.py",
     "np.abs(ui - t32) <= 1e-6 * np.maximum", "np.abs(ui - t32) <= 1e-3 * np.maximum", NT),
]


def _py_pins(root: str, test_file: str) -> int:
    env = dict(os.environ, NQ_ORACLE_LIB=oracle_build.LIB)
    r = subprocess.run([sys.executable, "-m", "pytest", test_file, "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=root, env=env, capture_output=True,
                       text=True, timeout=600)
    return r.returncode


def _tree(dst: str) -> None:
    """A copy of what the numpy oracles' pins import: tests, oracle (sources only), kvsynth."""
    ign = shutil.ignore_patterns("_build", "__pycache__", "*.so")
    for d in ("tests", "oracle", "kvsynth"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(dst, d), ignore=ign)
    shutil.copy(os.path.join(ROOT, "pytest.ini"), dst)


def test_every_planted_mistake_in_the_numpy_oracles_fails_a_pin(tmp_path):
    if not os.path.exists(oracle_build.LIB):
        oracle_build.build()
    srcs = {}
    for name, mod, old, new, _ in PY_MUTANTS:
        if mod not in srcs:
            srcs[mod] = open(os.path.join(ROOT, "oracle", mod)).read()
        assert srcs[mod].count(old) == 1, f"mutation site not unique or missing: {name}"
    clean = str(tmp_path / "clean")
    _tree(clean)
    assert _py_pins(clean, ATT) == 0 and _py_pins(clean, LM) == 0 and _py_pins(clean, NT) == 0, \
        "the pins fail on the unmodified numpy oracles"

    def one(k):
        name, mod, old, new, pin = PY_MUTANTS[k]
        root = str(tmp_path / f"mutant{k}")
        _tree(root)
        with open(os.path.join(root, "oracle", mod), "w") as f:
            f.write(srcs[mod].replace(old, new))
        return name, _py_pins(root, pin)

    with ThreadPoolExecutor(4) as ex:
        results = list(ex.map(one, range(len(PY_MUTANTS))))
    survivors = [name for name, rc in results if not (rc == 1 or rc < 0)]
    assert not survivors, f"mistakes no pin catches: {survivors}"
