"""The GPU encode's fp32 arithmetic, emulated on the host (tests/emul/encode_arith.c) and checked
against the oracle. The kernel's lattice codes may differ from the oracle's only inside the
near-tie bands; this test shows why:
- both of its divisions are one product with a two-part reciprocal h + l of the divisor and
  one fused multiply-add; h + l is 1/d to 2^-45 for every binary16 divisor and every h that a
  reciprocal accurate to one ulp may return (exhaustive);
- its group scale a/rho and the round-up to binary16 (integer rounding of the fp32 bits) equal
  the oracle's for every positive fp32 a (exhaustive);
- its u = x/s equals the correctly rounded quotient for every binary16 significand, both
  candidate reciprocals and every fp32 significand (exhaustive: 1.7e10 cases), and over
  random exponents for every quotient of at least 2^-100 (below, within one ulp, which moves
  no lattice distance by more than 2^-99, far inside the near-tie band): the lattice step sees
  the oracle's u;
- its E8 decision in fp32 (magic-number rounding, distance differences, arg-max/min keys
  carrying the index in their low bits) agrees with the oracle's exact nearest point except
  inside the Voronoi near-tie band, on millions of random groups and on groups built on and
  near the Voronoi facets, rounding boundaries and equal rounding errors.
CPU only.
"""
import os
import re
import shutil
import subprocess

import pytest

from oracle import build as oracle_build

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "emul", "encode_arith.c")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(oracle_build.LIB):
        oracle_build.build()
    out = str(tmp_path_factory.mktemp("emul") / "encode_arith")
    lib_dir = os.path.dirname(oracle_build.LIB)
    cmd = ["gcc", "-O3", "-fopenmp", "-ffp-contract=off", "-std=c11", "-Wall", SRC, "-o", out,
           f"-L{lib_dir}", "-loracle", f"-Wl,-rpath,{lib_dir}", "-lm"]
    # hardware fused multiply-add where the host has it (the software fmaf is exact too)
    try:
        subprocess.run(cmd[:1] + ["-mfma"] + cmd[1:], check=True, capture_output=True)
    except subprocess.CalledProcessError:
        subprocess.run(cmd, check=True, capture_output=True)
    return out


def test_encode_arithmetic_matches_the_oracle(harness):
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    r = subprocess.run([harness, "2000000", "300000", "1"], capture_output=True, text=True,
                       timeout=900, env=env)
    print(r.stdout)
    lines = {ln.split()[0] + (ln.split()[1] if ln.startswith("e8") else ""): ln
             for ln in r.stdout.splitlines() if ln.strip()}
    for name in ("scale_quotient", "f16_ceil", "reciprocal", "quotient", "quotient_range"):
        assert re.search(r"\bbad=0\b", lines[name]), lines[name]
    assert "stride=1" in lines["quotient"]                       # exhaustive
    assert int(re.search(r"cases=(\d+)", lines["quotient"]).group(1)) == 2 * (1024 << 23)
    # every positive finite fp32 for each of the three radii
    assert int(re.search(r"cases=(\d+)", lines["scale_quotient"]).group(1)) == 3 * (0x7f800000 - 1)
    for bits in (2, 3, 4):
        ln = lines[f"e8bits={bits}"]
        kv = dict(kv.split("=") for kv in ln.split()[1:])
        assert int(kv["groups"]) > 2_000_000
        assert int(kv["outside_band"]) == 0 and int(kv["gpu_not_nearest"]) == 0, ln
        assert int(kv["differ"]) > 0          # the crafted ties do reach the decision's edges
    assert r.returncode == 0 and "result ok" in r.stdout
