"""Host logic of the GPU parity checks (tests/gpu_helpers.py), on the CPU: the certificate that a
flagged mismatch must pass and the exact keep-set rule applied to the GPU's own scores. Wrong
"GPU results" are built here by hand; nothing runs on a GPU.
"""
import itertools

import numpy as np
import pytest

import oracle
from gpu_helpers import certify_group, gpu_keep_set, is_e8_code


def test_is_e8_code():
    assert is_e8_code(np.array([2, 2, 0, 0, 0, 0, 0, 0]))          # y = (1, 1, 0^6)
    assert is_e8_code(np.array([1] * 8))                              # y = (1/2)^8
    assert is_e8_code(np.array([-1, -1, 1, 1, 1, 1, 1, 1]))
    assert not is_e8_code(np.array([2, 0, 0, 0, 0, 0, 0, 0]))        # odd coordinate sum
    assert not is_e8_code(np.array([-1, 1, 1, 1, 1, 1, 1, 1]))       # odd number of minus signs
    assert not is_e8_code(np.array([1, 2, 1, 1, 1, 1, 1, 1]))        # mixed parity


def test_gpu_keep_set_against_brute_force():
    rng = np.random.default_rng(3)
    for T, W, e in [(1, 0, 600), (5, 10, 600), (40, 3, 900), (64, 8, 500), (30, 0, 600),
                    (50, 5, 0), (50, 5, 1000)]:
        for trial in range(20):
            s = np.round(rng.standard_normal(T), 1)                 # many exact ties
            s[rng.random(T) < 0.2] = -0.0
            n_keep = oracle.keep_count(T, W, e)
            got = gpu_keep_set(s, T, W, n_keep)
            # brute force: the protected set plus the m candidates first in (score desc,
            # position asc) order
            c_end = T - W
            cand = list(range(1, c_end)) if c_end > 1 else []
            prot = [0] + list(range(max(1, c_end), T)) if T > 0 else []
            m = n_keep - len(prot)
            best = sorted(cand, key=lambda t: (-float(s[t]) + 0.0, t))[:m]
            assert list(got) == sorted(prot + best)
            assert len(got) == n_keep


def test_certificate_accepts_the_other_side_of_a_tie():
    # u exactly between y = 0 and y = (1, 1, 0^6): both are nearest points (scale 1: u = x)
    u = np.array([0.5, 0.5, 0, 0, 0, 0, 0, 0], np.float32)
    c_or, _ = oracle.e8_nearest(u[None])
    c_or = c_or[0]
    alt = np.array([2, 2, 0, 0, 0, 0, 0, 0], np.int8)
    if np.array_equal(alt, c_or):
        alt = np.zeros(8, np.int8)
    assert abs(oracle.e8_margin(u, alt)) < 1e-12 and abs(oracle.e8_margin(u, c_or)) < 1e-12
    certify_group(u, alt, 0x3C00, c_or, 0x3C00, flag=1, bits=2)


@pytest.mark.parametrize("case", ["not-lattice", "outside-cube", "not-nearest", "unflagged",
                                  "scale-differs"])
def test_certificate_rejects(case):
    u = np.array([0.3, -0.2, 0.1, 0.7, -0.4, 0.2, 0.05, 0.9], np.float32)
    c_or, _ = oracle.e8_nearest(u[None])
    c_or = c_or[0]
    bits, s = 3, 0x3C00
    c, s_gpu, flag = c_or.copy(), s, 1
    if case == "not-lattice":
        c[0] += 1
    elif case == "outside-cube":
        c = np.array([8, 0, 0, 0, 0, 0, 0, 0], np.int8)
    elif case == "not-nearest":
        c[0] += 2
        c[1] += 2                                          # a lattice point, but not nearest
    elif case == "unflagged":
        c[0] += 2
        c[1] += 2
        flag = 0
    elif case == "scale-differs":
        s_gpu, flag = s + 1, 3                   # scales are compared bit for bit
    with pytest.raises(AssertionError):
        certify_group(u, c, s_gpu, c_or, s, flag, bits)


def test_lattice_codes_all_pass_membership():
    for y in itertools.product((-1, 0, 1), repeat=4):
        v = np.array(list(y) + [0, 0, 0, 0])
        if v.sum() % 2 == 0:
            assert is_e8_code(2 * v)
