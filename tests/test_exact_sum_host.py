"""The library's exact-sum accumulator (dit_amd/csrc/exact_sum.h, used by the key-mean
kernels), built for the host with g++ and checked against exact rational sums rounded once
to fp64: wide exponent ranges, fp32 denormals, cancellation, ties to even, limb boundaries.
CPU only."""
import ctypes
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    out = tmp_path_factory.mktemp("exact") / "libexact.so"
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC",
                    "-I", os.path.join(ROOT, "dit_amd", "csrc"),
                    os.path.join(ROOT, "tests", "exact_sum_host.cpp"), "-o", str(out)], check=True)
    L = ctypes.CDLL(str(out))
    L.exact_sum_host.restype = ctypes.c_double
    L.exact_sum_host.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_int64]
    return L


def _sum(L, xs):
    a = np.ascontiguousarray(xs, dtype=np.float64)
    return L.exact_sum_host(a.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), len(a))


def _exact(xs):
    return float(sum((Fraction(float(x)) for x in xs), Fraction(0)))


def _wide_fp32(rng, n, lo_exp, hi_exp):
    m = rng.uniform(1.0, 2.0, size=n)
    e = rng.integers(lo_exp, hi_exp + 1, size=n)
    s = rng.choice([-1.0, 1.0], size=n)
    return (s * np.ldexp(m, e)).astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("lo_exp,hi_exp", [(-3, 3), (-20, 20), (-60, 60), (-149, -100), (90, 127),
                                           (-149, 127)])
def test_random_fp32_values(lib, lo_exp, hi_exp):
    rng = np.random.default_rng(abs(lo_exp) * 1000 + hi_exp)
    for n in (1, 2, 7, 300, 3000):
        xs = _wide_fp32(rng, n, lo_exp, hi_exp)
        assert _sum(lib, xs) == _exact(xs), (n, lo_exp, hi_exp)


def test_exact_partial_sums_as_inputs(lib):
    """fp64 inputs that are exact sums of fp32 values (not themselves fp32), as the slab
    partial sums are."""
    rng = np.random.default_rng(3)
    xs = []
    for _ in range(500):
        a, b = _wide_fp32(rng, 2, -30, 30)
        s = a + b
        if Fraction(s) == Fraction(a) + Fraction(b):
            xs.append(s)
    xs = np.array(xs)
    assert _sum(lib, xs) == _exact(xs)


def test_ties_cancellation_and_edges(lib):
    two53 = 2.0 ** 53
    assert _sum(lib, [two53, 1.0]) == two53                      # tie -> even
    assert _sum(lib, [two53, 1.0, 2.0 ** -149]) == two53 + 2     # just above the tie
    assert _sum(lib, [two53 + 2, 1.0]) == two53 + 4               # tie -> even (upwards)
    assert _sum(lib, [-two53, -1.0]) == -two53
    assert _sum(lib, [2.0 ** 60, 1.0, -(2.0 ** 60)]) == 1.0
    assert _sum(lib, [3.5, -3.5]) == 0.0 and _sum(lib, []) == 0.0
    assert _sum(lib, [2.0 ** -149]) == 2.0 ** -149
    assert _sum(lib, [2.0 ** 127, 2.0 ** 127]) == 2.0 ** 128
    xs = [2.0 ** e for e in range(-149, 128)]                       # every limb boundary
    assert _sum(lib, xs) == _exact(xs)
    xs = [(-1.0) ** e * 2.0 ** e for e in range(-149, 128)]
    assert _sum(lib, xs) == _exact(xs)
    big = np.full(3 * (1 << 20) + 5, 2.0 ** 127 * 1.5)            # normalisation between adds
    assert _sum(lib, big) == float(Fraction(2.0 ** 127 * 1.5) * len(big))
