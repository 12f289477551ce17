"""The kernels' GELU (csrc/atlas_mem_gelu.h) evaluates erf by Abramowitz &
Stegun, Handbook of Mathematical Functions, formula 7.1.26, whose absolute
error is at most 1.5e-7.  The constants are read from the header itself and
the formula is checked against math.erf on a dense grid, so a mistyped
constant fails here, on the CPU."""
import math
import os
import re

import numpy as np

HDR = os.path.join(os.path.dirname(__file__), "..", "test_memorization_sequence_amd", "csrc", "atlas_mem_gelu.h")


def _constants():
    src = open(HDR).read()
    body = src[src.index("two_phi"):]
    p = float(re.search(r"fmaf\(([0-9.]+)f, x, 1\.0f\)", body).group(1))
    nums = re.search(r"const float poly = t \* (.*?);", body, re.S).group(1)
    vals = [float(v) for v in re.findall(r"-?[0-9]+\.[0-9]+(?=f)", nums)]
    # innermost first in the source: a5, a4, a3, a2, a1
    a5, a4, a3, a2, a1 = vals
    return p, (a1, a2, a3, a4, a5)


def _erf_as(x):
    p, (a1, a2, a3, a4, a5) = _constants()
    ax = np.abs(x)
    t = 1.0 / (1.0 + p * ax)
    y = 1.0 - t * (a1 + t * (a2 + t * (a3 + t * (a4 + t * a5)))) * np.exp(-ax * ax)
    return np.sign(x) * y


def test_constants_are_the_published_ones():
    p, a = _constants()
    assert p == 0.3275911
    assert a == (0.254829592, -0.284496736, 1.421413741, -1.453152027, 1.061405429)


def test_erf_error_bound():
    x = np.linspace(-6.0, 6.0, 200001)
    ref = np.array([math.erf(v) for v in x])
    assert np.max(np.abs(_erf_as(x) - ref)) <= 1.5e-7


def test_gelu_and_derivative():
    z = np.linspace(-8.0, 8.0, 40001)
    s2 = math.sqrt(2.0)
    exact = np.array([0.5 * v * (1.0 + math.erf(v / s2)) for v in z])
    dexact = np.array([0.5 * (1.0 + math.erf(v / s2)) + v * math.exp(-0.5 * v * v) / math.sqrt(2 * math.pi) for v in z])
    approx = 0.5 * z * (1.0 + _erf_as(z / s2))
    dapprox = 0.5 * (1.0 + _erf_as(z / s2)) + z * np.exp(-0.5 * z * z) / math.sqrt(2 * math.pi)
    assert np.max(np.abs(approx - exact) / (1.0 + np.abs(z))) <= 1.5e-7
    assert np.max(np.abs(dapprox - dexact)) <= 1.5e-7
