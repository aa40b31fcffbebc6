"""The GPU kernels' GELU (erf form) evaluates the standard normal CDF as
sigmoid(a1 x + a3 x^3 + a5 x^5), x clamped to [-9, 9], with constants fitted by
recsys_jagged_attention_gdpa_amd/csrc/fit_normal_cdf.py.  These tests read the
constants out of the kernel header and check the approximation's stated bound
against scipy's normal CDF (host-side check of the HIP path's arithmetic; the
oracle uses the exact erf)."""
import os
import re

import numpy as np
from scipy.special import expit, ndtr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "recsys_jagged_attention_gdpa_amd", "csrc", "ja_device.h")
BOUND = 1.9e-5


def _coefficients():
    text = open(HEADER).read()
    out = []
    for k in (1, 3, 5):
        m = re.search(rf"PHI_A{k}\s*=\s*([-+0-9.eE]+)f\s*\*\s*-LOG2E", text)
        assert m, f"PHI_A{k} not found"
        out.append(float(m.group(1)))
    return out


def _clamp():
    m = re.search(r"PHI_CLAMP\s*=\s*([0-9.]+)f", open(HEADER).read())
    assert m, "PHI_CLAMP not found"
    return float(m.group(1))


def _phi(x, c):
    a1, a3, a5 = c
    x = np.clip(x, -_clamp(), _clamp())
    return expit(x * (a1 + x * x * (a3 + a5 * x * x)))


def test_normal_cdf_error_bound_on_the_real_line():
    c = _coefficients()
    x = np.concatenate([np.linspace(-12, 12, 480001), np.linspace(-60, -12, 2001), np.linspace(12, 60, 2001)])
    err = np.abs(_phi(x, c) - ndtr(x))
    assert err.max() <= BOUND, err.max()


def test_normal_cdf_is_a_distribution_function():
    c = _coefficients()
    x = np.linspace(-30, 30, 60001)
    f = _phi(x, c)
    assert np.all(np.diff(f) >= -1e-12)                # monotone (up to 1e-12 where it is 1)
    y = np.roots([c[2], c[1], c[0]])                   # p(x) / x = 0 at x^2 = y: where the quintic turns over
    y = y[np.isreal(y) & (y.real > 0)].real
    assert np.all(np.sqrt(y) > _clamp())
    assert abs(_phi(0.0, c) - 0.5) == 0.0              # symmetric: odd polynomial
    assert np.allclose(f + _phi(-x, c), 1.0, atol=1e-15)
    assert f[0] < 1e-12 and f[-1] > 1 - 1e-12


def test_gelu_absolute_error():
    # |GELU error| = |x| |Phi error| <= 1.9e-5 |x|: against P values of order one
    # this is ~100 times below the bf16 rounding (2^-9 relative) of the operands.
    c = _coefficients()
    x = np.concatenate([np.linspace(-40, 40, 400001), np.array([-1e4, -1e3, 1e3, 1e4])])
    err = np.abs(x * _phi(x, c) - x * ndtr(x))
    assert np.all(err <= BOUND * np.maximum(1.0, np.abs(x)) + 1e-12)
    assert err[np.abs(x) > 10].max() < 1e-9  # clamped tails
