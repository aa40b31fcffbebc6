"""Fit the constants of the GPU kernels' standard normal CDF (GELU, erf form).

    python recsys_jagged_attention_gdpa_amd/csrc/fit_normal_cdf.py

The kernels evaluate Phi(x) ~= sigmoid(p(x)) with the odd polynomial
p(x) = a1 x + a3 x^3 + a5 x^5: one v_exp_f32 and one v_rcp_f32 plus three
multiply-adds, against about twice that for a rational erf approximation.
Phi is odd-symmetric about 1/2 and so is sigmoid(p), so the fit runs on
x >= 0.  Start: least squares of p against logit(Phi) on [0, 6]; then the
L^P norm of the error on [0, 12] for P = 8 .. 128, which approaches the
minimax fit.  Prints the coefficients and the largest |error| on a dense grid.
"""
import numpy as np
from scipy.optimize import minimize
from scipy.special import expit, log_ndtr, ndtr


def fit(degree=5, top=9.0, points=18001):
    x = np.linspace(0.0, top, points)
    target = ndtr(x)
    powers = np.arange(1, degree + 1, 2)
    near = x < 6.0
    logit = log_ndtr(x[near]) - log_ndtr(-x[near])
    c = np.linalg.lstsq(np.stack([x[near] ** k for k in powers], 1), logit, rcond=None)[0]

    def err(c):
        return expit(sum(ci * x ** k for ci, k in zip(c, powers))) - target

    for p in (8, 16, 32, 64, 128):
        def norm(c, p=p):
            e = np.abs(err(c)) / 1e-5
            m = e.max()
            return np.log(m) + np.log(np.sum((e / m) ** p)) / p
        c = minimize(norm, c, method="BFGS", options=dict(gtol=1e-12, maxiter=2000)).x
    return c, float(np.max(np.abs(err(c))))


if __name__ == "__main__":
    coef, worst = fit()
    for k, ck in zip((1, 3, 5), coef):
        print(f"a{k} = {float(ck)!r}")
    print(f"max |sigmoid(p(x)) - Phi(x)| = {worst:.3e}")
