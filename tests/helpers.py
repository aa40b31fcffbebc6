"""Shared test helpers: run the oracle on a synthetic workload, compare results."""
import numpy as np

from oracle import ref


def bias_kw(w):
    return dict(bias_kind=w.bias_kind, bias_table=w.bias_table, bias_lo=w.bias_lo,
                bias_hi=w.bias_hi)


def oracle_fwd(w, nthreads=0):
    if w.mode == "gdpa":
        o = ref.gdpa_fwd(w.q, w.k, w.v, w.q_off, w.kv_off, scale=w.scale, act=w.act,
                         lq_fixed=w.lq_fixed, causal=w.causal, nthreads=nthreads, **bias_kw(w))
        return {"o": o}
    o, lse = ref.attn_fwd(w.q, w.k, w.v, w.q_off, w.kv_off, scale=w.scale, lq_fixed=w.lq_fixed,
                          causal=w.causal, nthreads=nthreads, **bias_kw(w))
    return {"o": o, "lse": lse}


def oracle_bwd(w, nthreads=0):
    if w.mode == "gdpa":
        dq, dk, dv = ref.gdpa_bwd(w.q, w.k, w.v, w.dout, w.q_off, w.kv_off, scale=w.scale,
                                  act=w.act, causal=w.causal, nthreads=nthreads, **bias_kw(w))
    else:
        dq, dk, dv = ref.attn_bwd(w.q, w.k, w.v, w.dout, w.q_off, w.kv_off, scale=w.scale,
                                  causal=w.causal, nthreads=nthreads, **bias_kw(w))
    return {"dq": dq, "dk": dk, "dv": dv}


def max_rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    den = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / den)


def row_check(got, want, tau, what="", floor_frac=1e-6):
    """Per-row tolerance: for every row r (all leading dims, last dim = the row),
    max_d |got - want| <= tau * max_d |want|.  Rows whose reference is exactly zero
    must be exactly zero.  Rows whose reference maximum is below floor_frac times
    the tensor maximum are compared against that floor instead (reported)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if want.size == 0:
        return {"rows": 0, "worst": 0.0, "floored": 0}
    g = got.reshape(-1, got.shape[-1])
    r = want.reshape(-1, want.shape[-1])
    assert np.isfinite(g).all(), f"{what}: non-finite values in the GPU result"
    err = np.abs(g - r).max(axis=1)
    ref_max = np.abs(r).max(axis=1)
    zero = ref_max == 0
    bad_zero = zero & (err != 0)
    assert not bad_zero.any(), f"{what}: {int(bad_zero.sum())} rows should be exactly zero"
    floor = floor_frac * max(float(ref_max.max()), 1e-300)
    den = np.maximum(ref_max, floor)
    ratio = np.where(zero, 0.0, err / den)
    worst = int(np.argmax(ratio))
    assert ratio[worst] <= tau, (f"{what}: row {worst} err {err[worst]:.3e} ref max "
                                 f"{ref_max[worst]:.3e} ratio {ratio[worst]:.3e} > {tau}")
    return {"rows": len(ratio), "worst": float(ratio[worst]),
            "floored": int(((ref_max < floor) & ~zero).sum())}
