"""Shared test helpers: run the oracle on a synthetic workload, compare results."""
import math

import numpy as np
import torch

from oracle import mx, ref


def bias_kw(w):
    """Bias, sliding-window and rotary-embedding arguments of the oracle calls.  With
    bf16 operands the turned rows are bf16 values (rounded as the GPU rounds them)."""
    return dict(bias_kind=w.bias_kind, bias_table=w.bias_table, bias_lo=w.bias_lo,
                bias_hi=w.bias_hi, window=w.window, rope_base=w.rope_base,
                rope_bf16=w.dtype == torch.bfloat16)


def inputs(w):
    """q, k, v as the oracle reads them: MXFP8 tensors decoded (exactly) to float32."""
    out = []
    for name in ("q", "k", "v"):
        t = getattr(w, name)
        if name in w.mx:
            t = mx.decode_f32(t.numpy(), w.mx_scales[name].numpy())
        out.append(t)
    return out


def oracle_fwd(w, nthreads=0):
    q, k, v = inputs(w)
    if w.mode == "gdpa":
        o = ref.gdpa_fwd(q, k, v, w.q_off, w.kv_off, scale=w.scale, act=w.act,
                         lq_fixed=w.lq_fixed, causal=w.causal, nthreads=nthreads, **bias_kw(w))
        return {"o": o}
    o, lse = ref.attn_fwd(q, k, v, w.q_off, w.kv_off, scale=w.scale, lq_fixed=w.lq_fixed,
                          causal=w.causal, nthreads=nthreads, **bias_kw(w))
    return {"o": o, "lse": lse}


def fp8_pv(w):
    """Whether the HIP path forms P V with P in FP8: MXFP8 inputs with D = 64 or 128."""
    return bool(w.mx) and w.D >= 64


def oracle_fwd_fp8_pv(w):
    """The oracle forward with P in FP8 (oracle/mx.py, fwd_fp8_pv) for an MXFP8
    workload: O, for JFA the LSE, and per row the bound of one encoding step of
    its largest P term ('flip', [T, H])."""
    q, k, _ = inputs(w)
    o, lse, flip = mx.fwd_fp8_pv(w.mode, np.asarray(q), np.asarray(k), w.v.numpy(), w.mx_scales["v"].numpy(),
                                 w.q_off, w.kv_off, scale=w.scale, act=w.act, lq_fixed=w.lq_fixed,
                                 causal=w.causal, window=w.window, bias_kind=w.bias_kind,
                                 bias_table=None if w.bias_table is None else w.bias_table.numpy(),
                                 bias_lo=w.bias_lo, bias_hi=w.bias_hi)
    return {"o": o, "lse": lse, "flip": flip} if w.mode == "jfa" else {"o": o, "flip": flip}


def fp8_pv_check(got, want, flip, tau, what="", zero_rows=None, max_flip_frac=5e-3):
    """O rows against the oracle with P in FP8: max_d |got - want| <= tau * max_d |want|
    on every row but a few.  The GPU encodes P from its fp32 value, so a P element
    lying within that value's error of an E4M3 midpoint may land one step from the
    oracle's choice; a row may carry two such steps (flip_r bounds one), and rows
    that need them are counted.  The fp32 activation (hardware exp2 and reciprocal)
    is good to ~1e-6 relative and E4M3 midpoints are 2^-4 to 2^-3 apart, so about
    one element in 10^4 to 10^5 can land on the other side: at most max(4,
    max_flip_frac of the rows) rows may need a step (a planted error shows in far
    more rows, or beyond two steps).  Rows in zero_rows must be exactly zero."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if want.size == 0:
        return {"rows": 0, "flipped": 0}
    g = got.reshape(-1, got.shape[-1])
    r = want.reshape(-1, want.shape[-1])
    fl = np.asarray(flip, dtype=np.float64).reshape(-1)
    assert np.isfinite(g).all(), f"{what}: non-finite values in the GPU result"
    err = np.abs(g - r).max(axis=1)
    ref_max = np.abs(r).max(axis=1)
    zero = np.zeros(len(err), dtype=bool) if zero_rows is None else np.asarray(zero_rows).reshape(-1)
    assert not (zero & (ref_max != 0)).any(), f"{what}: oracle row expected zero is not"
    assert not (zero & (np.abs(g).max(axis=1) != 0)).any(), f"{what}: rows expected zero are not"
    plain = err <= tau * ref_max
    flipped = ~plain & ~zero
    ok_flip = err <= tau * ref_max + 2.0 * fl
    worst = int(np.argmax(np.where(zero, 0.0, err / np.maximum(tau * ref_max + 2.0 * fl, 1e-300))))
    n_flip = int(flipped.sum())
    print(f"[fp8-pv check] {what}: rows {len(err)}, rows needing an encoding step {n_flip}", flush=True)
    assert (ok_flip | zero).all(), (f"{what}: row {worst} err {err[worst]:.3e} ref max {ref_max[worst]:.3e} "
                                    f"flip {fl[worst]:.3e}")
    assert n_flip <= max(4, math.ceil(max_flip_frac * len(err))), f"{what}: {n_flip} rows needed an encoding step"
    return {"rows": len(err), "flipped": n_flip}


# Unit roundoffs the kernels work with: dX enters the dQ / dK products as bf16 (fp32
# for fp32 tensors); JFA's delta comes from O held to 16 bits (bf16 output plus its
# bf16 residual; fp32 O for fp32 tensors).
DX_UNIT = {torch.bfloat16: 2.0 ** -8, torch.float32: 2.0 ** -24}
DELTA_UNIT = {torch.bfloat16: 2.0 ** -16, torch.float32: 2.0 ** -24}


def oracle_bwd(w, nthreads=0, noise=False, delta_unit=None):
    """The oracle's gradients; with noise=True also the rounding-noise scale of every
    dQ row ('nq') and dK row ('nk'), see ref.bwd_noise (delta_unit: the relative
    precision of the O that delta is formed from, default the residual interface's)."""
    q, k, v = inputs(w)
    if noise:
        du = DELTA_UNIT[w.dtype] if delta_unit is None else delta_unit
        dq, dk, dv, nq, nk = ref.bwd_noise(w.mode, q, k, v, w.dout, w.q_off, w.kv_off, scale=w.scale,
                                           act=w.act if w.mode == "gdpa" else "silu", causal=w.causal,
                                           dx_unit=DX_UNIT[w.dtype], delta_unit=du, nthreads=nthreads,
                                           **bias_kw(w))
        return {"dq": dq, "dk": dk, "dv": dv, "nq": nq, "nk": nk}
    if w.mode == "gdpa":
        dq, dk, dv = ref.gdpa_bwd(q, k, v, w.dout, w.q_off, w.kv_off, scale=w.scale,
                                  act=w.act, causal=w.causal, nthreads=nthreads, **bias_kw(w))
    else:
        dq, dk, dv = ref.attn_bwd(q, k, v, w.dout, w.q_off, w.kv_off, scale=w.scale,
                                  causal=w.causal, nthreads=nthreads, **bias_kw(w))
    return {"dq": dq, "dk": dk, "dv": dv}


def oracle_dbias(w, nthreads=0):
    """dL/dtable [H, hi - lo + 1] for a workload with a bias table and per-sample queries."""
    q, k, v = inputs(w)
    if w.mode == "gdpa":
        return ref.gdpa_dbias(q, k, v, w.dout, w.q_off, w.kv_off, scale=w.scale, act=w.act,
                              causal=w.causal, nthreads=nthreads, **bias_kw(w))
    return ref.attn_dbias(q, k, v, w.dout, w.q_off, w.kv_off, scale=w.scale,
                          causal=w.causal, nthreads=nthreads, **bias_kw(w))


def max_rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    den = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / den)


def _visible_counts(w, b):
    """Keys each query row of sample b sees, and for each key the number of rows that
    see it and the number of those rows that see at least two keys."""
    lq, lk, win = int(w.lq[b]), int(w.lk[b]), w.window
    ia = np.arange(lq, dtype=np.int64) + lk - lq  # aligned positions
    ke = np.clip(ia + 1, 0, lk) if w.causal else (np.clip(ia + win, 0, lk) if win else np.full(lq, lk))
    kb = np.clip(ia - win + 1, 0, None) if win else np.zeros(lq, dtype=np.int64)
    n = np.maximum(ke - kb, 0)
    # key j is seen by rows i with kb_i <= j < ke_i: difference arrays over j
    seen = np.zeros(lk + 1, dtype=np.int64)
    multi = np.zeros(lk + 1, dtype=np.int64)
    ok = n > 0
    np.add.at(seen, kb[ok], 1)
    np.add.at(seen, ke[ok], -1)
    ok2 = n > 1
    np.add.at(multi, kb[ok2], 1)
    np.add.at(multi, ke[ok2], -1)
    return n, np.cumsum(seen)[:lk], np.cumsum(multi)[:lk]


def structural_zero_rows(w):
    """Rows that are zero by structure, as [T, H] booleans (the same for every head):
    query rows that see no key (O, dQ; also LSE = -inf) and key rows that no query
    sees (dK, dV).  Returns (query_rows_out, query_rows_in, key_rows)."""
    q_out = np.zeros(w.total_q_out, dtype=bool)
    q_in = np.zeros(w.total_q, dtype=bool)
    k_rows = np.zeros(w.total_k, dtype=bool)
    for b in range(w.B):
        n, seen, _ = _visible_counts(w, b)
        lq, lk = int(w.lq[b]), int(w.lk[b])
        o0 = b * w.lq_fixed if w.q_off is None else int(w.q_off[b])
        q_out[o0:o0 + lq] = n == 0
        if w.q_off is not None:
            q_in[o0:o0 + lq] = n == 0
        k0 = int(w.kv_off[b])
        k_rows[k0:k0 + lk] = seen == 0
    rep = lambda m: np.repeat(m[:, None], w.H, axis=1)
    return rep(q_out), rep(q_in), rep(k_rows)


def softmax_cancel_rows(w):
    """JFA gradient rows shaped by the softmax identity (each row of dX sums to zero)
    rather than by structure, as [T, H] booleans: a query row with exactly one
    visible key has P = 1 and dP - delta = 0, so dX = 0 and dQ = 0, and a key seen
    only by such rows gets dK = 0 -- the oracle returns exact zeros there, the GPU the
    rounding of dP - delta; a query row with exactly two visible keys has
    dX_i1 = -dX_i0, so dQ_i = scale dX_i0 (k_0 - k_1), whose two roundings match
    rather than add as the noise scale assumes.  Such rows are bounded by their noise
    floor like any other and counted apart.  Returns (dq_rows, dk_rows)."""
    q_in = np.zeros(w.total_q, dtype=bool)
    k_rows = np.zeros(w.total_k, dtype=bool)
    if w.mode == "jfa" and w.q_off is not None:
        for b in range(w.B):
            n, seen, multi = _visible_counts(w, b)
            q0, k0 = int(w.q_off[b]), int(w.kv_off[b])
            q_in[q0:q0 + int(w.lq[b])] = (n == 1) | (n == 2)
            k_rows[k0:k0 + int(w.lk[b])] = (seen > 0) & (multi == 0)
    rep = lambda m: np.repeat(m[:, None], w.H, axis=1)
    return rep(q_in), rep(k_rows)


# Bar for a row below its rounding-noise floor: |error| <= NOISE_BAR times the
# row's noise scale (ref.bwd_noise).  In fp64 emulations of the kernels' roundings
# (bf16 weights normalised by their sum, delta from a 16-bit output, bf16 dX) the
# error stays within 1.8 times that scale over 36,000 causal rows.  The scale
# assumes independent roundings of the terms, so it overestimates rows whose terms
# cancel in pairs (a causal row with two keys: dQ = scale dX_10 (k_0 - k_1), both
# dX rounded alike), which are the rows that fall below the floor.
NOISE_BAR = 2.0
MAX_FLOORED_FRAC = 1e-3


def row_check(got, want, tau, what="", floor_frac=1e-6, zero_rows=None, noise=None, cancel_rows=None):
    """Per-row tolerance: for every row r (all leading dims, last dim = the row),
    max_d |got - want| <= tau * max(max_d |want|, floor_r).  Rows listed in zero_rows
    (zero by structure: no valid pair) must be exactly zero.  floor_r is the row's
    rounding-noise floor NOISE_BAR * noise_r / tau when `noise` (one value per row) is
    given, else floor_frac times the tensor maximum: a row smaller than its floor is
    decided by the roundings of its own terms, and is held to that size instead.
    Such floored rows are counted and must stay within MAX_FLOORED_FRAC of the rows
    (rounded up: a small batch may floor one row), apart from cancel_rows (shaped by
    the softmax identity, see softmax_cancel_rows), which are counted separately.
    Returns a report (rows, worst ratio, floored counts)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if want.size == 0:
        return {"rows": 0, "worst": 0.0, "floored": 0, "cancel": 0}
    g = got.reshape(-1, got.shape[-1])
    r = want.reshape(-1, want.shape[-1])
    assert np.isfinite(g).all(), f"{what}: non-finite values in the GPU result"
    err = np.abs(g - r).max(axis=1)
    ref_max = np.abs(r).max(axis=1)
    zero = np.zeros(len(err), dtype=bool) if zero_rows is None else np.asarray(zero_rows).reshape(-1)
    cancel = np.zeros(len(err), dtype=bool) if cancel_rows is None else np.asarray(cancel_rows).reshape(-1)
    assert not (zero & (ref_max != 0)).any(), f"{what}: oracle row expected zero is not"
    bad_zero = zero & (np.abs(g).max(axis=1) != 0)
    assert not bad_zero.any(), f"{what}: {int(bad_zero.sum())} rows should be exactly zero"
    if noise is not None:
        floor = NOISE_BAR * np.asarray(noise, dtype=np.float64).reshape(-1) / tau
    else:
        floor = np.full(len(err), floor_frac * float(ref_max.max()))
    floor = np.maximum(floor, 1e-300)
    den = np.maximum(ref_max, floor)
    ratio = np.where(zero, 0.0, err / den)
    worst = int(np.argmax(ratio))
    floored = (ref_max < floor) & ~zero
    n_cancel = int((floored & cancel).sum())
    n_floored = int((floored & ~cancel).sum())
    rows = len(ratio)
    print(f"[row-check] {what}: rows {rows}, worst ratio {ratio[worst]:.3e}, floored {n_floored}"
          f" (+{n_cancel} softmax-identity zeros)", flush=True)
    assert ratio[worst] <= tau, (f"{what}: row {worst} err {err[worst]:.3e} ref max "
                                 f"{ref_max[worst]:.3e} floor {floor[worst]:.3e} ratio {ratio[worst]:.3e} > {tau}")
    assert n_floored <= math.ceil(MAX_FLOORED_FRAC * rows), (f"{what}: {n_floored} of {rows} rows below "
                                                             f"their rounding-noise floor")
    return {"rows": rows, "worst": float(ratio[worst]), "floored": n_floored, "cancel": n_cancel}
