"""Shared test helpers: run the oracle on a synthetic workload, compare results."""
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


def oracle_bwd(w, nthreads=0):
    q, k, v = inputs(w)
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


def structural_zero_rows(w):
    """Rows that are zero by structure, as [T, H] booleans (the same for every head):
    query rows that see no key (O, dQ; also LSE = -inf) and key rows that no query
    sees (dK, dV).  Returns (query_rows_out, query_rows_in, key_rows)."""
    lq, lk = w.lq.astype(np.int64), w.lk.astype(np.int64)
    q_out = np.zeros(w.total_q_out, dtype=bool)
    q_in = np.zeros(w.total_q, dtype=bool)
    k_rows = np.zeros(w.total_k, dtype=bool)
    big = np.int64(1) << 40
    win = w.window
    for b in range(w.B):
        # row i sees keys [kb, ke); its aligned position is ia = i + lk - lq
        ia = np.arange(lq[b]) + lk[b] - lq[b]
        ke = np.clip(ia + 1, 0, lk[b]) if w.causal else (np.clip(ia + win, 0, lk[b]) if win else
                                                         np.full(lq[b], lk[b]))
        kb = np.clip(ia - win + 1, 0, None) if win else np.zeros(lq[b], dtype=np.int64)
        n = np.maximum(ke - kb, 0)
        o0 = b * w.lq_fixed if w.q_off is None else int(w.q_off[b])
        q_out[o0:o0 + lq[b]] = n == 0
        if w.q_off is not None:
            q_in[o0:o0 + lq[b]] = n == 0
        # key j is seen by the rows whose aligned position lies in [lo_j, hi_j]
        j = np.arange(lk[b])
        lo_j = j if w.causal else (j - win + 1 if win else j - big)
        hi_j = j + win - 1 if win else j + big
        cnt = np.minimum(hi_j, lk[b] - 1) - np.maximum(lo_j, lk[b] - lq[b]) + 1
        k0 = int(w.kv_off[b])
        k_rows[k0:k0 + lk[b]] = cnt <= 0
    rep = lambda m: np.repeat(m[:, None], w.H, axis=1)
    return rep(q_out), rep(q_in), rep(k_rows)


def softmax_grad_floor(w, name):
    """Absolute error floor for JFA's dQ (name 'dq') and dK ('dk').

    Their elements are sums of P_ij (dP_ij - delta_i) terms, where dP_ij and delta_i
    are fp32 dot products of length D of size up to D max|dO| max|V|.  Rows that
    cancel keep the absolute rounding of that difference: this floor is 16 fp32
    unit roundoffs (2^-20) of its largest possible size, times scale and max|K|
    (dQ) or max|Q| (dK).  With the rotary embedding a turned element can reach
    sqrt(2) times the largest input element, and turning the gradient back mixes
    the errors of a pair (another sqrt(2)): a factor 2."""
    if w.mode != "jfa" or name not in ("dq", "dk") or w.dout is None:
        return 0.0
    other = w.k if name == "dq" else w.q
    mx = lambda t: float(t.float().abs().max()) if t.numel() else 0.0
    turn = 2.0 if w.rope_base else 1.0
    return turn * w.scale * mx(other) * mx(w.dout) * mx(w.v) * w.D * 2.0 ** -20


def row_check(got, want, tau, what="", floor_frac=1e-6, zero_rows=None, abs_floor=0.0):
    """Per-row tolerance: for every row r (all leading dims, last dim = the row),
    max_d |got - want| <= tau * max_d |want|.  Rows listed in zero_rows (zero by
    structure: no valid pair) must be exactly zero.  Rows whose reference maximum is
    below floor_frac times the tensor maximum (including rows that are zero only by
    cancellation) are compared against that floor instead (reported), as are rows
    below abs_floor."""
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
    zero = np.zeros(len(err), dtype=bool) if zero_rows is None else np.asarray(zero_rows).reshape(-1)
    assert not (zero & (ref_max != 0)).any(), f"{what}: oracle row expected zero is not"
    bad_zero = zero & (np.abs(g).max(axis=1) != 0)
    assert not bad_zero.any(), f"{what}: {int(bad_zero.sum())} rows should be exactly zero"
    floor = max(floor_frac * float(ref_max.max()), abs_floor, 1e-300)
    den = np.maximum(ref_max, floor)
    ratio = np.where(zero, 0.0, err / den)
    worst = int(np.argmax(ratio))
    assert ratio[worst] <= tau, (f"{what}: row {worst} err {err[worst]:.3e} ref max "
                                 f"{ref_max[worst]:.3e} ratio {ratio[worst]:.3e} > {tau}")
    return {"rows": len(ratio), "worst": float(ratio[worst]),
            "floored": int(((ref_max < floor) & ~zero).sum())}
