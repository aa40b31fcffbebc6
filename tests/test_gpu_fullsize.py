"""Parity at the workloads' full sizes, in the launch configuration the benchmark
times (the library's own persistent grids over the whole batch).

The GPU runs the whole batch; the oracle recomputes sampled (sample, head)
slices one by one: always the longest sample, plus seeded random ones.  Each
slice is compared row by row with the same bar as the small parity tests.
"""
import time

import numpy as np
import pytest
import torch

from recsys_jagged_attention_gdpa_amd import synth
from tests.gpu_helpers import TAU, announce, check_lse, gpu_bwd, gpu_fwd, np64, to_dev
from tests.helpers import (fp8_pv, fp8_pv_check, oracle_bwd, oracle_fwd, oracle_fwd_fp8_pv, row_check,
                           softmax_cancel_rows, structural_zero_rows)

pytestmark = pytest.mark.gpu


def _single_head(w, b, h):
    """Workload holding only sample b and head h (contiguous copies)."""
    s = w.subset([b])
    pick = lambda t: None if t is None else t[:, h:h + 1, :].contiguous()
    tab = None if s.bias_table is None else s.bias_table[h:h + 1].contiguous()
    scales = None if not s.mx_scales else {n: pick(sc) for n, sc in s.mx_scales.items()}
    return synth.Workload(**{**s.__dict__, "H": 1, "q": pick(s.q), "k": pick(s.k), "v": pick(s.v),
                             "dout": pick(s.dout), "bias_table": tab, "mx_scales": scales})


# (workload, random slices besides the longest sample)
CASES = [("tiny_gdpa_fp32", 2), ("gdpa_xattn_short_kv", 3), ("jfa_causal_self", 3),
         ("pma_gdpa_fwd", 3), ("longtail_gdpa", 2), ("jfa_swa_causal_self", 1),
         ("jfa_rope_causal_self", 1), ("pma_gdpa_fwd_mxfp8", 3), ("gdpa_xattn_short_kv_mxfp8", 3),
         ("jfa_causal_self_fwd_mxfp8", 1)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,n_random", CASES)
def test_full_size_sampled_slices(name, n_random):
    t0 = time.time()
    w = synth.make(name)
    announce(f"full-size {name}: B={w.B} H={w.H} D={w.D} Tq={w.total_q} Tk={w.total_k} "
             f"(generated in {time.time() - t0:.1f}s)")
    d = to_dev(w)
    f = gpu_fwd(w, d)
    g = gpu_bwd(w, d, f) if (w.backward and w.q_off is not None) else None
    torch.cuda.synchronize()
    out = {k: v.detach().cpu() for k, v in f.items() if v is not None}
    if g is not None:
        out.update({k: v.detach().cpu() for k, v in g.items()})
    del d, f, g
    torch.cuda.empty_cache()
    announce(f"full-size {name}: GPU done at {time.time() - t0:.1f}s")

    rng = np.random.default_rng(77)
    lens = w.lq if w.q_off is not None else w.lk
    longest = int(np.argmax(lens * w.lk))
    # the longest sample on two heads, then seeded random (sample, head) slices
    h0 = int(rng.integers(w.H))
    picks = [(longest, h0)] + ([(longest, (h0 + 1 + int(rng.integers(w.H - 1))) % w.H)] if w.H > 1 else [])
    for b in rng.choice(w.B, size=min(n_random, w.B), replace=False):
        picks.append((int(b), int(rng.integers(w.H))))
    tau = TAU[w.dtype]
    for b, h in picks:
        ws = _single_head(w, b, h)
        o0 = b * w.lq_fixed if w.q_off is None else int(w.q_off[b])
        n = int(ws.total_q_out)
        zq_out, zq_in, zk = structural_zero_rows(ws)
        if fp8_pv(ws):  # MXFP8 with P in FP8: the oracle encodes P the same way
            want = oracle_fwd_fp8_pv(ws)
            fp8_pv_check(np64(out["o"][o0:o0 + n, h:h + 1]), want["o"], want["flip"], tau,
                         f"{name} b={b} h={h} O", zero_rows=zq_out)
        else:
            want = oracle_fwd(ws)
            row_check(np64(out["o"][o0:o0 + n, h:h + 1]), want["o"], tau, f"{name} b={b} h={h} O",
                      zero_rows=zq_out)
        if w.mode == "jfa":
            check_lse(np64(out["lse"][h:h + 1, o0:o0 + n]), want["lse"], f"{name} b={b} h={h} LSE")
        if "dq" in out:
            wb = oracle_bwd(ws, noise=True)
            cq, ck = softmax_cancel_rows(ws)
            k0, k1 = int(w.kv_off[b]), int(w.kv_off[b + 1])
            for nm, z, rows, nz, c in (("dq", zq_in, slice(o0, o0 + n), wb["nq"], cq),
                                       ("dk", zk, slice(k0, k1), wb["nk"], ck),
                                       ("dv", zk, slice(k0, k1), None, None)):
                row_check(np64(out[nm][rows, h:h + 1]), wb[nm], tau, f"{name} b={b} h={h} {nm}",
                          zero_rows=z, noise=nz, cancel_rows=c)
        announce(f"full-size {name}: slice b={b} (Lq={int(ws.lq[0])}, Lk={int(ws.lk[0])}) h={h} "
                 f"ok at {time.time() - t0:.1f}s")


@pytest.mark.timeout(900)
def test_full_size_bias_gradient_sampled_entries():
    # The long-tail workload's backward with the bias-table gradient, whole batch,
    # in the library's launch configuration.  The oracle recomputes sampled
    # interior entries one by one (an interior entry is read by one relative
    # position, so it costs one pass over the query rows); each is compared
    # against tau times the largest sampled entry of its head.
    from oracle import ref
    t0 = time.time()
    w = synth.make("longtail_gdpa")
    announce(f"full-size dbias longtail_gdpa: B={w.B} H={w.H} Tq={w.total_q} bias [{w.bias_lo}, {w.bias_hi}]")
    d = to_dev(w)
    import recsys_jagged_attention_gdpa_amd as ja
    g = ja.gdpa_backward(d["q"], d["k"], d["v"], d["dout"], d["q_off"], d["kv_off"], act=w.act,
                         scale=w.scale, causal=w.causal, bias=d["bias"], bias_kind=w.bias_kind,
                         bias_lo=w.bias_lo, bias_hi=w.bias_hi, with_dbias=True)
    torch.cuda.synchronize()
    db = np64(g[3])
    del d, g
    torch.cuda.empty_cache()
    announce(f"full-size dbias: GPU done at {time.time() - t0:.1f}s")
    assert np.isfinite(db).all()
    W = w.bias_hi - w.bias_lo + 1
    rng = np.random.default_rng(5)
    for h in (0, int(rng.integers(1, w.H))):
        positions = [w.bias_lo + 1, -200, -1, 0, 1, 100, w.bias_hi - 1]
        got, want = [], []
        for pos in positions:
            c = pos - w.bias_lo
            assert 0 < c < W - 1
            want.append(ref.gdpa_dbias_entry(w.q, w.k, w.v, w.dout, w.q_off, w.kv_off, scale=w.scale,
                                             act=w.act, causal=w.causal, bias_kind=w.bias_kind,
                                             bias_table=w.bias_table, bias_lo=w.bias_lo,
                                             bias_hi=w.bias_hi, h=h, c=c))
            got.append(db[h, c])
        got, want = np.array(got), np.array(want)
        ratio = np.abs(got - want).max() / np.abs(want).max()
        announce(f"full-size dbias head {h}: entries {positions} worst ratio {ratio:.2e} "
                 f"({time.time() - t0:.1f}s)")
        assert ratio <= TAU[w.dtype], (h, got, want)
