"""Parity of the bias-table gradient (HIP path) with the fp64 oracle.

Bar: per head row of the table gradient, max |gpu - oracle| <= tau * max |oracle|
(tau = 2e-2 for bf16 inputs, 1e-4 for fp32), the same per-row rule as the other
outputs; the gradient is deterministic bit for bit.
"""
import numpy as np
import pytest
import torch

import recsys_jagged_attention_gdpa_amd as ja
from recsys_jagged_attention_gdpa_amd import synth
from tests.gpu_helpers import TAU, announce, gpu_fwd, np64, to_dev
from tests.helpers import oracle_dbias, row_check

pytestmark = pytest.mark.gpu


def gpu_dbias(w, d, fwd=None):
    kw = dict(bias=d["bias"], bias_kind=w.bias_kind, bias_lo=w.bias_lo, bias_hi=w.bias_hi,
              scale=w.scale, causal=w.causal, window=w.window, rope_base=w.rope_base, with_dbias=True)
    if w.mode == "gdpa":
        g = ja.gdpa_backward(d["q"], d["k"], d["v"], d["dout"], d["q_off"], d["kv_off"], act=w.act, **kw)
    else:
        fwd = fwd or gpu_fwd(w, d)
        g = ja.attn_backward(d["q"], d["k"], d["v"], fwd["o"], d["dout"], fwd["lse"], d["q_off"],
                             d["kv_off"], o_residual=fwd.get("o_res"), **kw)
    return g


def check_dbias(w, label):
    announce(f"dbias {label} mode={w.mode} B={w.B} H={w.H} D={w.D} dtype={w.dtype} causal={w.causal} "
             f"bias={w.bias_kind} [{w.bias_lo}, {w.bias_hi}] act={w.act} Tq={w.total_q} Tk={w.total_k}")
    d = to_dev(w)
    g = gpu_dbias(w, d)
    torch.cuda.synchronize()
    want = oracle_dbias(w)
    rep = row_check(np64(g[3]), want, TAU[w.dtype], f"{label} dbias")
    announce(f"dbias {label}: worst row ratio {rep['worst']:.2e} (bar {TAU[w.dtype]})")
    return rep, g


LQ = [1, 70, 300, 0, 129, 5, 40, 200]
LK = [32, 1, 17, 0, 300, 65, 40, 129]


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
@pytest.mark.parametrize("bias,lo,hi", [("rel", -40, 25), ("rel", -400, 400), ("keypos", 0, 63),
                                        ("keypos", 5, 4100)])
@pytest.mark.parametrize("causal", [False, True])
def test_bias_gradient_matches_oracle(mode, bias, lo, hi, causal):
    # Short (<= 32 keys) and long samples, ragged tails, empty samples, entries clamped
    # on both sides, a table wider than every position range, the largest row (4096).
    if hi - lo + 1 > 4096:
        hi = lo + 4095
    w = synth.custom(mode=mode, lq=LQ, lk=LK, H=2, D=128, seed=abs(lo) + hi, act="gelu_erf", causal=causal,
                     bias_kind=bias, bias_lo=lo, bias_hi=hi, bias_sigma=0.3)
    check_dbias(w, f"{mode} {bias} causal={causal}")


@pytest.mark.parametrize("mode,act,D", [("gdpa", "silu", 32), ("gdpa", "gelu_tanh", 64), ("jfa", None, 64),
                                        ("gdpa", "gelu_erf", 128)])
def test_bias_gradient_dims_and_acts(mode, act, D):
    w = synth.custom(mode=mode, lq=[90, 3, 257], lk=[130, 3, 200], H=3, D=D, seed=D, act=act or "silu",
                     causal=False, bias_kind="rel", bias_lo=-100, bias_hi=50)
    check_dbias(w, f"{mode} {act} D={D}")


@pytest.mark.parametrize("bias,lo,hi", [("rel", -1, 0), ("keypos", 3, 4)])
def test_bias_gradient_two_entries(bias, lo, hi):
    # Two entries: every position clamps to one of the two ends.
    w = synth.custom(mode="gdpa", lq=LQ, lk=LK, H=2, D=64, seed=5, act="gelu_tanh", causal=False,
                     bias_kind=bias, bias_lo=lo, bias_hi=hi)
    check_dbias(w, f"two entries {bias}")


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
def test_bias_gradient_fp32(mode):
    w = synth.custom(mode=mode, lq=[9, 0, 23, 1, 17], lk=[9, 5, 23, 1, 0], H=2, D=32, dtype=torch.float32,
                     seed=4, causal=True, bias_kind="rel", bias_lo=-5, bias_hi=7)
    check_dbias(w, f"fp32 {mode}")


def test_bias_gradient_single_entry_and_deterministic():
    # One-entry table: every pair reads it.  Two runs agree bit for bit, and the
    # other outputs equal those of the backward without the gradient.
    w = synth.custom(mode="gdpa", lq=LQ, lk=LK, H=2, D=64, seed=3, act="silu", causal=True,
                     bias_kind="rel", bias_lo=0, bias_hi=0)
    _, g1 = check_dbias(w, "one entry")
    d = to_dev(w)
    from tests.gpu_helpers import gpu_bwd
    g2 = ja.gdpa_backward(d["q"], d["k"], d["v"], d["dout"], d["q_off"], d["kv_off"], act=w.act,
                          scale=w.scale, causal=True, bias=d["bias"], bias_kind="rel", bias_lo=0,
                          bias_hi=0, with_dbias=True)
    plain = gpu_bwd(w, d)
    torch.cuda.synchronize()
    assert torch.equal(g1[3], g2[3])
    for n, i in (("dq", 0), ("dk", 1), ("dv", 2)):
        assert torch.equal(g2[i], plain[n]), n


def test_jfa_bias_gradient_sums_to_zero_at_scale():
    # Softmax rows: each head's table gradient sums to zero (to rounding), at a
    # size well past the oracle's reach.
    w = synth.custom(mode="jfa", lq=[3000, 17, 1500, 700], H=4, D=128, seed=8, causal=True,
                     bias_kind="rel", bias_lo=-512, bias_hi=512, with_dout=True)
    announce(f"dbias zero-sum JFA Tq={w.total_q}")
    d = to_dev(w)
    g = gpu_dbias(w, d)
    db = np64(g[3])
    assert np.isfinite(db).all()
    mag = np.abs(db).sum(axis=1)
    assert (np.abs(db.sum(axis=1)) <= 1e-3 * mag).all(), (db.sum(axis=1), mag)


def test_autograd_bias_gradient():
    w = synth.custom(mode="jfa", lq=[40, 7, 130], lk=[33, 7, 100], H=2, D=64, seed=6, causal=True,
                     bias_kind="keypos", bias_lo=0, bias_hi=90)
    announce("dbias autograd")
    d = to_dev(w)
    table = d["bias"].clone().requires_grad_(True)
    o = ja.jagged_attention(d["q"], d["k"], d["v"], d["q_off"], d["kv_off"], scale=w.scale, causal=True,
                            bias=table, bias_kind="keypos", bias_lo=0, bias_hi=90)
    o.backward(d["dout"])
    row_check(np64(table.grad), oracle_dbias(w), TAU[w.dtype], "autograd dbias")


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
def test_bias_gradient_bitwise_run_to_run_with_many_samples(mode):
    # 320 samples, many sharing a cost (lengths from a small set): the planner must
    # place equal-cost samples in a fixed order, since the table gradient's fp32
    # summation order follows the unit list.  Several calls, bitwise equal.
    rng = np.random.default_rng(21)
    lens = rng.choice([17, 64, 100, 130, 257], size=320).tolist()
    w = synth.custom(mode=mode, lq=lens, lk=lens, H=2, D=64, seed=8, act="gelu_erf", causal=mode == "jfa",
                     bias_kind="rel", bias_lo=-128, bias_hi=128)
    d = to_dev(w)
    announce(f"dbias determinism {mode}: B={w.B} Tq={w.total_q}")
    runs = [gpu_dbias(w, d)[3].clone() for _ in range(4)]
    torch.cuda.synchronize()
    for r in runs[1:]:
        assert torch.equal(runs[0], r)
