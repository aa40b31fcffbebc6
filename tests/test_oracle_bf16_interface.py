"""Why the JFA forward can return the rounding residual of its bf16 output.

The JFA backward needs delta_i = <dO_i, O_i>.  Formed from the bf16 O alone (as
FlashAttention does), O's rounding moves every dS_ij of a row by P_ij times the
error of delta, however small the true gradient row is.  Evaluated in exact
fp64 arithmetic except for that delta, the backward misses the per-row parity
bar on rows that are small by cancellation; with delta from O + residual (the
bf16 output plus its bf16 rounding residual) it meets the bar.  This is why the
library offers the residual and the parity tests use it.
"""
import numpy as np
import pytest
import torch

from recsys_jagged_attention_gdpa_amd import synth
from tests.helpers import oracle_bwd, row_check


def _bwd_with_delta_from(w, o_view):
    dq = np.zeros((w.total_q, w.H, w.D))
    for b in range(w.B):
        q0, q1 = int(w.q_off[b]), int(w.q_off[b + 1])
        n = q1 - q0
        if n == 0:
            continue
        q, k, v = (t[q0:q1].double().permute(1, 0, 2) for t in (w.q, w.k, w.v))
        do = w.dout[q0:q1].double().permute(1, 0, 2)
        x = (w.scale * q @ k.transpose(-1, -2)).masked_fill(
            ~torch.tril(torch.ones(n, n, dtype=torch.bool)), float("-inf"))
        p = torch.softmax(x, -1)
        delta = (do * o_view(p @ v)).sum(-1, keepdim=True)
        ds = p * (do @ v.transpose(-1, -2) - delta)
        dq[q0:q1] = (w.scale * ds @ k).permute(1, 0, 2).numpy()
    return dq


def _bf16(o):
    return o.float().to(torch.bfloat16).double()


def _bf16_plus_residual(o):
    o32 = o.float()
    hi = o32.to(torch.bfloat16).float()
    return hi.double() + (o32 - hi).to(torch.bfloat16).double()


def test_delta_from_bf16_output_alone_misses_the_bar_and_residual_fixes_it():
    w = synth.make("jfa_causal_self", B=6, max_len=900)
    want = oracle_bwd(w)["dq"]
    with pytest.raises(AssertionError):
        row_check(_bwd_with_delta_from(w, _bf16), want, 2e-2, "delta from bf16 O")
    rep = row_check(_bwd_with_delta_from(w, _bf16_plus_residual), want, 2e-2,
                    "delta from O + residual")
    assert rep["worst"] < 2e-3
