"""The JFA forward that allocates nothing (jagged_attn_fwd_noalloc) against the
forward that takes a workspace (jagged_attn_fwd), through the C ABI.

Both run the same kernels on the same inputs, so their outputs (O, LSE, the O
rounding residual) must be equal bit for bit: on two calls in a row, the second
with a smaller batch (the built-in scratch keeps the first call's contents, which
the planner must overwrite), and again after the workspace forward has run.  A
problem whose forward workspace exceeds the built-in scratch is refused with
JA_ERR_WORKSPACE before anything is launched.
"""
import ctypes

import numpy as np
import pytest
import torch

from recsys_jagged_attention_gdpa_amd import _lib, synth
from tests.gpu_helpers import announce, to_dev

pytestmark = pytest.mark.gpu


def _run(w, noalloc):
    d = to_dev(w)
    prob = _lib.make_problem(batch=w.B, heads=w.H, head_dim=w.D, dtype=w.dtype, total_q=w.total_q,
                             total_k=w.total_k, q_offsets=d["q_off"], kv_offsets=d["kv_off"],
                             causal=w.causal, scale=w.scale, window=w.window)
    o = torch.full((w.total_q, w.H, w.D), 3.0, dtype=w.dtype, device="cuda")
    lse = torch.full((w.H, w.total_q), 3.0, dtype=torch.float32, device="cuda")
    res = torch.full_like(o, 3.0)
    if noalloc:
        _lib.jagged_attn_fwd_noalloc(prob, d["q"], d["k"], d["v"], o, lse, res)
    else:
        ws = torch.empty(_lib.ja_workspace_size(prob, _lib.PASS_FWD), dtype=torch.uint8, device="cuda")
        _lib.jagged_attn_fwd(prob, d["q"], d["k"], d["v"], o, lse, res, ws)
    torch.cuda.synchronize()
    return o, lse, res


def _same(a, b, what):
    for x, y, n in zip(a, b, ("o", "lse", "o_res")):
        assert torch.equal(x, y), f"{what}: {n} differs"


def test_noalloc_forward_matches_workspace_forward_twice():
    big = synth.custom(mode="jfa", lq=[700, 1, 300, 0, 129, 31, 2000], lk=[700, 5, 300, 9, 200, 31, 2000],
                       H=4, D=128, seed=31, causal=True, with_dout=False)
    small = synth.custom(mode="jfa", lq=[40, 130, 3], lk=[12, 130, 64], H=2, D=64, seed=32,
                         with_dout=False)
    announce("noalloc: big batch")
    _same(_run(big, True), _run(big, False), "big batch")
    announce("noalloc: smaller batch next")
    _same(_run(small, True), _run(small, False), "smaller batch")
    announce("noalloc: big batch again after the workspace forward")
    _same(_run(big, True), _run(big, False), "big batch again")


def test_noalloc_forward_refuses_problems_beyond_its_scratch():
    # a batch with one row per sample and a million samples needs unit lists larger
    # than the built-in scratch; nothing may be launched (the pointers are fake)
    B = 1 << 20
    prob = _lib.make_problem(batch=B, heads=1, head_dim=64, dtype=torch.bfloat16, total_q=B, total_k=B,
                             q_offsets=0x1000, kv_offsets=0x2000)
    assert _lib.ja_workspace_size(prob, _lib.PASS_FWD) > _lib.NOALLOC_SCRATCH_BYTES
    lib = _lib.load()
    P = ctypes.c_void_p
    st = lib.jagged_attn_fwd_noalloc(ctypes.byref(prob), P(0x10), P(0x20), P(0x30), P(0x40), P(0x50), None,
                                     None)
    assert st == _lib.STATUS_CODES["JA_ERR_WORKSPACE"]
