"""The opt-in offsets validation (JA_CHECK_OFFSETS=1) and the window clamp, on the GPU.

With the variable set, a device kernel checks the offsets before anything else runs
and the call returns JA_ERR_BAD_OFFSETS when they break the layout rules (start at 0,
never decrease, end at the row counts, key counts within max_kv_len), leaving every
output untouched.  Invalid offsets are only ever passed with the check on: without it
they are undefined behaviour.  A window wider than every sample (up to INT_MAX) keeps
every pair, bit for bit the unwindowed result.
"""
import ctypes

import numpy as np
import pytest
import torch

import recsys_jagged_attention_gdpa_amd as ja
from recsys_jagged_attention_gdpa_amd import _lib, synth
from tests.gpu_helpers import announce, gpu_bwd, gpu_fwd, to_dev

pytestmark = pytest.mark.gpu


def _call_fwd(w, q_off, kv_off, total_q=None, total_k=None, max_kv_len=0):
    """jagged_gdpa_fwd through the C ABI with the given (device) offsets; returns
    (status, o) with o pre-filled with a sentinel."""
    dev = "cuda"
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    prob = _lib.make_problem(batch=w.B, heads=w.H, head_dim=w.D, dtype=w.dtype,
                             total_q=w.total_q if total_q is None else total_q,
                             total_k=w.total_k if total_k is None else total_k,
                             q_offsets=q_off, kv_offsets=kv_off, causal=w.causal, scale=w.scale,
                             act=w.act, max_kv_len=max_kv_len)
    o = torch.full((w.total_q, w.H, w.D), 7.0, dtype=w.dtype, device=dev)
    ws = torch.empty(max(_lib.ja_workspace_size(prob, _lib.PASS_FWD), 256), dtype=torch.uint8, device=dev)
    lib = _lib.load()
    st = lib.jagged_gdpa_fwd(ctypes.byref(prob), _lib._ptr(q), _lib._ptr(k), _lib._ptr(v), _lib._ptr(o),
                             _lib._ptr(ws), _lib._nbytes(ws), _lib._stream(None))
    torch.cuda.synchronize()
    return st, o


def test_bad_offsets_are_caught_before_any_attention_kernel(monkeypatch):
    w = synth.custom(mode="gdpa", lq=[40, 70, 5], lk=[50, 20, 64], H=2, D=64, seed=3, with_dout=False)
    q_off = torch.from_numpy(w.q_off).cuda()
    kv_off = torch.from_numpy(w.kv_off).cuda()
    monkeypatch.setenv("JA_CHECK_OFFSETS", "1")
    announce("offsets check: valid offsets")
    st, o = _call_fwd(w, q_off, kv_off)
    assert st == 0
    monkeypatch.delenv("JA_CHECK_OFFSETS")
    st0, o0 = _call_fwd(w, q_off, kv_off)
    assert st0 == 0 and torch.equal(o, o0)  # the check changes nothing on valid offsets
    monkeypatch.setenv("JA_CHECK_OFFSETS", "1")
    bad = {
        "non-monotone query offsets": (torch.tensor([0, 60, 40, 115], dtype=torch.int32).cuda(), kv_off, {}),
        "query offsets not starting at 0": (torch.tensor([5, 45, 110, 115], dtype=torch.int32).cuda(), kv_off, {}),
        "key offsets not ending at total_k": (q_off, torch.tensor([0, 50, 70, 130], dtype=torch.int32).cuda(), {}),
        "non-monotone key offsets": (q_off, torch.tensor([0, 50, 30, 134], dtype=torch.int32).cuda(), {}),
        "a key count above max_kv_len": (q_off, kv_off, {"max_kv_len": 60}),
    }
    for what, (qo, ko, kw) in bad.items():
        announce(f"offsets check: {what}")
        st, o = _call_fwd(w, qo, ko, **kw)
        assert st == _lib.STATUS_CODES["JA_ERR_BAD_OFFSETS"], (what, st)
        assert (o == 7.0).all(), f"{what}: an output was written"


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
@pytest.mark.parametrize("causal", [False, True])
def test_window_wider_than_everything_is_no_window(mode, causal):
    w = synth.custom(mode=mode, lq=[300, 1, 77, 0, 129], lk=[300, 5, 40, 9, 200], H=2, D=64, seed=11,
                     causal=causal, act="silu")
    d = to_dev(w)
    announce(f"window INT_MAX vs none: {mode} causal={causal}")
    plain_f = gpu_fwd(w, d)
    plain_b = gpu_bwd(w, d, plain_f)
    wide = synth.Workload(**{**w.__dict__, "window": 2**31 - 1})
    wide_f = gpu_fwd(wide, d)
    wide_b = gpu_bwd(wide, d, wide_f)
    torch.cuda.synchronize()
    for n in plain_f:
        if plain_f[n] is not None:
            assert torch.equal(plain_f[n], wide_f[n]), n
    for n in plain_b:
        assert torch.equal(plain_b[n], wide_b[n]), n
