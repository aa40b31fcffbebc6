"""ctypes shim over the fp64 oracle in ``ref.c`` — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this module.  It shares no code with the GPU library and never
imports the product package.

Arrays are numpy (torch CPU tensors are accepted and converted).  Inputs are
read as float32 (bf16 values convert exactly), outputs are float64 in the same
token-major layout ``[T, H, D]``; JFA's log-sum-exp is ``[T, H]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ref.c")
_LIB = os.path.join(_HERE, "libjagged_ref.so")

ACTS = {"silu": 0, "gelu_tanh": 1, "gelu_erf": 2}
BIAS = {"none": 0, "rel": 1, "keypos": 2}

_lib = None


def build(force: bool = False) -> str:
    """Compile ref.c with gcc (-O2, OpenMP, no fast-math) into libjagged_ref.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-D_DEFAULT_SOURCE", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        # ... scale, [act,] causal, window, rope_base, bias_kind, table, lo, hi, [h, c,] nthreads
        lib.ref_gdpa_fwd.argtypes = [P, P, P, P, P, ctypes.c_int32, P, I, I, I, D, I, I, I, D, I, P, I,
                                     I, I]
        lib.ref_attn_fwd.argtypes = [P, P, P, P, P, P, ctypes.c_int32, P, I, I, I, D, I, I, D, I, P, I,
                                     I, I]
        lib.ref_gdpa_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, D, I, I, I, D, I, P, I, I, I]
        lib.ref_attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, D, I, I, D, I, P, I, I, I]
        lib.ref_gdpa_dbias.argtypes = [P, P, P, P, P, P, P, I, I, I, D, I, I, I, D, I, P, I, I, I]
        lib.ref_attn_dbias.argtypes = [P, P, P, P, P, P, P, I, I, I, D, I, I, D, I, P, I, I, I]
        lib.ref_gdpa_dbias_entry.argtypes = [P, P, P, P, P, P, P, I, I, I, D, I, I, I, D, I, P, I, I,
                                             I, I, I]
        lib.ref_bwd_noise.argtypes = [I, P, P, P, P, P, P, P, P, P, P, P, I, I, I, D, I, I, I, D, I, P,
                                      I, I, D, D, I]
        lib.ref_bwd_noise.restype = ctypes.c_int
        lib.ref_act.argtypes = [I, P, P, P, ctypes.c_int64]
        lib.ref_rope.argtypes = [P, P, P, I, ctypes.c_int64, I, I, D]
        lib.ref_rope.restype = ctypes.c_int
        lib.ref_max_threads.argtypes = []
        for f in (lib.ref_gdpa_fwd, lib.ref_attn_fwd, lib.ref_gdpa_bwd, lib.ref_attn_bwd,
                  lib.ref_gdpa_dbias, lib.ref_attn_dbias, lib.ref_gdpa_dbias_entry,
                  lib.ref_max_threads):
            f.restype = ctypes.c_int
        lib.ref_act.restype = None
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().ref_max_threads())


def _f32(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _i32(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a):
    return None if a is None else a.ctypes.data


def _rope_arg(base, bf16):
    """The C side's rope_base: the base, negated when the turned rows are rounded to bf16."""
    base = float(base)
    assert base >= 0.0
    return -base if (bf16 and base > 0.0) else base


class _Args:
    def __init__(self, q, k, v, q_off, kv_off, lq_fixed, bias_kind, bias_table, bias_lo, bias_hi):
        self.q, self.k, self.v = _f32(q), _f32(k), _f32(v)
        self.q_off, self.kv_off = _i32(q_off), _i32(kv_off)
        assert self.q.ndim == 3 and self.k.shape == self.v.shape and self.k.ndim == 3
        self.H, self.D = self.q.shape[1], self.q.shape[2]
        assert self.k.shape[1:] == (self.H, self.D)
        self.B = len(self.kv_off) - 1
        if self.q_off is None:
            self.lq_fixed = int(lq_fixed if lq_fixed else self.q.shape[0])
            assert self.q.shape[0] == self.lq_fixed
            self.t_out = self.B * self.lq_fixed
        else:
            assert len(self.q_off) == self.B + 1 and self.q_off[-1] == self.q.shape[0]
            self.lq_fixed = 0
            self.t_out = self.q.shape[0]
        assert self.kv_off[-1] == self.k.shape[0]
        self.bias_kind = BIAS[bias_kind]
        self.bias_table = _f32(bias_table) if self.bias_kind else None
        if self.bias_kind:
            assert self.bias_table.shape == (self.H, bias_hi - bias_lo + 1)
        self.bias_lo, self.bias_hi = int(bias_lo), int(bias_hi)


def gdpa_fwd(q, k, v, q_off, kv_off, *, scale, act, lq_fixed=0, causal=False, window=0,
             rope_base=0.0, rope_bf16=False, bias_kind="none", bias_table=None, bias_lo=0, bias_hi=0,
             nthreads=0):
    """GDPA forward: O_i = sum_j act(scale q_i.k_j + bias_ij) v_j over valid j (q, k turned
    by the rotary embedding first when rope_base > 0)."""
    a = _Args(q, k, v, q_off, kv_off, lq_fixed, bias_kind, bias_table, bias_lo, bias_hi)
    o = np.empty((a.t_out, a.H, a.D), dtype=np.float64)
    rc = _load().ref_gdpa_fwd(_ptr(a.q), _ptr(a.k), _ptr(a.v), _ptr(o), _ptr(a.q_off), a.lq_fixed,
                              _ptr(a.kv_off), a.B, a.H, a.D, float(scale), ACTS[act], int(causal),
                              int(window), _rope_arg(rope_base, rope_bf16), a.bias_kind,
                              _ptr(a.bias_table),
                              a.bias_lo, a.bias_hi, int(nthreads))
    assert rc == 0
    return o


def attn_fwd(q, k, v, q_off, kv_off, *, scale, lq_fixed=0, causal=False, window=0,
             rope_base=0.0, rope_bf16=False, bias_kind="none", bias_table=None, bias_lo=0, bias_hi=0,
             nthreads=0):
    """JFA forward: row softmax over valid keys; returns (O, LSE[T, H])."""
    a = _Args(q, k, v, q_off, kv_off, lq_fixed, bias_kind, bias_table, bias_lo, bias_hi)
    o = np.empty((a.t_out, a.H, a.D), dtype=np.float64)
    lse = np.empty((a.t_out, a.H), dtype=np.float64)
    rc = _load().ref_attn_fwd(_ptr(a.q), _ptr(a.k), _ptr(a.v), _ptr(o), _ptr(lse), _ptr(a.q_off),
                              a.lq_fixed, _ptr(a.kv_off), a.B, a.H, a.D, float(scale), int(causal),
                              int(window), _rope_arg(rope_base, rope_bf16), a.bias_kind,
                              _ptr(a.bias_table),
                              a.bias_lo, a.bias_hi, int(nthreads))
    assert rc == 0
    return o, lse


def _bwd(fn, with_act, q, k, v, dout, q_off, kv_off, scale, act, causal, window, rope_base,
         rope_bf16, bias_kind, bias_table, bias_lo, bias_hi, nthreads):
    assert q_off is not None, "backward of a shared query block is not part of the oracle"
    a = _Args(q, k, v, q_off, kv_off, 0, bias_kind, bias_table, bias_lo, bias_hi)
    do = _f32(dout)
    assert do.shape == a.q.shape
    dq = np.empty(a.q.shape, dtype=np.float64)
    dk = np.empty(a.k.shape, dtype=np.float64)
    dv = np.empty(a.v.shape, dtype=np.float64)
    args = [_ptr(a.q), _ptr(a.k), _ptr(a.v), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(a.q_off),
            _ptr(a.kv_off), a.B, a.H, a.D, float(scale)]
    if with_act:
        args.append(ACTS[act])
    args += [int(causal), int(window), _rope_arg(rope_base, rope_bf16), a.bias_kind,
             _ptr(a.bias_table),
             a.bias_lo, a.bias_hi, int(nthreads)]
    rc = fn(*args)
    assert rc == 0, rc
    return dq, dk, dv


def gdpa_bwd(q, k, v, dout, q_off, kv_off, *, scale, act, causal=False, window=0,
             rope_base=0.0, rope_bf16=False,
             bias_kind="none", bias_table=None, bias_lo=0, bias_hi=0, nthreads=0):
    """GDPA backward of L = <O, dout>: returns (dQ, dK, dV) in float64."""
    return _bwd(_load().ref_gdpa_bwd, True, q, k, v, dout, q_off, kv_off, scale, act, causal, window,
                rope_base, rope_bf16, bias_kind, bias_table, bias_lo, bias_hi, nthreads)


def attn_bwd(q, k, v, dout, q_off, kv_off, *, scale, causal=False, window=0,
             rope_base=0.0, rope_bf16=False,
             bias_kind="none", bias_table=None, bias_lo=0, bias_hi=0, nthreads=0):
    """JFA backward of L = <O, dout>: returns (dQ, dK, dV) in float64."""
    return _bwd(_load().ref_attn_bwd, False, q, k, v, dout, q_off, kv_off, scale, None, causal, window,
                rope_base, rope_bf16, bias_kind, bias_table, bias_lo, bias_hi, nthreads)


def bwd_noise(mode, q, k, v, dout, q_off, kv_off, *, scale, act="silu", causal=False, window=0,
              rope_base=0.0, rope_bf16=False, bias_kind="none", bias_table=None, bias_lo=0,
              bias_hi=0, dx_unit=2.0 ** -8, delta_unit=2.0 ** -16, nthreads=0):
    """Backward (mode 'gdpa' or 'jfa') plus the rounding-noise scale of every dQ row
    (nq [total_q, H]) and dK row (nk [total_k, H]): dx_unit max_d sqrt(sum_j t_jd^2)
    over the terms t_jd = scale dX_ij k_jd (dK: over i, with q_id) of the row's sum,
    the error that sum carries when each dX is rounded to a unit roundoff of
    dx_unit, plus (JFA) the error from delta formed with relative error
    delta_unit.  Returns (dQ, dK, dV, nq, nk)."""
    assert q_off is not None
    a = _Args(q, k, v, q_off, kv_off, 0, bias_kind, bias_table, bias_lo, bias_hi)
    do = _f32(dout)
    assert do.shape == a.q.shape
    dq = np.empty(a.q.shape, dtype=np.float64)
    dk = np.empty(a.k.shape, dtype=np.float64)
    dv = np.empty(a.v.shape, dtype=np.float64)
    nq = np.empty(a.q.shape[:2], dtype=np.float64)
    nk = np.empty(a.k.shape[:2], dtype=np.float64)
    rc = _load().ref_bwd_noise(int(mode == "jfa"), _ptr(a.q), _ptr(a.k), _ptr(a.v), _ptr(do), _ptr(dq),
                               _ptr(dk), _ptr(dv), _ptr(nq), _ptr(nk), _ptr(a.q_off), _ptr(a.kv_off),
                               a.B, a.H, a.D, float(scale), ACTS[act or "silu"], int(causal), int(window),
                               _rope_arg(rope_base, rope_bf16), a.bias_kind, _ptr(a.bias_table),
                               a.bias_lo, a.bias_hi, float(dx_unit), float(delta_unit), int(nthreads))
    assert rc == 0, rc
    return dq, dk, dv, nq, nk


def _dbias(fn, with_act, q, k, v, dout, q_off, kv_off, scale, act, causal, window, rope_base,
           rope_bf16, bias_kind, bias_table, bias_lo, bias_hi, nthreads):
    assert q_off is not None and bias_kind != "none"
    a = _Args(q, k, v, q_off, kv_off, 0, bias_kind, bias_table, bias_lo, bias_hi)
    do = _f32(dout)
    assert do.shape == a.q.shape
    dt = np.empty((a.H, a.bias_hi - a.bias_lo + 1), dtype=np.float64)
    args = [_ptr(a.q), _ptr(a.k), _ptr(a.v), _ptr(do), _ptr(dt), _ptr(a.q_off), _ptr(a.kv_off),
            a.B, a.H, a.D, float(scale)]
    if with_act:
        args.append(ACTS[act])
    args += [int(causal), int(window), _rope_arg(rope_base, rope_bf16), a.bias_kind,
             _ptr(a.bias_table),
             a.bias_lo, a.bias_hi, int(nthreads)]
    rc = fn(*args)
    assert rc == 0, rc
    return dt


def gdpa_dbias(q, k, v, dout, q_off, kv_off, *, scale, act, causal=False, window=0,
               rope_base=0.0, rope_bf16=False,
               bias_kind, bias_table, bias_lo, bias_hi, nthreads=0):
    """GDPA: dL/dtable [H, hi - lo + 1] of L = <O, dout> (float64)."""
    return _dbias(_load().ref_gdpa_dbias, True, q, k, v, dout, q_off, kv_off, scale, act, causal,
                  window, rope_base, rope_bf16, bias_kind, bias_table, bias_lo, bias_hi, nthreads)


def attn_dbias(q, k, v, dout, q_off, kv_off, *, scale, causal=False, window=0,
               rope_base=0.0, rope_bf16=False,
               bias_kind, bias_table, bias_lo, bias_hi, nthreads=0):
    """JFA: dL/dtable [H, hi - lo + 1] of L = <O, dout> (float64)."""
    return _dbias(_load().ref_attn_dbias, False, q, k, v, dout, q_off, kv_off, scale, None, causal,
                  window, rope_base, rope_bf16, bias_kind, bias_table, bias_lo, bias_hi, nthreads)


def gdpa_dbias_entry(q, k, v, dout, q_off, kv_off, *, scale, act, causal=False, window=0,
                     rope_base=0.0, rope_bf16=False, bias_kind, bias_table, bias_lo, bias_hi, h, c, nthreads=0):
    """One entry (head h, index c) of the GDPA table gradient, in float64."""
    a = _Args(q, k, v, q_off, kv_off, 0, bias_kind, bias_table, bias_lo, bias_hi)
    do = _f32(dout)
    out = np.zeros(1, dtype=np.float64)
    rc = _load().ref_gdpa_dbias_entry(_ptr(a.q), _ptr(a.k), _ptr(a.v), _ptr(do), _ptr(out),
                                      _ptr(a.q_off), _ptr(a.kv_off), a.B, a.H, a.D, float(scale),
                                      ACTS[act], int(causal), int(window),
                                      _rope_arg(rope_base, rope_bf16),
                                      a.bias_kind,
                                      _ptr(a.bias_table),
                                      a.bias_lo, a.bias_hi, int(h), int(c), int(nthreads))
    assert rc == 0, rc
    return float(out[0])


def rope(x, off, *, rope_base, rope_bf16=False):
    """The rotary turn of a [rows, H, D] tensor by sample-local positions (off: int32
    [B+1], or None for one block whose row r sits at position r), in float64; with
    rope_bf16 each turned element rounded to the nearest bf16 value (ties to even)."""
    x = _f32(x)
    o = _i32(off)
    y = np.empty(x.shape, dtype=np.float64)
    B = 1 if o is None else len(o) - 1
    rc = _load().ref_rope(_ptr(x), _ptr(y), _ptr(o), B, x.shape[0], x.shape[1], x.shape[2],
                          _rope_arg(rope_base, rope_bf16))
    assert rc == 0, rc
    return y


def act(name, x):
    """Activation and its derivative, element-wise, in float64."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    y = np.empty_like(x)
    dy = np.empty_like(x)
    _load().ref_act(ACTS[name], _ptr(x), _ptr(y), _ptr(dy), x.size)
    return y, dy
