"""ctypes binding of libjagged_attn.so (include/jagged_attn.h).

The functions named like the C entry points only marshal arguments: tensors
become device pointers, the problem becomes a ``JaProblem`` struct and the
stream is torch's current stream.  Every step of the computation runs in the
library's HIP kernels; if the library is missing this module raises instead of
falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
import threading
import warnings

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libjagged_attn.so")

JA_OK = 0
STATUS = {0: "JA_OK", 1: "JA_ERR_NULL", 2: "JA_ERR_SHAPE", 3: "JA_ERR_UNSUPPORTED",
          4: "JA_ERR_WORKSPACE", 5: "JA_ERR_BAD_OFFSETS", 6: "JA_ERR_HIP"}
STATUS_CODES = {v: k for k, v in STATUS.items()}
DTYPES = {torch.bfloat16: 0, torch.float32: 1}
ACTS = {"silu": 0, "gelu_tanh": 1, "gelu_erf": 2}
BIAS = {"none": 0, "rel": 1, "keypos": 2}
PASS_FWD, PASS_BWD, PASS_BWD_DBIAS = 0, 1, 2

EXPORTS = ("ja_workspace_size", "jagged_gdpa_fwd", "jagged_gdpa_bwd", "jagged_attn_fwd",
           "jagged_attn_bwd", "jagged_gdpa_fwd_mx", "jagged_attn_fwd_mx", "jagged_attn_fwd_noalloc",
           "jagged_rope", "ja_profile_kernel", "ja_profile_busy", "ja_status_string", "ja_last_hip_error", "ja_version")
NOALLOC_SCRATCH_BYTES = 4 << 20  # JA_NOALLOC_SCRATCH_BYTES
KERNELS = {"plan": 0, "fwd": 1, "bwd_fused": 2, "bwd_kv": 3, "bwd_q": 4, "bwd_delta": 5,
           "fwd_short": 6, "bwd_dbias": 7, "rope": 8, "rope_back": 9, "check_offsets": 10}


class JaProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("total_q", ctypes.c_int64), ("total_k", ctypes.c_int64),
        ("q_offsets", ctypes.c_void_p), ("lq_fixed", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("kv_offsets", ctypes.c_void_p), ("scale", ctypes.c_float), ("act", ctypes.c_int32),
        ("bias_kind", ctypes.c_int32), ("bias_lo", ctypes.c_int32), ("bias_hi", ctypes.c_int32),
        ("bias_table", ctypes.c_void_p), ("max_kv_len", ctypes.c_int32), ("window", ctypes.c_int32),
        ("rope_base", ctypes.c_float), ("rope_inputs_turned", ctypes.c_int32),
    ]


class JaError(RuntimeError):
    def __init__(self, fn, status, lib):
        self.status = status
        msg = lib.ja_status_string(status).decode()
        extra = f" (hip error {lib.ja_last_hip_error()})" if status == 6 else ""
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}{extra}")


_lib = None
_lock = threading.Lock()


def stale_reason(path: str = LIB_PATH):
    """Why the library at `path` may not match the sources next to it (None when
    its build stamp, written by build.py, equals the current sources' digest)."""
    from . import build as _build
    stamp = path + ".sources"
    if not os.path.exists(stamp):
        return f"{stamp} is missing (library built without a source stamp)"
    with open(stamp) as fh:
        built = fh.read().strip()
    if built != _build.sources_digest():
        return "the C/HIP sources or compiler options changed since the library was built"
    return None


def load(path: str = LIB_PATH):
    """Load the shared library (once).  Raises if it has not been built; warns
    when it was built from other sources than the ones in the tree."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m recsys_jagged_attention_gdpa_amd.build`")
        why = stale_reason(path)
        if why is not None:
            warnings.warn(f"{path}: {why}; rebuild with `python -m recsys_jagged_attention_gdpa_amd.build`",
                          RuntimeWarning, stacklevel=2)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        PP = ctypes.POINTER(JaProblem)
        lib.ja_workspace_size.argtypes = [PP, ctypes.c_int]
        lib.ja_workspace_size.restype = ctypes.c_size_t
        lib.jagged_gdpa_fwd.argtypes = [PP, P, P, P, P, P, ctypes.c_size_t, P]
        lib.jagged_attn_fwd.argtypes = [PP, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.jagged_gdpa_bwd.argtypes = [PP, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.jagged_attn_bwd.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.jagged_gdpa_fwd_mx.argtypes = [PP, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.jagged_attn_fwd_mx.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        lib.jagged_attn_fwd_noalloc.argtypes = [PP, P, P, P, P, P, P, P]
        lib.jagged_rope.argtypes = [PP, P, P, P, P, P]
        for f in (lib.jagged_gdpa_fwd, lib.jagged_attn_fwd, lib.jagged_gdpa_bwd, lib.jagged_attn_bwd,
                  lib.jagged_gdpa_fwd_mx, lib.jagged_attn_fwd_mx, lib.jagged_attn_fwd_noalloc,
                  lib.jagged_rope):
            f.restype = ctypes.c_int
        lib.ja_profile_kernel.argtypes = [ctypes.c_int, P, P]
        lib.ja_profile_kernel.restype = ctypes.c_int
        lib.ja_profile_busy.argtypes = [ctypes.c_int, P, ctypes.c_int]
        lib.ja_profile_busy.restype = ctypes.c_int
        lib.ja_status_string.argtypes = [ctypes.c_int]
        lib.ja_status_string.restype = ctypes.c_char_p
        lib.ja_last_hip_error.argtypes = []
        lib.ja_last_hip_error.restype = ctypes.c_int
        lib.ja_version.argtypes = []
        lib.ja_version.restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(stream)


def make_problem(*, batch, heads, head_dim, dtype, total_q, total_k, q_offsets, kv_offsets,
                 lq_fixed=0, causal=False, scale=None, act="silu", bias_kind="none",
                 bias_table=None, bias_lo=0, bias_hi=0, max_kv_len=0, window=0,
                 rope_base=0.0, rope_inputs_turned=False) -> JaProblem:
    """Fill a JaProblem.  Offsets and the bias table are device tensors (or raw pointers)."""
    p = JaProblem()
    p.batch, p.heads, p.head_dim = int(batch), int(heads), int(head_dim)
    p.dtype = DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    p.total_q, p.total_k = int(total_q), int(total_k)
    p.q_offsets = _ptr(q_offsets)
    p.lq_fixed = int(lq_fixed)
    p.causal = int(bool(causal))
    p.kv_offsets = _ptr(kv_offsets)
    p.scale = float(head_dim ** -0.5 if scale is None else scale)
    p.act = ACTS[act] if isinstance(act, str) else int(act)
    p.bias_kind = BIAS[bias_kind] if isinstance(bias_kind, str) else int(bias_kind)
    p.bias_lo, p.bias_hi = int(bias_lo), int(bias_hi)
    p.bias_table = _ptr(bias_table)
    p.max_kv_len = int(max_kv_len)
    p.window = int(window)
    p.rope_base = float(rope_base)
    p.rope_inputs_turned = int(bool(rope_inputs_turned))
    return p


def _check(fn, status):
    if status != JA_OK:
        raise JaError(fn, status, load())


# ---- same-name wrappers of the C entry points (argument marshalling only) ----
def ja_workspace_size(problem: JaProblem, pass_: int) -> int:
    return int(load().ja_workspace_size(ctypes.byref(problem), int(pass_)))


def jagged_gdpa_fwd(problem, q, k, v, o, workspace, stream=None):
    _check("jagged_gdpa_fwd", load().jagged_gdpa_fwd(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(workspace),
        _nbytes(workspace), _stream(stream)))


def jagged_attn_fwd_noalloc(problem, q, k, v, o, lse, o_residual, stream=None):
    _check("jagged_attn_fwd_noalloc", load().jagged_attn_fwd_noalloc(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(o_residual),
        _stream(stream)))


def jagged_rope(problem, q, k, q_turned, k_turned, stream=None):
    _check("jagged_rope", load().jagged_rope(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(q_turned), _ptr(k_turned), _stream(stream)))


def jagged_attn_fwd(problem, q, k, v, o, lse, o_residual, workspace, stream=None):
    _check("jagged_attn_fwd", load().jagged_attn_fwd(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(o_residual),
        _ptr(workspace), _nbytes(workspace), _stream(stream)))


def jagged_gdpa_bwd(problem, q, k, v, dout, dq, dk, dv, dbias, workspace, stream=None):
    _check("jagged_gdpa_bwd", load().jagged_gdpa_bwd(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(dbias), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def jagged_attn_bwd(problem, q, k, v, o, o_residual, dout, lse, dq, dk, dv, dbias, workspace,
                    stream=None):
    _check("jagged_attn_bwd", load().jagged_attn_bwd(
        ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(o_residual), _ptr(dout),
        _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dbias), _ptr(workspace), _nbytes(workspace),
        _stream(stream)))


def jagged_gdpa_fwd_mx(problem, q, q_scale, k, k_scale, v, v_scale, o, workspace, stream=None):
    _check("jagged_gdpa_fwd_mx", load().jagged_gdpa_fwd_mx(
        ctypes.byref(problem), _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(v), _ptr(v_scale),
        _ptr(o), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def jagged_attn_fwd_mx(problem, q, q_scale, k, k_scale, v, v_scale, o, lse, o_residual, workspace,
                       stream=None):
    _check("jagged_attn_fwd_mx", load().jagged_attn_fwd_mx(
        ctypes.byref(problem), _ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(v), _ptr(v_scale),
        _ptr(o), _ptr(lse), _ptr(o_residual), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def ja_profile_kernel(kernel, start_event, stop_event):
    """Record raw hipEvent_t handles around `kernel` ("fwd", "bwd_fused", ...) in later calls
    on this thread (each kernel has its own pair); pass None, None to stop for that kernel."""
    kid = KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    _check("ja_profile_kernel", load().ja_profile_kernel(kid, start_event, stop_event))


def ja_profile_busy(kernel, buffer):
    """Have every workgroup of `kernel` write its busy cycles into the int64 device tensor
    `buffer` (one entry per workgroup) in later calls on this thread; None to stop."""
    kid = KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    cap = 0 if buffer is None else buffer.numel()
    _check("ja_profile_busy", load().ja_profile_busy(kid, _ptr(buffer), cap))


def _nbytes(t):
    if t is None:
        return 0
    if isinstance(t, torch.Tensor):
        return t.numel() * t.element_size()
    raise TypeError("workspace must be a torch tensor")
