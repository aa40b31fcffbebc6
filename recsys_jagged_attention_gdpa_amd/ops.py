"""Tensor-level API over the C ABI: allocate outputs and workspace with torch,
call the library, and expose autograd functions.

    o = gdpa(q, k, v, q_offsets, kv_offsets, act="gelu_tanh")
    o = jagged_attention(q, k, v, q_offsets, kv_offsets, causal=True)

q is [Tq, H, D] (or [Lq, H, D] shared by every sample when q_offsets is None),
k and v are [Tk, H, D]; offsets are int32 [B+1] on the same device.
max_kv_len (0 = unknown) is an optional upper bound on every sample's key
count; a bound of at most 32 lets the library skip its long-sequence kernels.
window (0 = none) keeps the pairs whose aligned distance i + Lk - Lq - j is
below it (and, without causal masking, above minus it): sliding-window
attention.  rope_base (0 = none) turns q and k by the rotary embedding of
their sample-local positions before the scores are formed; gradients are with
respect to the rows as given.  rope() turns q and k once; pass its output with
rope_inputs_turned=True to a forward and its backward (the autograd functions
do so), which then turn nothing on the way in.
"""
from __future__ import annotations

import torch

from . import _lib


def _problem(q, k, q_offsets, kv_offsets, *, causal, scale, act, bias, bias_kind, bias_lo,
             bias_hi, max_kv_len=0, window=0, rope_base=0.0, rope_inputs_turned=False):
    B = int(kv_offsets.numel()) - 1
    H, D = int(q.shape[1]), int(q.shape[2])
    return _lib.make_problem(
        batch=B, heads=H, head_dim=D, dtype=q.dtype, total_q=int(q.shape[0]),
        total_k=int(k.shape[0]), q_offsets=q_offsets, kv_offsets=kv_offsets,
        lq_fixed=0 if q_offsets is not None else int(q.shape[0]), causal=causal, scale=scale,
        act=act, bias_kind=bias_kind if bias is not None else "none", bias_table=bias,
        bias_lo=bias_lo, bias_hi=bias_hi, max_kv_len=max_kv_len, window=window, rope_base=rope_base,
        rope_inputs_turned=rope_inputs_turned)


def _check_inputs(q, k, v, q_offsets, kv_offsets, bias):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous 3-D device tensor")
    if k.shape != v.shape or k.shape[1:] != q.shape[1:] or q.dtype != k.dtype or k.dtype != v.dtype:
        raise ValueError("q, k, v shapes / dtypes disagree")
    for name, t in (("q_offsets", q_offsets), ("kv_offsets", kv_offsets)):
        if t is not None and (t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    if bias is not None and (bias.dtype != torch.float32 or not bias.is_cuda or not bias.is_contiguous()):
        raise ValueError("bias table must be a contiguous float32 device tensor")


def _workspace(problem, pass_, device):
    n = _lib.ja_workspace_size(problem, pass_)
    if n == 0:
        raise ValueError("invalid problem (ja_workspace_size returned 0)")
    return torch.empty(n, dtype=torch.uint8, device=device)


def gdpa_forward(q, k, v, q_offsets, kv_offsets, *, act="silu", scale=None, causal=False,
                 bias=None, bias_kind="none", bias_lo=0, bias_hi=0, max_kv_len=0, window=0,
                 rope_base=0.0, rope_inputs_turned=False):
    _check_inputs(q, k, v, q_offsets, kv_offsets, bias)
    p = _problem(q, k, q_offsets, kv_offsets, causal=causal, scale=scale, act=act, bias=bias,
                 bias_kind=bias_kind, bias_lo=bias_lo, bias_hi=bias_hi, max_kv_len=max_kv_len,
                 window=window, rope_base=rope_base, rope_inputs_turned=rope_inputs_turned)
    rows = q.shape[0] if q_offsets is not None else p.batch * q.shape[0]
    o = torch.empty((rows, q.shape[1], q.shape[2]), dtype=q.dtype, device=q.device)
    ws = _workspace(p, _lib.PASS_FWD, q.device)
    _lib.jagged_gdpa_fwd(p, q, k, v, o, ws)
    return o


def attn_forward(q, k, v, q_offsets, kv_offsets, *, scale=None, causal=False, bias=None,
                 bias_kind="none", bias_lo=0, bias_hi=0, residual=True, max_kv_len=0, window=0,
                 rope_base=0.0, rope_inputs_turned=False):
    """Returns (O, LSE[H, T], O_residual); O_residual is None for fp32 or residual=False."""
    _check_inputs(q, k, v, q_offsets, kv_offsets, bias)
    p = _problem(q, k, q_offsets, kv_offsets, causal=causal, scale=scale, act="silu", bias=bias,
                 bias_kind=bias_kind, bias_lo=bias_lo, bias_hi=bias_hi, max_kv_len=max_kv_len,
                 window=window, rope_base=rope_base, rope_inputs_turned=rope_inputs_turned)
    rows = q.shape[0] if q_offsets is not None else p.batch * q.shape[0]
    o = torch.empty((rows, q.shape[1], q.shape[2]), dtype=q.dtype, device=q.device)
    lse = torch.empty((q.shape[1], rows), dtype=torch.float32, device=q.device)
    o_res = torch.empty_like(o) if (residual and q.dtype == torch.bfloat16) else None
    ws = _workspace(p, _lib.PASS_FWD, q.device)
    _lib.jagged_attn_fwd(p, q, k, v, o, lse, o_res, ws)
    return o, lse, o_res


def rope(q, k, q_offsets, kv_offsets, *, rope_base, out=None):
    """q and k turned by the rotary embedding of their sample-local positions (q_offsets
    None: a shared block, row r at position r), as new tensors or into out = (q_out, k_out)
    (which may be q and k themselves)."""
    _check_inputs(q, k, k, q_offsets, kv_offsets, None)
    p = _problem(q, k, q_offsets, kv_offsets, causal=False, scale=None, act="silu", bias=None,
                 bias_kind="none", bias_lo=0, bias_hi=0, rope_base=rope_base)
    qt, kt = out if out is not None else (torch.empty_like(q), torch.empty_like(k))
    _lib.jagged_rope(p, q, k, qt, kt)
    return qt, kt


def _check_mx(q, k, v, scales):
    for name, t in (("q", q), ("k", k), ("v", v)):
        sc = scales[name]
        if not t.is_cuda or not t.is_contiguous() or t.dim() != 3 or t.dtype != torch.uint8:
            raise ValueError(f"{name} must hold MXFP8 codes: a contiguous 3-D uint8 device tensor")
        if (sc.dtype != torch.uint8 or not sc.is_cuda or not sc.is_contiguous()
                or tuple(sc.shape) != (t.shape[0], t.shape[1], t.shape[2] // 32)):
            raise ValueError(f"{name} scale codes must be a contiguous uint8 [T, H, D/32] device tensor")
    if k.shape != v.shape or k.shape[1:] != q.shape[1:]:
        raise ValueError("q, k, v shapes disagree")


def mx_forward(mode, q, q_scale, k, k_scale, v, v_scale, q_offsets, kv_offsets, *, act="silu", scale=None,
               causal=False, bias=None, bias_kind="none", bias_lo=0, bias_hi=0, residual=True,
               max_kv_len=0, window=0):
    """Forward on MXFP8 inputs (E4M3 codes uint8 [T, H, D], E8M0 scale codes uint8
    [T, H, D/32]); bf16 outputs.  mode "gdpa" returns O; "jfa" returns (O, LSE, O_residual)."""
    _check_mx(q, k, v, {"q": q_scale, "k": k_scale, "v": v_scale})
    B = int(kv_offsets.numel()) - 1
    H, D = int(q.shape[1]), int(q.shape[2])
    p = _lib.make_problem(
        batch=B, heads=H, head_dim=D, dtype=torch.bfloat16, total_q=int(q.shape[0]), total_k=int(k.shape[0]),
        q_offsets=q_offsets, kv_offsets=kv_offsets, lq_fixed=0 if q_offsets is not None else int(q.shape[0]),
        causal=causal, scale=scale, act=act, bias_kind=bias_kind if bias is not None else "none",
        bias_table=bias, bias_lo=bias_lo, bias_hi=bias_hi, max_kv_len=max_kv_len, window=window)
    rows = q.shape[0] if q_offsets is not None else B * q.shape[0]
    o = torch.empty((rows, H, D), dtype=torch.bfloat16, device=q.device)
    ws = _workspace(p, _lib.PASS_FWD, q.device)
    if mode == "gdpa":
        _lib.jagged_gdpa_fwd_mx(p, q, q_scale, k, k_scale, v, v_scale, o, ws)
        return o
    lse = torch.empty((H, rows), dtype=torch.float32, device=q.device)
    o_res = torch.empty_like(o) if residual else None
    _lib.jagged_attn_fwd_mx(p, q, q_scale, k, k_scale, v, v_scale, o, lse, o_res, ws)
    return o, lse, o_res


def _dbias_out(p, bias, with_dbias):
    """Bias-gradient output [H, hi - lo + 1] and the workspace pass that goes with it."""
    if not with_dbias:
        return None, _lib.PASS_BWD
    if bias is None:
        raise ValueError("with_dbias needs a bias table")
    return torch.empty_like(bias), _lib.PASS_BWD_DBIAS


def gdpa_backward(q, k, v, dout, q_offsets, kv_offsets, *, act="silu", scale=None, causal=False,
                  bias=None, bias_kind="none", bias_lo=0, bias_hi=0, max_kv_len=0, window=0,
                  rope_base=0.0, rope_inputs_turned=False, with_dbias=False):
    """(dQ, dK, dV), plus the bias table's gradient last when with_dbias."""
    _check_inputs(q, k, v, q_offsets, kv_offsets, bias)
    p = _problem(q, k, q_offsets, kv_offsets, causal=causal, scale=scale, act=act, bias=bias,
                 bias_kind=bias_kind, bias_lo=bias_lo, bias_hi=bias_hi, max_kv_len=max_kv_len,
                 window=window, rope_base=rope_base, rope_inputs_turned=rope_inputs_turned)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    db, pass_ = _dbias_out(p, bias, with_dbias)
    ws = _workspace(p, pass_, q.device)
    _lib.jagged_gdpa_bwd(p, q, k, v, dout.contiguous(), dq, dk, dv, db, ws)
    return (dq, dk, dv, db) if with_dbias else (dq, dk, dv)


def attn_backward(q, k, v, o, dout, lse, q_offsets, kv_offsets, *, o_residual=None, scale=None,
                  causal=False, bias=None, bias_kind="none", bias_lo=0, bias_hi=0, max_kv_len=0,
                  window=0, rope_base=0.0, rope_inputs_turned=False, with_dbias=False):
    """(dQ, dK, dV), plus the bias table's gradient last when with_dbias."""
    _check_inputs(q, k, v, q_offsets, kv_offsets, bias)
    p = _problem(q, k, q_offsets, kv_offsets, causal=causal, scale=scale, act="silu", bias=bias,
                 bias_kind=bias_kind, bias_lo=bias_lo, bias_hi=bias_hi, max_kv_len=max_kv_len,
                 window=window, rope_base=rope_base, rope_inputs_turned=rope_inputs_turned)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    db, pass_ = _dbias_out(p, bias, with_dbias)
    ws = _workspace(p, pass_, q.device)
    _lib.jagged_attn_bwd(p, q, k, v, o, o_residual, dout.contiguous(), lse, dq, dk, dv, db, ws)
    return (dq, dk, dv, db) if with_dbias else (dq, dk, dv)


class _GDPAFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, q_offsets, kv_offsets, act, scale, causal, bias, bias_kind, bias_lo,
                bias_hi, max_kv_len, window, rope_base):
        kw = dict(act=act, scale=scale, causal=causal, bias=bias, bias_kind=bias_kind,
                  bias_lo=bias_lo, bias_hi=bias_hi, max_kv_len=max_kv_len, window=window,
                  rope_base=rope_base, rope_inputs_turned=rope_base > 0)
        if rope_base > 0:  # turned once, for the forward and the backward
            q, k = rope(q, k, q_offsets, kv_offsets, rope_base=rope_base)
        ctx.kw = kw
        ctx.save_for_backward(q, k, v, q_offsets, kv_offsets)
        return gdpa_forward(q, k, v, q_offsets, kv_offsets, **kw)

    @staticmethod
    def backward(ctx, do):
        q, k, v, q_offsets, kv_offsets = ctx.saved_tensors
        want_db = ctx.needs_input_grad[8]  # the bias table
        g = gdpa_backward(q, k, v, do, q_offsets, kv_offsets, with_dbias=want_db, **ctx.kw)
        db = g[3] if want_db else None
        return g[0], g[1], g[2], None, None, None, None, None, db, None, None, None, None, None, None


class _JFAFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, q_offsets, kv_offsets, scale, causal, bias, bias_kind, bias_lo,
                bias_hi, max_kv_len, window, rope_base):
        kw = dict(scale=scale, causal=causal, bias=bias, bias_kind=bias_kind, bias_lo=bias_lo,
                  bias_hi=bias_hi, max_kv_len=max_kv_len, window=window, rope_base=rope_base,
                  rope_inputs_turned=rope_base > 0)
        if rope_base > 0:  # turned once, for the forward and the backward
            q, k = rope(q, k, q_offsets, kv_offsets, rope_base=rope_base)
        o, lse, o_res = attn_forward(q, k, v, q_offsets, kv_offsets, **kw)
        ctx.kw = kw
        ctx.save_for_backward(q, k, v, o, lse, o_res, q_offsets, kv_offsets)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, o_res, q_offsets, kv_offsets = ctx.saved_tensors
        want_db = ctx.needs_input_grad[7]  # the bias table
        g = attn_backward(q, k, v, o, do, lse, q_offsets, kv_offsets, o_residual=o_res,
                          with_dbias=want_db, **ctx.kw)
        db = g[3] if want_db else None
        return g[0], g[1], g[2], None, None, None, None, db, None, None, None, None, None, None


def gdpa(q, k, v, q_offsets, kv_offsets, *, act="silu", scale=None, causal=False, bias=None,
         bias_kind="none", bias_lo=0, bias_hi=0, max_kv_len=0, window=0, rope_base=0.0):
    """Jagged GDPA with autograd (backward needs per-sample query offsets; a bias table
    that requires grad gets its gradient)."""
    return _GDPAFunction.apply(q, k, v, q_offsets, kv_offsets, act, scale, causal, bias,
                               bias_kind, bias_lo, bias_hi, max_kv_len, window, rope_base)


def jagged_attention(q, k, v, q_offsets, kv_offsets, *, scale=None, causal=False, bias=None,
                     bias_kind="none", bias_lo=0, bias_hi=0, max_kv_len=0, window=0,
                     rope_base=0.0):
    """Jagged flash attention (softmax) with autograd (a bias table that requires grad gets
    its gradient)."""
    return _JFAFunction.apply(q, k, v, q_offsets, kv_offsets, scale, causal, bias, bias_kind,
                              bias_lo, bias_hi, max_kv_len, window, rope_base)
