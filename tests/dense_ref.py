"""Padded dense attention with an explicit mask, in torch float64 on the CPU.

This is the brute-force check of the jagged oracle: every sample is padded to
the batch maximum, an explicit [B, Lq_max, Lk_max] mask is built, and the
products, activations and softmax come from torch library routines.  Gradients
come from torch autograd.  It shares nothing with the oracle's loop nests.
"""
import numpy as np
import torch
import torch.nn.functional as F


def _act(name, x):
    if name == "silu":
        return F.silu(x)
    if name == "gelu_tanh":
        return F.gelu(x, approximate="tanh")
    return F.gelu(x, approximate="none")


def _pad(x, off, lens, L):
    """[T, H, D] jagged -> [B, H, L, D] zero-padded."""
    B = len(lens)
    H, D = x.shape[1], x.shape[2]
    out = torch.zeros(B, H, L, D, dtype=x.dtype)
    for b in range(B):
        s, n = int(off[b]), int(lens[b])
        out[b, :, :n] = x[s:s + n].permute(1, 0, 2)
    return out


def _rope(xp, base):
    """Rotary embedding of padded [B, H, L, D] rows by their padded (sample-local)
    index t: the halves of the head dimension form complex numbers
    z_d = x_d + i x_{d + D/2}, multiplied by exp(i t base^(-2d/D))."""
    D = xp.shape[-1]
    half = D // 2
    t = torch.arange(xp.shape[2], dtype=torch.float64).view(1, 1, -1, 1)
    freq = torch.pow(torch.tensor(float(base), dtype=torch.float64),
                     -2.0 * torch.arange(half, dtype=torch.float64) / D)
    z = torch.complex(xp[..., :half], xp[..., half:]) * torch.polar(torch.ones_like(t * freq), t * freq)
    return torch.cat([z.real, z.imag], dim=-1)


def _unpad(xp, off, lens, T):
    H, D = xp.shape[1], xp.shape[3]
    out = torch.zeros(T, H, D, dtype=xp.dtype)
    for b in range(len(lens)):
        s, n = int(off[b]), int(lens[b])
        out[s:s + n] = xp[b, :, :n].permute(1, 0, 2)
    return out


def dense(w, *, grads=True):
    """Return dict with o (and lse for JFA; dq, dk, dv if grads) as float64 numpy arrays
    in the jagged token-major layout."""
    B, H, D = w.B, w.H, w.D
    lq = w.lq.astype(np.int64)
    lk = w.lk.astype(np.int64)
    Lq = max(int(lq.max()) if B else 0, 1)
    Lk = max(int(lk.max()) if B else 0, 1)
    q = w.q.double().clone().requires_grad_(grads)
    k = w.k.double().clone().requires_grad_(grads)
    v = w.v.double().clone().requires_grad_(grads)
    if w.q_off is None:
        qp = q.permute(1, 0, 2).unsqueeze(0).expand(B, H, w.lq_fixed, D)
        qp = F.pad(qp, (0, 0, 0, Lq - w.lq_fixed))
        out_off = np.arange(B + 1) * w.lq_fixed
    else:
        qp = _pad(q, w.q_off, lq, Lq)
        out_off = w.q_off
    kp = _pad(k, w.kv_off, lk, Lk)
    vp = _pad(v, w.kv_off, lk, Lk)
    if w.rope_base:
        qp, kp = _rope(qp, w.rope_base), _rope(kp, w.rope_base)

    i = torch.arange(Lq).view(1, Lq, 1)
    j = torch.arange(Lk).view(1, 1, Lk)
    lq_t = torch.from_numpy(lq).view(B, 1, 1)
    lk_t = torch.from_numpy(lk).view(B, 1, 1)
    mask = (i < lq_t) & (j < lk_t)
    if w.causal:
        mask = mask & (j <= i + lk_t - lq_t)
    if w.window:
        ia = i + lk_t - lq_t  # aligned query position
        mask = mask & (ia - j < w.window)
        if not w.causal:
            mask = mask & (j - ia < w.window)
    mask = mask.unsqueeze(1)  # [B, 1, Lq, Lk]

    x = w.scale * torch.matmul(qp, kp.transpose(-1, -2))
    tab = None
    if w.bias_kind != "none":
        tab = w.bias_table.double().clone().requires_grad_(grads)
        ii, jj = torch.arange(Lq).view(Lq, 1), torch.arange(Lk).view(1, Lk)
        idx = (ii - jj) if w.bias_kind == "rel" else jj.expand(Lq, Lk)
        idx = idx.clamp(w.bias_lo, w.bias_hi) - w.bias_lo
        x = x + tab[:, idx].unsqueeze(0)  # [1, H, Lq, Lk]

    res = {}
    if w.mode == "gdpa":
        p = _act(w.act, x) * mask  # mask after the activation
        op = torch.matmul(p, vp)
    else:
        xm = x.masked_fill(~mask, float("-inf"))
        rowvalid = mask.any(-1, keepdim=True)
        xs = torch.where(rowvalid, xm, torch.zeros_like(xm))
        p = torch.softmax(xs, dim=-1) * rowvalid
        op = torch.matmul(p, vp)
        lse = torch.logsumexp(xs, dim=-1, keepdim=True)
        lse = torch.where(rowvalid, lse, torch.full_like(lse, float("-inf"))).squeeze(-1)
        # [B, H, Lq] -> [T_out, H]
        lse_out = torch.zeros(int(out_off[-1]), H, dtype=torch.float64)
        for b in range(B):
            s, n = int(out_off[b]), int(lq[b])
            lse_out[s:s + n] = lse[b, :, :n].T.detach()
        res["lse"] = lse_out.numpy()
    o = _unpad(op, out_off, lq, int(out_off[-1]))
    res["o"] = o.detach().numpy()
    if grads and w.dout is not None:
        loss = (o * w.dout.double()).sum()
        loss.backward()
        res["dq"] = q.grad.numpy()
        res["dk"] = k.grad.numpy()
        res["dv"] = v.grad.numpy()
        if tab is not None:
            res["dbias"] = tab.grad.numpy()
    return res
