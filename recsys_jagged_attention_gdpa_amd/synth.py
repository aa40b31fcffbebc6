"""Seeded synthetic jagged workloads.

This module only draws inputs: lengths, offsets, Q / K / V, bias tables and
upstream gradients.  It holds none of the attention arithmetic, so both the GPU
tests and the CPU oracle can be fed from it.

The workloads model the pages' production statistics: per-sample lengths from
hundreds to tens of thousands of tokens and a jagged length sparsity of 0.5
("GEM Training: How Meta Doubled the Efficiency...", section "What happened";
"Meta redesigns AI training infrastructure...", sections "Eliminating Compute
Waste in Asymmetric Workloads" and "Key Numbers").  Sparsity here is
1 - sum(L_b) / (B * max L_b).

Recipe (shared by every workload):
  * ``rng = numpy.random.default_rng(seed)`` (PCG64);
  * draw order: lengths, Q, K, V, bias table, dO;
  * normals are drawn in float32 as ``sigma * standard_normal``; "N(0, s2)" in a
    workload description means variance s2;
  * bf16 workloads round the float32 draws to bf16 (round to nearest even);
  * offsets are int32 ``[0, cumsum(L)]``.

MXFP8 inputs (tensors named in ``mx``) are given as element codes uint8
[T, H, D] and scale codes uint8 [T, H, D / 32] (blocks of 32 head-dimension
elements), drawn after everything else: one scale code per block uniform on
{125 .. 128}, then the element codes are the FP8 E4M3 casts (torch's
``float8_e4m3fn``) of the tensor's float32 normal draws divided by the block's
scale 2^(code - 127), clamped to +-448 first.  This stands in for the upstream
kernels that quantise their outputs; the attention itself only decodes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass
class Workload:
    name: str
    mode: str  # "gdpa" or "jfa"
    B: int
    H: int
    D: int
    dtype: torch.dtype
    q_off: Optional[np.ndarray]  # int32 [B+1], or None for one shared query block
    lq_fixed: int
    kv_off: np.ndarray  # int32 [B+1]
    q: torch.Tensor  # [Tq, H, D] (or [lq_fixed, H, D])
    k: torch.Tensor  # [Tk, H, D]
    v: torch.Tensor
    dout: Optional[torch.Tensor]  # [Tq_out, H, D]
    act: str  # "silu", "gelu_tanh", "gelu_erf" (ignored for jfa)
    scale: float
    causal: bool
    bias_kind: str  # "none", "rel", "keypos"
    bias_table: Optional[torch.Tensor]  # float32 [H, hi - lo + 1]
    bias_lo: int
    bias_hi: int
    backward: bool  # whether the workload includes a backward pass
    window: int = 0  # sliding window: a query sees keys at aligned distance < window (0: no window)
    rope_base: float = 0.0  # rotary embedding of q and k by sample-local position (0: none)
    mx: tuple = ()  # names ("q", "k", "v") of tensors given in MXFP8: the tensor holds uint8 codes
    mx_scales: Optional[dict] = None  # name -> uint8 scale codes [T, H, D / 32]

    @property
    def lq(self) -> np.ndarray:
        if self.q_off is None:
            return np.full(self.B, self.lq_fixed, dtype=np.int64)
        return np.diff(self.q_off.astype(np.int64))

    @property
    def lk(self) -> np.ndarray:
        return np.diff(self.kv_off.astype(np.int64))

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def total_q_out(self) -> int:
        return int(self.B * self.lq_fixed) if self.q_off is None else self.total_q

    @property
    def total_k(self) -> int:
        return int(self.k.shape[0])

    def subset(self, samples) -> "Workload":
        """A workload made of the listed samples only, in that order (offsets rebased)."""
        samples = [int(b) for b in samples]

        def gather(t, off, idx):
            if t is None:
                return None
            parts = [t[int(off[b]):int(off[b + 1])] for b in idx]
            return torch.cat(parts, 0) if parts else t[:0]

        def offs(off, idx):
            lens = [int(off[b + 1]) - int(off[b]) for b in idx]
            return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)

        if self.q_off is None:
            q, q_off = self.q, None
            out_off = np.arange(self.B + 1, dtype=np.int64) * self.lq_fixed
        else:
            q, q_off = gather(self.q, self.q_off, samples), offs(self.q_off, samples)
            out_off = self.q_off
        scales = None
        if self.mx_scales:
            scales = {}
            for name, sc in self.mx_scales.items():
                if name == "q":
                    scales[name] = sc if self.q_off is None else gather(sc, self.q_off, samples)
                else:
                    scales[name] = gather(sc, self.kv_off, samples)
        return dataclasses.replace(
            self, B=len(samples), q_off=q_off, q=q,
            kv_off=offs(self.kv_off, samples), k=gather(self.k, self.kv_off, samples),
            v=gather(self.v, self.kv_off, samples), dout=gather(self.dout, out_off, samples),
            mx_scales=scales)


def _normal(rng, shape, sigma, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return torch.from_numpy(x).to(dtype)


def _mx_encode(rng, x: torch.Tensor):
    """MXFP8 codes of float32 draws x [T, H, D]: (element codes, scale codes)."""
    T, H, D = x.shape
    sc = rng.integers(125, 129, size=(T, H, D // 32)).astype(np.uint8)
    step = torch.from_numpy(np.ldexp(1.0, sc.astype(np.int64) - 127).astype(np.float32))
    y = (x.float().reshape(T, H, D // 32, 32) / step[..., None]).clamp(-448.0, 448.0)
    codes = y.reshape(T, H, D).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, torch.from_numpy(sc)


def _mx_inputs(rng, mx, q, k, v):
    """Codes for the tensors named in mx (in the order q, k, v) and their scale codes."""
    scales, enc = {}, {"q": q, "k": k, "v": v}
    for name in ("q", "k", "v"):
        if name in mx:
            enc[name], scales[name] = _mx_encode(rng, enc[name])
    return enc["q"], enc["k"], enc["v"], scales


def _offsets(lens):
    return np.concatenate([[0], np.cumsum(np.asarray(lens, dtype=np.int64))]).astype(np.int32)


# Workload catalogue.  Each entry: the full-size parameters.  ``make`` can shrink
# B and the maximum length for parity tests while keeping the distribution's
# shape (lengths are still jagged with a ragged tail).
CATALOGUE = {
    # Tiny fp32 GDPA, self-attention, SiLU, no bias.
    "tiny_gdpa_fp32": dict(mode="gdpa", B=4, H=2, D=32, dtype="fp32", q_len=("uniform", 1, 64),
                           kv_len="same", qkv_sigma=1.0, act="silu", causal=False, bias=None,
                           backward=True),
    # GDPA cross-attention, short K/V: jagged queries U{1..1024}, 32 keys per sample.
    "gdpa_xattn_short_kv": dict(mode="gdpa", B=1024, H=4, D=128, dtype="bf16",
                                q_len=("uniform", 1, 1024), kv_len=("fixed", 32),
                                qkv_sigma=math.sqrt(0.5), act="gelu_tanh", causal=False, bias=None,
                                backward=True),
    # JFA causal self-attention, L ~ U{1..8192}.
    "jfa_causal_self": dict(mode="jfa", B=64, H=8, D=128, dtype="bf16", q_len=("uniform", 1, 8192),
                            kv_len="same", qkv_sigma=1.0, act=None, causal=True, bias=None,
                            backward=True),
    # PMA-style GDPA: 16 shared seed queries against jagged K/V U{1..4096}, key-position bias.
    "pma_gdpa_fwd": dict(mode="gdpa", B=2048, H=4, D=64, dtype="bf16", q_len=("shared", 16),
                         kv_len=("uniform", 1, 4096), qkv_sigma=1.0, act="silu", causal=False,
                         bias=("keypos", 0, 4095, math.sqrt(0.1)), backward=False),
    # Long-tail GDPA self-attention, L log-uniform on [100, 16384], relative-position bias.
    "longtail_gdpa": dict(mode="gdpa", B=256, H=8, D=128, dtype="bf16",
                          q_len=("loguniform", 100, 16384), kv_len="same", qkv_sigma=1.0,
                          act="gelu_erf", causal=False, bias=("rel", -512, 512, math.sqrt(0.1)),
                          backward=True),
    # The JFA causal self-attention batch with a sliding window of 1024 keys (the
    # pages report sliding-window attention on long-sequence self-attention).
    "jfa_swa_causal_self": dict(mode="jfa", B=64, H=8, D=128, dtype="bf16", q_len=("uniform", 1, 8192),
                                kv_len="same", qkv_sigma=1.0, act=None, causal=True, bias=None,
                                backward=True, window=1024, same_draw_as="jfa_causal_self"),
    # The same batch with q and k turned by the rotary embedding (base 10000) of
    # their positions (the pages pair rotary embedding with long-sequence
    # self-attention).
    "jfa_rope_causal_self": dict(mode="jfa", B=64, H=8, D=128, dtype="bf16", q_len=("uniform", 1, 8192),
                                 kv_len="same", qkv_sigma=1.0, act=None, causal=True, bias=None,
                                 backward=True, rope_base=10000.0, same_draw_as="jfa_causal_self"),
    # The pooling and cross-attention forwards with MXFP8 queries, keys and values
    # (the pages report MXFP8-based attention; the quantisation happens upstream).
    "pma_gdpa_fwd_mxfp8": dict(mode="gdpa", B=2048, H=4, D=64, dtype="bf16", q_len=("shared", 16),
                               kv_len=("uniform", 1, 4096), qkv_sigma=1.0, act="silu", causal=False,
                               bias=("keypos", 0, 4095, math.sqrt(0.1)), backward=False, mx=("q", "k", "v"),
                               same_draw_as="pma_gdpa_fwd"),
    "jfa_causal_self_fwd_mxfp8": dict(mode="jfa", B=64, H=8, D=128, dtype="bf16", q_len=("uniform", 1, 8192),
                                      kv_len="same", qkv_sigma=1.0, act=None, causal=True, bias=None,
                                      backward=False, mx=("q", "k", "v"), same_draw_as="jfa_causal_self"),
    "gdpa_xattn_short_kv_mxfp8": dict(mode="gdpa", B=1024, H=4, D=128, dtype="bf16",
                                      q_len=("uniform", 1, 1024), kv_len=("fixed", 32),
                                      qkv_sigma=math.sqrt(0.5), act="gelu_tanh", causal=False, bias=None,
                                      backward=False, mx=("q", "k", "v"), same_draw_as="gdpa_xattn_short_kv"),
}


def _draw_lengths(rng, spec, B, max_len):
    kind = spec[0]
    if kind == "uniform":
        lo, hi = spec[1], spec[2] if max_len is None else min(spec[2], max_len)
        return rng.integers(lo, hi + 1, size=B)
    if kind == "loguniform":
        lo, hi = spec[1], spec[2] if max_len is None else min(spec[2], max_len)
        lo = min(lo, hi)
        return np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=B))).astype(np.int64)
    if kind == "fixed":
        return np.full(B, spec[1], dtype=np.int64)
    raise ValueError(spec)


def make(name: str, seed: Optional[int] = None, *, B: Optional[int] = None,
         max_len: Optional[int] = None, with_dout: Optional[bool] = None) -> Workload:
    """Draw workload ``name``.  ``B`` and ``max_len`` shrink it for parity tests."""
    spec = CATALOGUE[name]
    if seed is None:  # a variant of another workload draws the same batch
        seed = 1000 + list(CATALOGUE).index(spec.get("same_draw_as", name)) + 1
    rng = np.random.default_rng(seed)
    B = spec["B"] if B is None else B
    H, D = spec["H"], spec["D"]
    dtype = torch.float32 if spec["dtype"] == "fp32" else torch.bfloat16
    sigma = spec["qkv_sigma"]

    q_off, lq_fixed = None, 0
    if spec["q_len"][0] == "shared":
        lq_fixed = spec["q_len"][1]
        lq = None
    else:
        lq = _draw_lengths(rng, spec["q_len"], B, max_len)
        q_off = _offsets(lq)
    if spec["kv_len"] == "same":
        lk = lq
    else:
        lk = _draw_lengths(rng, spec["kv_len"], B, max_len)
    kv_off = _offsets(lk)

    tq = lq_fixed if q_off is None else int(q_off[-1])
    tk = int(kv_off[-1])
    mx = tuple(spec.get("mx", ()))
    q = _normal(rng, (tq, H, D), sigma, torch.float32 if "q" in mx else dtype)
    k = _normal(rng, (tk, H, D), sigma, torch.float32 if "k" in mx else dtype)
    v = _normal(rng, (tk, H, D), sigma, torch.float32 if "v" in mx else dtype)

    bias_kind, table, lo, hi = "none", None, 0, 0
    if spec["bias"] is not None:
        bias_kind, lo, hi, bsig = spec["bias"]
        table = _normal(rng, (H, hi - lo + 1), bsig, torch.float32)

    backward = spec["backward"] if with_dout is None else with_dout
    dout = None
    if backward:
        t_out = B * lq_fixed if q_off is None else tq
        dout = _normal(rng, (t_out, H, D), 1.0, dtype)
    scales = None
    if mx:
        q, k, v, scales = _mx_inputs(rng, mx, q, k, v)
    return Workload(name=name, mode=spec["mode"], B=B, H=H, D=D, dtype=dtype, q_off=q_off,
                    lq_fixed=lq_fixed, kv_off=kv_off, q=q, k=k, v=v, dout=dout,
                    act=spec["act"] or "silu", scale=1.0 / math.sqrt(D), causal=spec["causal"],
                    bias_kind=bias_kind, bias_table=table, bias_lo=lo, bias_hi=hi,
                    backward=spec["backward"], window=spec.get("window", 0),
                    rope_base=float(spec.get("rope_base", 0.0)), mx=mx, mx_scales=scales)


def custom(*, mode="gdpa", lq, lk=None, H=2, D=64, dtype=torch.bfloat16, seed=0, sigma=1.0,
           act="silu", causal=False, bias_kind="none", bias_lo=0, bias_hi=0, bias_sigma=0.3,
           shared_q=None, scale=None, with_dout=True, window=0, rope_base=0.0, mx=()) -> Workload:
    """A workload with explicit per-sample lengths (edge cases, small shapes).

    ``shared_q`` = n gives one shared block of n query rows (``lq`` is ignored);
    ``mx`` names the tensors ("q", "k", "v") given in MXFP8 (``dtype`` is then the
    type of the others and of the outputs)."""
    rng = np.random.default_rng(seed)
    lk = lq if lk is None else lk
    B = len(lk)
    q_off, lq_fixed = (None, int(shared_q)) if shared_q else (_offsets(lq), 0)
    kv_off = _offsets(lk)
    tq = lq_fixed if q_off is None else int(q_off[-1])
    tk = int(kv_off[-1])
    mx = tuple(mx)
    assert set(mx) <= {"q", "k", "v"}
    q = _normal(rng, (tq, H, D), sigma, torch.float32 if "q" in mx else dtype)
    k = _normal(rng, (tk, H, D), sigma, torch.float32 if "k" in mx else dtype)
    v = _normal(rng, (tk, H, D), sigma, torch.float32 if "v" in mx else dtype)
    table = None
    if bias_kind != "none":
        table = _normal(rng, (H, bias_hi - bias_lo + 1), bias_sigma, torch.float32)
    dout = None
    if with_dout:
        t_out = B * lq_fixed if q_off is None else tq
        dout = _normal(rng, (t_out, H, D), 1.0, dtype)
    scales = None
    if mx:
        q, k, v, scales = _mx_inputs(rng, mx, q, k, v)
    return Workload(name="custom", mode=mode, B=B, H=H, D=D, dtype=dtype, q_off=q_off,
                    lq_fixed=lq_fixed, kv_off=kv_off, q=q, k=k, v=v, dout=dout, act=act,
                    scale=(1.0 / math.sqrt(D)) if scale is None else scale, causal=causal,
                    bias_kind=bias_kind, bias_table=table, bias_lo=bias_lo, bias_hi=bias_hi,
                    backward=with_dout, window=int(window), rope_base=float(rope_base), mx=mx,
                    mx_scales=scales)
