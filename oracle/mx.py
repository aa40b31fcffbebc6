"""MXFP8 decoding for the oracle — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this module.  It shares no code with the GPU library.

The pages report MXFP8-based attention (ultra-low-precision training of
attention modules, with the quantisation fused into the upstream projection
and normalisation kernels: "Meta redesigns AI training infrastructure...",
sections "Custom Kernels and 5D Parallelism for Trillion-Parameter Scale" and
"Key Numbers"; "GEM Training: How Meta Doubled the Efficiency of an LLM-Scale
Ads Foundation Model", body) without defining the format.  The reading here is
the OCP Microscaling (MX) format MXFP8 with E4M3 elements:

  * a block of 32 consecutive elements shares one scale X stored as E8M0, an
    8-bit biased exponent: X = 2^(E - 127), code 255 = NaN;
  * each element is FP8 E4M3: sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent field 0 encodes subnormals m/8 * 2^-6, the all-ones
    exponent with all-ones mantissa is NaN (no infinities), largest finite
    magnitude 1.75 * 2^8 = 448;
  * the value of an element is X times its E4M3 value.

In the attention tensors a block is 32 consecutive head-dimension elements of
one row and head: codes [T, H, D] and scale codes [T, H, D / 32], both uint8.
Attention on MXFP8 inputs is the plain definition applied to the decoded
values (decoding is exact in float64).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32


def e4m3_value(codes) -> np.ndarray:
    """Float64 value of FP8 E4M3 codes (uint8 array)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    sub = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, v)


def e8m0_value(codes) -> np.ndarray:
    """Float64 value 2^(E - 127) of E8M0 scale codes (uint8 array); 255 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def decode(codes, scales) -> np.ndarray:
    """Values [T, H, D] of MXFP8 codes [T, H, D] with scale codes [T, H, D / 32]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    T, H, D = codes.shape
    assert D % BLOCK == 0 and scales.shape == (T, H, D // BLOCK), (codes.shape, scales.shape)
    x = e4m3_value(codes).reshape(T, H, D // BLOCK, BLOCK)
    return (x * e8m0_value(scales)[..., None]).reshape(T, H, D)


def decode_f32(codes, scales) -> np.ndarray:
    """decode() as float32, for the oracle's float32 inputs.  Every finite MXFP8
    value with a scale code up to 246 is a float32 value; anything else is refused."""
    v = decode(codes, scales)
    with np.errstate(over="ignore"):
        f = v.astype(np.float32)
    assert np.isfinite(v).all() and np.array_equal(f.astype(np.float64), v), \
        "MXFP8 values outside what float32 holds exactly"
    return f


# ------------------------------------------------------- P in FP8 for PV
# The MXFP8 forward with D = 64 or 128 forms P V on a block-scaled FP8 matrix
# product, so P itself is encoded as E4M3.  What it computes, step by step (the
# reading of "MXFP8-based attention" with P in FP8, written out):
#   1. value rows re-encoded to one scale per key: S_j = the largest block scale
#      code of row j (and head), each element's E4M3 value times 2^(s_jb - S_j)
#      rounded to the nearest E4M3 value (ties to the even code);
#   2. P as in plain attention (GDPA: act(X); JFA: 2^(X log2 e - M_i) against a
#      whole number M_i, the row normaliser l_i = sum_j of those unencoded P);
#   3. P'_ij = P_ij 2^(S_j - 127); per query row and block of 32 sample-local keys
#      a power-of-two scale 2^E_b that puts the block's largest |P'| in [128, 256)
#      (E_b = k - 8 for a largest value f 2^k with f in [0.5, 1); 0 when all are
#      zero; E_b clamped to [-126, 127]); each P' rounded to the nearest E4M3 value
#      on that scale: Pq_ij = nearest(P'_ij 2^-E_b) 2^E_b;
#   4. O_i = sum_j Pq_ij V'_j (JFA: divided by l_i), V' the re-encoded E4M3 values.
# A whole-number M_i is what makes the result independent of which one: moving
# it by n multiplies P' and 2^E_b by 2^n and leaves every rounding unchanged.

_E4M3_POS = e4m3_value(np.arange(127, dtype=np.uint8))  # codes 0 .. 126: 0 to 448, increasing


def e4m3_nearest(x) -> np.ndarray:
    """Float64 value of the finite E4M3 number nearest to x, ties to the even code
    (mantissa bit 0); the sign of x is kept (also for zero).  |x| of 464 or more
    (past the largest value, 448, by half its step) has no finite nearest value and
    is refused."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    assert np.all(a < 464.0), "E4M3 encoding past the largest finite value"
    idx = np.searchsorted(_E4M3_POS, a)  # first code whose value is >= |x|
    lo = np.clip(idx - 1, 0, 126)
    hi = np.clip(idx, 0, 126)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    return np.copysign(_E4M3_POS[code], x)


def reencode_rows(codes, scales):
    """Step 1: (values [T, H, D] as E4M3 values on the row's common scale, S [T, H])
    for MXFP8 codes [T, H, D] with scale codes [T, H, D / 32]."""
    c = e4m3_value(np.asarray(codes, dtype=np.uint8))
    s = np.asarray(scales, dtype=np.uint8).astype(np.int64)
    S = s.max(axis=-1)
    shift = np.repeat(s - S[..., None], BLOCK, axis=-1)
    return e4m3_nearest(c * np.ldexp(1.0, shift)), S


def _encode_p(pp):
    """Steps 3: Pq for P' [rows, keys] (keys sample-local from 0), blocks of 32 keys."""
    out = np.zeros_like(pp)
    for k0 in range(0, pp.shape[1], BLOCK):
        blk = pp[:, k0:k0 + BLOCK]
        m = np.abs(blk).max(axis=1)
        e = np.where(m > 0, np.frexp(m)[1] - 8, 0)
        e = np.clip(e, -126, 127)[:, None].astype(np.float64)
        out[:, k0:k0 + BLOCK] = e4m3_nearest(blk * 2.0 ** -e) * 2.0 ** e
    return out


def fwd_fp8_pv(mode, q, k, v_codes, v_scales, q_off, kv_off, *, scale, act="silu", lq_fixed=0, causal=False,
               window=0, bias_kind="none", bias_table=None, bias_lo=0, bias_hi=0, row_chunk=512):
    """The MXFP8 forward with P in FP8 (steps 1-4 above), in float64.  q, k: decoded
    values [T, H, D] (float); v: codes and scale codes.  q_off None: a shared block of
    lq_fixed query rows.  The activation is the oracle's own (ref.act).  Returns O [Tq_out, H, D]
    and, for JFA, LSE [Tq_out, H] (natural log; -inf for rows without a key) and the
    row bound of one rounding step of the largest P term, flip [Tq_out, H]: one P
    element encoded one E4M3 step away moves O_i by at most flip_i."""
    from oracle import ref
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    kv_off = np.asarray(kv_off, dtype=np.int64)
    vv, S = reencode_rows(v_codes, v_scales)
    B = len(kv_off) - 1
    H, D = q.shape[1], q.shape[2]
    q_rows = [(0, lq_fixed)] * B if q_off is None else [(int(q_off[b]), int(q_off[b + 1])) for b in range(B)]
    t_out = B * lq_fixed if q_off is None else q.shape[0]
    o = np.zeros((t_out, H, D))
    lse = np.full((t_out, H), -np.inf)
    flip = np.zeros((t_out, H))
    tab = None if bias_table is None else np.asarray(bias_table, dtype=np.float64)
    for b in range(B):
        q0, q1 = q_rows[b]
        k0, k1 = int(kv_off[b]), int(kv_off[b + 1])
        lq, lk = q1 - q0, k1 - k0
        o0 = b * lq_fixed if q_off is None else q0
        if lq == 0 or lk == 0:
            continue
        j = np.arange(lk)[None, :]
        for h in range(H):
            for r0 in range(0, lq, row_chunk):
                i = np.arange(r0, min(lq, r0 + row_chunk))[:, None]
                x = scale * (q[q0 + i[:, 0], h] @ k[k0:k1, h].T)
                if bias_kind == "rel":
                    x = x + tab[h][np.clip(i - j, bias_lo, bias_hi) - bias_lo]
                elif bias_kind == "keypos":
                    x = x + tab[h][np.clip(j, bias_lo, bias_hi) - bias_lo] + 0 * i
                dist = i + lk - lq - j  # aligned distance
                ok = np.ones(x.shape, dtype=bool)
                if causal:
                    ok &= dist >= 0
                if window:
                    ok &= (dist < window) & (True if causal else (-dist < window))
                if mode == "gdpa":
                    p = np.where(ok, ref.act(act, x)[0], 0.0)
                    norm = np.ones(len(i))
                else:
                    l2 = np.where(ok, x * np.log2(np.e), -np.inf)
                    mrow = l2.max(axis=1)
                    has = np.isfinite(mrow)
                    M = np.where(has, np.ceil(np.where(has, mrow, 0.0)), 0.0)
                    p = np.where(ok, np.exp2(l2 - M[:, None]), 0.0)
                    lsum = p.sum(axis=1)
                    norm = np.where(lsum > 0, 1.0 / np.where(lsum > 0, lsum, 1.0), 0.0)
                    rows = o0 + i[:, 0]
                    lse[rows, h] = np.where(lsum > 0, (M + np.log2(np.where(lsum > 0, lsum, 1.0))) * np.log(2.0),
                                            -np.inf)
                pq = _encode_p(p * np.ldexp(1.0, S[k0:k1, h] - 127)[None, :])
                v = vv[k0:k1, h]
                o[o0 + i[:, 0], h] = (pq @ v) * norm[:, None]
                flip[o0 + i[:, 0], h] = 0.125 * (np.abs(pq) * np.abs(v).max(axis=1)[None, :]).max(axis=1) * norm
    return o, lse, flip
