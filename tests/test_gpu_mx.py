"""MXFP8 forward on the HIP path against the fp64 oracle.

q, k and v arrive as FP8 E4M3 codes with one E8M0 scale code per block of 32
head-dimension elements; the oracle decodes them exactly.  With D = 64 or 128
the GPU forms P V with P in FP8, and the oracle encodes P the same way (value
rows re-encoded to one scale per key, P' per 32-key block on its own scale),
then runs the rest in fp64; with D = 32 P stays bf16 and the oracle is plain
attention of the decoded values.  Same per-row bar as the bf16 path (tau = 2e-2;
rows with no visible key exactly zero); with P in FP8 a few rows may also carry
an element encoded one step apart (see fp8_pv_check).
"""
import pytest
import torch

from recsys_jagged_attention_gdpa_amd import synth
from tests.gpu_helpers import announce, gpu_fwd, mx_parity, to_dev

pytestmark = pytest.mark.gpu

# short (<= 32 keys) and long samples, Lq != Lk, empty samples, ragged tails
LQ = [1, 70, 300, 0, 129, 5, 40, 260, 33]
LK = [32, 1, 17, 0, 300, 65, 40, 129, 500]
MX = ("q", "k", "v")


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_mx_forward_matches_oracle(mode, causal, D):
    w = synth.custom(mode=mode, lq=LQ, lk=LK, H=2, D=D, seed=D + causal, act="gelu_tanh", causal=causal,
                     with_dout=False, mx=MX)
    mx_parity(w, label=f"mxfp8 {mode} causal={causal} D={D}")


@pytest.mark.parametrize("mode,bias,act", [("gdpa", "rel", "gelu_erf"), ("gdpa", "keypos", "silu"),
                                           ("jfa", "rel", "silu"), ("jfa", "keypos", "silu")])
def test_mx_forward_with_bias_and_window(mode, bias, act):
    w = synth.custom(mode=mode, lq=[600, 31, 128, 1, 0], lk=[600, 31, 200, 3, 7], H=3, D=128, seed=5,
                     act=act, causal=True, window=150, bias_kind=bias, bias_lo=-60 if bias == "rel" else 0,
                     bias_hi=60 if bias == "rel" else 300, with_dout=False, mx=MX)
    mx_parity(w, label=f"mxfp8 {mode} bias={bias}")


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
@pytest.mark.parametrize("shared,D", [(16, 64), (48, 64), (11, 128), (24, 64)])
def test_mx_forward_shared_queries(mode, shared, D):
    # 16 rows or fewer: one-wave 32-row units (GDPA: rows of two key blocks packed
    # into one block's lanes); 24: one-wave units unpacked; 48: the 4-wave units
    w = synth.custom(mode=mode, lq=None, lk=[700, 0, 1, 31, 33, 257, 4000], H=4, D=D, seed=3,
                     shared_q=shared, act="silu", bias_kind="keypos", bias_lo=0, bias_hi=4095,
                     with_dout=False, mx=MX)
    mx_parity(w, label=f"mxfp8 shared-q={shared} {mode}")


@pytest.mark.parametrize("case", ["wide scores", "wide values"])
def test_mx_jfa_without_residual_and_wide_scales(case):
    w = synth.custom(mode="jfa", lq=LQ, lk=LK, H=2, D=128, seed=9, with_dout=False, mx=MX)
    gen = torch.Generator().manual_seed(1)
    rnd = lambda lo, hi, sc: torch.randint(lo, hi, tuple(sc.shape), generator=gen, dtype=torch.int64).to(torch.uint8)
    if case == "wide scores":
        # every scale code over 2^-20 .. 2^+13 and the score scale times 2^-8: scores,
        # and with them the LSE, reach magnitudes of 10^4 (the LSE bar is relative)
        scales = {n: rnd(107, 141, w.mx_scales[n]) for n in MX}
        w = synth.Workload(**{**w.__dict__, "mx_scales": scales, "scale": w.scale * 2.0 ** -8})
    else:
        # value scale codes over 2^-27 .. 2^+27 (every decoded value stays inside bf16's
        # normal range); query / key codes over 2^-9 .. 2^0
        scales = {"q": rnd(118, 128, w.mx_scales["q"]), "k": rnd(118, 128, w.mx_scales["k"]),
                  "v": rnd(100, 155, w.mx_scales["v"])}
        w = synth.Workload(**{**w.__dict__, "mx_scales": scales})
    # value scales spread the O rows over 2^33 in magnitude: every row is compared on its
    # own scale.  Scores of 10^4 carry fp32 roundings of ~10^-3, far more than E4M3
    # midpoints are apart: there O is held to the encoding's error bound instead
    mx_parity(w, label=f"mxfp8 jfa {case}", o_floor_frac=1e-15, emulate=case != "wide scores")
    d = to_dev(w)
    a = gpu_fwd(w, d, residual=True)
    b = gpu_fwd(w, d, residual=False)
    torch.cuda.synchronize()
    announce("mxfp8 jfa residual on/off: LSE equal")
    assert torch.equal(a["lse"], b["lse"])


def test_mx_forward_is_deterministic():
    w = synth.custom(mode="gdpa", lq=LQ, lk=LK, H=2, D=128, seed=4, act="gelu_erf", with_dout=False, mx=MX)
    d = to_dev(w)
    announce("mxfp8 determinism")
    a, b = gpu_fwd(w, d), gpu_fwd(w, d)
    torch.cuda.synchronize()
    assert torch.equal(a["o"], b["o"])


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
def test_mx_short_only_batch_with_key_bound(mode):
    # every sample has at most 32 keys: with the bound the long kernels are not launched
    w = synth.custom(mode=mode, lq=[1, 700, 0, 33, 64], lk=[32, 5, 9, 0, 31], H=2, D=128, seed=13, act="silu",
                     with_dout=False, mx=MX)
    mx_parity(w, label=f"mxfp8 short-only {mode}", max_kv_len=32)


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
def test_mx_all_empty_samples(mode):
    # no query rows and no keys at all: nothing is read, the outputs have no rows
    w = synth.custom(mode=mode, lq=[0, 0, 0], lk=[0, 0, 0], H=2, D=64, seed=1, with_dout=False, mx=MX)
    mx_parity(w, label=f"mxfp8 empty {mode}")
    # keys but no queries, and queries but no keys (rows exactly zero, LSE -inf)
    w = synth.custom(mode=mode, lq=[0, 5, 0], lk=[40, 0, 3], H=2, D=64, seed=2, with_dout=False, mx=MX)
    mx_parity(w, label=f"mxfp8 one-sided {mode}")
