"""Sliding-window attention on the HIP path against the fp64 oracle.

A window w keeps the pairs whose aligned distance ia - j (ia = i + Lk - Lq) is
below w, and without causal masking also above -w.  Same per-row bar as the
other parity tests (tau = 2e-2 bf16, 1e-4 fp32; rows with no visible key exactly
zero).
"""
import pytest
import torch

from recsys_jagged_attention_gdpa_amd import synth
from tests.gpu_helpers import announce, gpu_bwd, gpu_fwd, parity, to_dev

pytestmark = pytest.mark.gpu

# short (<= 32 keys) and long samples, Lq != Lk, empty samples, ragged tails
LQ = [1, 70, 300, 0, 129, 5, 40, 260, 33]
LK = [32, 1, 17, 0, 300, 65, 40, 129, 500]


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("window", [1, 7, 64, 100, 257])
def test_window_matches_oracle(mode, causal, window):
    w = synth.custom(mode=mode, lq=LQ, lk=LK, H=2, D=128, seed=window + 7 * causal, act="gelu_tanh",
                     causal=causal, window=window)
    parity(w, label=f"window {mode} causal={causal} w={window}")


@pytest.mark.parametrize("mode,bias,D", [("gdpa", "rel", 64), ("jfa", "keypos", 32), ("jfa", "rel", 128)])
def test_window_with_bias_and_dims(mode, bias, D):
    w = synth.custom(mode=mode, lq=[600, 31, 128, 1], lk=[600, 31, 200, 3], H=3, D=D, seed=D, act="silu",
                     causal=True, window=150, bias_kind=bias, bias_lo=-60 if bias == "rel" else 0,
                     bias_hi=60 if bias == "rel" else 300, bias_sigma=0.3)
    parity(w, label=f"window {mode} bias={bias} D={D}")


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
def test_window_shared_queries_and_fp32(mode):
    w = synth.custom(mode=mode, lq=None, lk=[700, 0, 1, 31, 33, 257], H=2, D=64, seed=3, shared_q=24,
                     act="silu", window=40, with_dout=False)
    parity(w, backward=False, label=f"window shared-q {mode}")
    w = synth.custom(mode=mode, lq=[9, 0, 23, 1, 17], lk=[9, 5, 23, 1, 0], H=2, D=32, dtype=torch.float32,
                     seed=4, causal=True, window=5)
    parity(w, label=f"window fp32 {mode}")


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
@pytest.mark.parametrize("causal", [False, True])
def test_window_wider_than_every_sample_is_bitwise_no_window(mode, causal):
    w = synth.custom(mode=mode, lq=LQ, lk=LK, H=2, D=64, seed=11, causal=causal, act="gelu_erf")
    wide = synth.Workload(**{**w.__dict__, "window": 4096})
    announce(f"window wide-vs-none {mode} causal={causal}")
    d = to_dev(w)
    a, b = gpu_fwd(w, d), gpu_fwd(wide, d)
    ga, gb = gpu_bwd(w, d, a), gpu_bwd(wide, d, b)
    torch.cuda.synchronize()
    for n in a:
        if a[n] is not None:
            assert torch.equal(a[n], b[n]), n
    for n in ga:
        assert torch.equal(ga[n], gb[n]), n


def test_window_bias_gradient():
    from tests.test_gpu_dbias import check_dbias
    w = synth.custom(mode="gdpa", lq=LQ, lk=LK, H=2, D=128, seed=2, act="gelu_erf", causal=False,
                     window=90, bias_kind="rel", bias_lo=-120, bias_hi=40)
    check_dbias(w, "window 90")
