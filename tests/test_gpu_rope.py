"""Rotary position embedding on the HIP path against the fp64 oracle.

q and k rows are turned by the angle t * base^(-2d/D) of their sample-local
position t (pairs d, d + D/2) before the scores; gradients are returned with
respect to the rows as given.  Same per-row bar as the other parity tests
(tau = 2e-2 bf16, 1e-4 fp32; rows with no visible key exactly zero).
"""
import pytest
import torch

from recsys_jagged_attention_gdpa_amd import synth
from tests.gpu_helpers import announce, gpu_bwd, gpu_fwd, parity, to_dev

pytestmark = pytest.mark.gpu

# short (<= 32 keys) and long samples, Lq != Lk, empty samples, ragged tails,
# positions into the thousands
LQ = [1, 70, 300, 0, 129, 5, 40, 260, 33, 2100]
LK = [32, 1, 17, 0, 300, 65, 40, 129, 500, 2100]


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_rope_matches_oracle(mode, causal, D):
    w = synth.custom(mode=mode, lq=LQ, lk=LK, H=2, D=D, seed=D + causal, act="gelu_tanh",
                     causal=causal, rope_base=10000.0)
    parity(w, label=f"rope {mode} causal={causal} D={D}")


@pytest.mark.parametrize("mode,bias,base", [("gdpa", "rel", 500.0), ("jfa", "keypos", 1e6),
                                            ("gdpa", "keypos", 10000.0)])
def test_rope_with_bias_window_and_bases(mode, bias, base):
    w = synth.custom(mode=mode, lq=[600, 31, 128, 1], lk=[600, 31, 200, 3], H=3, D=64, seed=9,
                     act="gelu_erf", causal=True, window=150 if mode == "jfa" else 0, bias_kind=bias,
                     bias_lo=-60 if bias == "rel" else 0, bias_hi=60 if bias == "rel" else 300,
                     rope_base=base)
    parity(w, label=f"rope {mode} bias={bias} base={base}")


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
def test_rope_shared_queries_and_fp32(mode):
    w = synth.custom(mode=mode, lq=None, lk=[700, 0, 1, 31, 33, 257], H=2, D=64, seed=3, shared_q=24,
                     act="silu", with_dout=False, rope_base=10000.0)
    parity(w, backward=False, label=f"rope shared-q {mode}")
    w = synth.custom(mode=mode, lq=[9, 0, 23, 1, 17, 130], lk=[9, 5, 23, 1, 0, 70], H=2, D=32,
                     dtype=torch.float32, seed=4, causal=True, rope_base=10000.0)
    parity(w, label=f"rope fp32 {mode}")


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
def test_rope_one_row_samples_are_bitwise_unrotated(mode):
    """Position 0 turns by angle 0: the turned copies equal the inputs bit for bit,
    and so does every output and gradient."""
    w = synth.custom(mode=mode, lq=[1] * 40, lk=[1] * 40, H=2, D=64, seed=12, act="silu",
                     rope_base=10000.0)
    plain = synth.Workload(**{**w.__dict__, "rope_base": 0.0})
    announce(f"rope position-0 identity {mode}")
    d = to_dev(w)
    a, b = gpu_fwd(w, d), gpu_fwd(plain, d)
    ga, gb = gpu_bwd(w, d, a), gpu_bwd(plain, d, b)
    torch.cuda.synchronize()
    for n in a:
        if a[n] is not None:
            assert torch.equal(a[n], b[n]), n
    for n in ga:
        assert torch.equal(ga[n], gb[n]), n


def test_rope_bias_gradient():
    from tests.test_gpu_dbias import check_dbias
    w = synth.custom(mode="jfa", lq=LQ, lk=LK, H=2, D=128, seed=2, causal=True,
                     bias_kind="rel", bias_lo=-120, bias_hi=40, rope_base=10000.0)
    check_dbias(w, "rope")
