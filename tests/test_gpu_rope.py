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


def _turned_rows_match(got, want64, what):
    """GPU turned rows against the oracle's: the same value in every element but for
    at most one in a million, and those one unit in the last place apart (the two
    sides' fp64 sine and cosine may differ in their last bit)."""
    g = got.cpu()
    if g.dtype == torch.bfloat16:
        w = torch.from_numpy(want64).float().to(torch.bfloat16)  # exact: already bf16 values
        gi, wi = g.view(torch.int16).int(), w.view(torch.int16).int()
    else:
        w = torch.from_numpy(want64).float()  # nearest float32 of the fp64 turn
        gi, wi = g.view(torch.int32).long(), w.view(torch.int32).long()
    diff = (gi - wi).abs()
    n_bad = int((diff != 0).sum())
    assert n_bad <= max(1, g.numel() // 1_000_000) and int(diff.max()) <= 1, (what, n_bad, int(diff.max()))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_rope_call_turns_rows_as_the_oracle(dtype):
    from oracle import ref
    import recsys_jagged_attention_gdpa_amd as ja
    w = synth.custom(mode="jfa", lq=LQ, lk=LK, H=3, D=64, seed=21, dtype=dtype, rope_base=10000.0)
    announce(f"rope call {dtype}: Tq={w.total_q} Tk={w.total_k}")
    d = to_dev(w)
    qt, kt = ja.rope(d["q"], d["k"], d["q_off"], d["kv_off"], rope_base=w.rope_base)
    torch.cuda.synchronize()
    bf = dtype == torch.bfloat16
    _turned_rows_match(qt, ref.rope(w.q, w.q_off, rope_base=w.rope_base, rope_bf16=bf), "q")
    _turned_rows_match(kt, ref.rope(w.k, w.kv_off, rope_base=w.rope_base, rope_bf16=bf), "k")
    # in place gives the same rows
    q2, k2 = d["q"].clone(), d["k"].clone()
    ja.rope(q2, k2, d["q_off"], d["kv_off"], rope_base=w.rope_base, out=(q2, k2))
    torch.cuda.synchronize()
    assert torch.equal(q2, qt) and torch.equal(k2, kt)


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_pre_turned_inputs_give_the_same_results(mode, dtype):
    """Turning once with the rope call and passing the turned rows to the forward and
    the backward gives, bit for bit, what the calls that turn q and k themselves give."""
    import recsys_jagged_attention_gdpa_amd as ja
    w = synth.custom(mode=mode, lq=LQ, lk=LK, H=2, D=128 if dtype == torch.bfloat16 else 32, seed=8,
                     dtype=dtype, act="gelu_tanh", causal=True, rope_base=10000.0)
    announce(f"rope pre-turned {mode} {dtype}")
    d = to_dev(w)
    f = gpu_fwd(w, d)
    g = gpu_bwd(w, d, f)
    qt, kt = ja.rope(d["q"], d["k"], d["q_off"], d["kv_off"], rope_base=w.rope_base)
    kw = dict(scale=w.scale, causal=w.causal, rope_base=w.rope_base, rope_inputs_turned=True)
    if mode == "gdpa":
        o = ja.gdpa_forward(qt, kt, d["v"], d["q_off"], d["kv_off"], act=w.act, **kw)
        dq, dk, dv = ja.gdpa_backward(qt, kt, d["v"], d["dout"], d["q_off"], d["kv_off"], act=w.act, **kw)
        f2 = {"o": o}
    else:
        o, lse, o_res = ja.attn_forward(qt, kt, d["v"], d["q_off"], d["kv_off"], **kw)
        dq, dk, dv = ja.attn_backward(qt, kt, d["v"], o, d["dout"], lse, d["q_off"], d["kv_off"],
                                      o_residual=o_res, **kw)
        f2 = {"o": o, "lse": lse, "o_res": o_res}
    torch.cuda.synchronize()
    for n, t in f.items():
        if t is not None:
            assert torch.equal(f2[n], t), n
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.equal(t, g[n]), n


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
def test_autograd_turns_once_and_matches_the_direct_calls(mode):
    import recsys_jagged_attention_gdpa_amd as ja
    w = synth.custom(mode=mode, lq=LQ, lk=LK, H=2, D=64, seed=15, act="silu", causal=True,
                     rope_base=10000.0)
    announce(f"rope autograd {mode}")
    d = to_dev(w)
    f = gpu_fwd(w, d)
    g = gpu_bwd(w, d, f)
    q, k, v = (d[n].clone().requires_grad_() for n in ("q", "k", "v"))
    if mode == "gdpa":
        o = ja.gdpa(q, k, v, d["q_off"], d["kv_off"], act=w.act, scale=w.scale, causal=w.causal,
                    rope_base=w.rope_base)
    else:
        o = ja.jagged_attention(q, k, v, d["q_off"], d["kv_off"], scale=w.scale, causal=w.causal,
                                rope_base=w.rope_base)
    o.backward(d["dout"])
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), f["o"])
    for n, t in (("dq", q.grad), ("dk", k.grad), ("dv", v.grad)):
        assert torch.equal(t, g[n]), n
