"""Parity of the HIP path with the fp64 oracle, element by element.

Bar (per row of every output, O, dQ, dK, dV): max |gpu - oracle| <= tau * max |oracle|,
tau = 2e-2 for bf16 inputs with fp32 accumulation and 1e-4 for fp32 inputs; rows the
oracle makes exactly zero must be exactly zero.  JFA's LSE must match to 1e-3.
"""
import numpy as np
import pytest
import torch

from recsys_jagged_attention_gdpa_amd import synth
from tests.gpu_helpers import gpu_bwd, gpu_fwd, parity, to_dev

pytestmark = pytest.mark.gpu


def test_tiny_fp32_workload():
    parity(synth.make("tiny_gdpa_fp32"), label="tiny_gdpa_fp32")


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_asymmetric_with_bias(mode, causal):
    w = synth.custom(mode=mode, lq=[7, 0, 40, 1, 23], lk=[9, 5, 33, 1, 0], H=2, D=32,
                     dtype=torch.float32, seed=3, causal=causal, act="gelu_erf",
                     bias_kind="rel", bias_lo=-6, bias_hi=6)
    parity(w, label=f"fp32 {mode} causal={causal}")


# Lengths that span several 128-row query tiles and 64-row key tiles with ragged
# tails, plus empty and single-row samples and asymmetric lengths.
LQ = [300, 0, 1, 129, 64, 77, 513, 5]
LK = [300, 7, 1, 129, 200, 0, 31, 33]


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("act", ["silu", "gelu_tanh", "gelu_erf"])
def test_gdpa_bf16_acts_and_dims(D, act):
    w = synth.custom(mode="gdpa", lq=LQ, lk=LK, H=2, D=D, seed=D + len(act), act=act,
                     sigma=0.7)
    parity(w, label=f"gdpa D={D} {act}")


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_jfa_bf16_dims(D, causal):
    w = synth.custom(mode="jfa", lq=LQ, lk=LK, H=3, D=D, seed=7 * D, causal=causal)
    parity(w, label=f"jfa D={D} causal={causal}")


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
@pytest.mark.parametrize("bias", ["rel", "keypos"])
@pytest.mark.parametrize("causal", [False, True])
def test_bias_kinds(mode, bias, causal):
    lo, hi = (-40, 40) if bias == "rel" else (0, 150)
    w = synth.custom(mode=mode, lq=[250, 3, 64, 130], lk=[250, 40, 180, 16], H=2, D=64,
                     seed=11, causal=causal, act="gelu_erf", bias_kind=bias, bias_lo=lo,
                     bias_hi=hi, bias_sigma=0.3)
    parity(w, label=f"{mode} bias={bias} causal={causal}")


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
def test_shared_query_block_forward(mode):
    w = synth.custom(mode=mode, lq=None, lk=[300, 0, 1, 64, 65, 129, 17], H=4, D=64, seed=5,
                     shared_q=16, act="silu", bias_kind="keypos", bias_lo=0, bias_hi=255,
                     with_dout=False)
    parity(w, backward=False, label=f"shared-q {mode}")


@pytest.mark.parametrize("lk", [1, 17, 31, 32, 33])
def test_short_kv_backward_paths(lk):
    # lk <= 32 takes the fused short-K/V unit, lk > 32 the split dK/dV + dQ units.
    lq = [1, 70, 300, 0, 129]
    w = synth.custom(mode="gdpa", lq=lq, lk=[lk] * len(lq), H=2, D=128, seed=lk,
                     act="gelu_tanh", sigma=0.7)
    parity(w, label=f"short-kv lk={lk}")
    w = synth.custom(mode="jfa", lq=lq, lk=[lk] * len(lq), H=2, D=128, seed=lk + 1)
    parity(w, label=f"short-kv jfa lk={lk}")


@pytest.mark.parametrize("name,B,max_len", [
    ("gdpa_xattn_short_kv", 48, 700),
    ("jfa_causal_self", 6, 900),
    ("pma_gdpa_fwd", 64, 1500),
    ("longtail_gdpa", 5, 1200),
])
def test_scaled_down_workloads(name, B, max_len):
    w = synth.make(name, B=B, max_len=max_len)
    parity(w, label=f"{name} scaled B={B} max_len={max_len}")


def test_deterministic_run_to_run():
    from tests.gpu_helpers import gpu_bwd, gpu_fwd, to_dev
    w = synth.custom(mode="jfa", lq=LQ, lk=LK, H=2, D=128, seed=1, causal=True)
    d = to_dev(w)
    a, b = gpu_fwd(w, d), gpu_fwd(w, d)
    ga, gb = gpu_bwd(w, d, a), gpu_bwd(w, d, b)
    for n in ("o", "lse"):
        assert torch.equal(a[n], b[n]), n
    for n in ("dq", "dk", "dv"):
        assert torch.equal(ga[n], gb[n]), n


@pytest.mark.parametrize("causal", [False, True])
def test_jfa_backward_without_residual_is_exact_backward_of_bf16_output(causal):
    # Without the forward's rounding residual, delta = <dO, O> uses the bf16 O the
    # caller passes.  The GPU must then match, row by row, the exact fp64 backward
    # in which only delta is formed from that same bf16 O.
    from tests.gpu_helpers import gpu_bwd, gpu_fwd, np64, to_dev
    from tests.helpers import row_check, softmax_cancel_rows, structural_zero_rows
    w = synth.custom(mode="jfa", lq=[300, 1, 77, 129], lk=[300, 1, 40, 200], H=2, D=128, seed=9,
                     causal=causal)
    d = to_dev(w)
    f = gpu_fwd(w, d, residual=False)
    assert f["o_res"] is None
    g = gpu_bwd(w, d, f)
    o_gpu = f["o"].double().cpu()
    want = {n: np.zeros((t, w.H, w.D)) for n, t in (("dq", w.total_q), ("dk", w.total_k), ("dv", w.total_k))}
    # rounding-noise scales of this interface's own terms (see ref.bwd_noise): bf16 dX
    # operands, and delta formed in fp32 on the GPU from the bf16 O both sides use
    noise = {"dq": np.zeros((w.total_q, w.H)), "dk": np.zeros((w.total_k, w.H))}
    for b in range(w.B):
        q0, q1 = int(w.q_off[b]), int(w.q_off[b + 1])
        k0, k1 = int(w.kv_off[b]), int(w.kv_off[b + 1])
        lq, lk = q1 - q0, k1 - k0
        if lq == 0 or lk == 0:
            continue
        q = w.q[q0:q1].double().permute(1, 0, 2)
        k, v = (t[k0:k1].double().permute(1, 0, 2) for t in (w.k, w.v))
        do = w.dout[q0:q1].double().permute(1, 0, 2)
        i, j = torch.arange(lq).view(-1, 1), torch.arange(lk).view(1, -1)
        ok = (j <= i + lk - lq) if causal else torch.ones(lq, lk, dtype=torch.bool)
        x = (w.scale * q @ k.transpose(-1, -2)).masked_fill(~ok, float("-inf"))
        rows = ok.any(-1).view(1, -1, 1)
        p = torch.where(rows, torch.softmax(torch.where(rows, x, torch.zeros_like(x)), -1), torch.zeros_like(x))
        p = p * ok
        delta = (do * o_gpu[q0:q1].permute(1, 0, 2)).sum(-1, keepdim=True)
        ds = p * (do @ v.transpose(-1, -2) - delta)
        want["dq"][q0:q1] = (w.scale * ds @ k).permute(1, 0, 2).numpy()
        want["dk"][k0:k1] = (w.scale * ds.transpose(-1, -2) @ q).permute(1, 0, 2).numpy()
        want["dv"][k0:k1] = (p.transpose(-1, -2) @ do).permute(1, 0, 2).numpy()
        oabs = (do.abs() * o_gpu[q0:q1].permute(1, 0, 2).abs()).sum(-1, keepdim=True)  # [H, lq, 1]
        u_dx, u_dl = 2.0 ** -8, 2.0 ** -22
        nq = u_dx * w.scale * ((ds ** 2) @ (k ** 2)).sqrt().amax(-1) + \
            u_dl * w.scale * oabs[..., 0] * (p @ k.abs()).amax(-1)
        nk = u_dx * w.scale * ((ds ** 2).transpose(-1, -2) @ (q ** 2)).sqrt().amax(-1) + \
            u_dl * w.scale * ((p * oabs).transpose(-1, -2) @ q.abs()).amax(-1)
        noise["dq"][q0:q1] = nq.T.numpy()
        noise["dk"][k0:k1] = nk.T.numpy()
    cq, ck = softmax_cancel_rows(w)
    _, zq, zk = structural_zero_rows(w)
    for n, nz, c, z in (("dq", noise["dq"], cq, zq), ("dk", noise["dk"], ck, zk), ("dv", None, None, zk)):
        row_check(np64(g[n]), want[n], 2e-2, f"no-residual {n}", noise=nz, cancel_rows=c, zero_rows=z)


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
@pytest.mark.parametrize("rows,D,causal", [(1, 32, False), (32, 128, False), (33, 64, False), (20, 128, True),
                                           (16, 64, True), (9, 128, False)])
def test_shared_query_block_sizes(mode, rows, D, causal):
    # Up to 32 shared rows run as one-wave units over 32-row tiles (GDPA with at
    # most 16: the two key blocks' rows packed into one block's lanes); 33 rows
    # take the 4-wave path.  Samples with <= 32 keys go to the short-K/V units.
    w = synth.custom(mode=mode, lq=None, lk=[700, 0, 1, 31, 32, 33, 96, 257], H=2, D=D, seed=rows + D,
                     shared_q=rows, act="gelu_erf", causal=causal, bias_kind="rel", bias_lo=-50,
                     bias_hi=40, bias_sigma=0.3, with_dout=False)
    parity(w, backward=False, label=f"shared-q {mode} rows={rows} D={D} causal={causal}")


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
@pytest.mark.parametrize("lq,lk", [([0, 0, 0], [0, 0, 0]), ([0, 0], [0, 40]), ([3, 70, 0], [0, 0, 0]),
                                   ([5, 200], [0, 0])])
def test_empty_batches_and_keyless_rows(mode, lq, lk):
    # Nothing to compute (no pairs at all): every output row is exactly zero
    # (JFA: LSE = -inf), including rows that exist but see no key.
    w = synth.custom(mode=mode, lq=lq, lk=lk, H=2, D=64, seed=2)
    parity(w, label=f"empty {mode} lq={lq} lk={lk}")


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
@pytest.mark.parametrize("H,D,scale", [(1, 32, 0.3), (16, 64, None), (5, 128, 0.05)])
def test_head_counts_and_explicit_scale(mode, H, D, scale):
    w = synth.custom(mode=mode, lq=[150, 1, 40, 33], lk=[90, 300, 32, 65], H=H, D=D, seed=H * D, scale=scale,
                     act="silu", causal=True)
    parity(w, label=f"{mode} H={H} D={D} scale={scale}")


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
@pytest.mark.parametrize("hint", [32, 33])
def test_key_count_bound_hint(mode, hint):
    # Every sample has at most 32 keys.  A bound of at most 32 leaves the
    # long-sequence kernels unlaunched; the results must not change (the same
    # short-K/V units compute every output either way).
    lq, lk = [1, 70, 300, 0, 129, 5, 2], [32, 1, 17, 0, 31, 32, 0]
    w = synth.custom(mode=mode, lq=lq, lk=lk, H=2, D=128, seed=hint, act="gelu_erf", causal=True,
                     bias_kind="rel", bias_lo=-40, bias_hi=10, bias_sigma=0.3)
    parity(w, label=f"hint {mode} max_kv_len={hint}", max_kv_len=hint)
    d = to_dev(w)
    base = gpu_fwd(w, d)
    d["max_kv_len"] = hint
    hinted = gpu_fwd(w, d)
    for n in base:
        if base[n] is not None:
            assert torch.equal(base[n], hinted[n]), n
    gb, gh = gpu_bwd(w, {**d, "max_kv_len": 0}, base), gpu_bwd(w, d, hinted)
    for n in ("dq", "dk", "dv"):
        assert torch.equal(gb[n], gh[n]), n


def test_key_count_bound_hint_shared_queries():
    w = synth.custom(mode="gdpa", lq=None, lk=[32, 0, 1, 31, 17], H=2, D=64, seed=9, shared_q=16,
                     act="silu", with_dout=False)
    parity(w, backward=False, label="hint shared-q", max_kv_len=32)
