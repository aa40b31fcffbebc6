"""Pin the oracle's rotary position embedding.

The pages name a rotary embedding fused into their block-attention kernel
("Meta redesigns AI training infrastructure...", section "Custom Kernels and
5D Parallelism for Trillion-Parameter Scale") but do not define it; the reading
is RoFormer's rotation in split-half form: element d < D/2 and element d + D/2
of a row at sample-local position t turn by the angle t * base^(-2d/D).  The
checks below are fixed by that definition's consequences, not by re-typing it:
  * closed forms: with unit-vector queries and keys the score is
    scale * cos((i - j) theta_d) (same pair element) or scale * sin((i - j) theta_d)
    (partner element), read back through one-hot values;
  * relative positions: prefixing a sample with zero rows shifts every position
    and changes no output row (GDPA, act(0) = 0);
  * positions are sample-local: a jagged batch equals each sample alone;
  * position 0 is the identity: one-row samples are bitwise the unrotated result;
  * gradients: central differences of <O, dO>, and padded dense attention in
    complex form with torch autograd;
  * the turn alone keeps every pair's length; its bf16 variant (turned rows of
    bf16 operands) is the nearest bf16 value of the exact turn, ties to even,
    checked against that definition (within half a bf16 step, even on ties, on
    constructed midpoints and subnormals); attention with that variant equals
    plain attention of the rounded rows.
"""
import math

import numpy as np
import pytest
import torch

from oracle import ref
from recsys_jagged_attention_gdpa_amd import synth
from tests.dense_ref import dense
from tests.helpers import max_rel, oracle_bwd, oracle_dbias, oracle_fwd

BASE = 10000.0


def _one_sample(q, k, v, *, mode="gdpa", act="silu", scale=1.0, rope_base=BASE, causal=False):
    lq, lk = q.shape[0], k.shape[0]
    w = synth.custom(mode=mode, lq=[lq], lk=[lk], H=1, D=q.shape[-1], dtype=torch.float32,
                     act=act, scale=scale, causal=causal, rope_base=rope_base)
    return synth.Workload(**{**w.__dict__, "q": q, "k": k, "v": v})


@pytest.mark.parametrize("D,d", [(8, 0), (8, 3), (32, 1), (32, 15), (64, 20), (128, 63)])
@pytest.mark.parametrize("partner", [False, True])
def test_unit_vector_scores_are_cos_and_sin_of_the_position_difference(D, d, partner):
    """q_i = a e_d, k_j = b e_d (or e_{d + D/2}): X_ij = scale a b cos((i - j) theta_d)
    (or scale a b sin((i - j) theta_d)), theta_d = base^(-2d/D).  With one-hot values
    v_j = e_j the GDPA output row i holds act(X_ij) at column j."""
    Lq, Lk, a, b, scale = 7, 6, 1.5, 0.75, 0.9
    q = torch.zeros(Lq, 1, D)
    q[:, 0, d] = a
    k = torch.zeros(Lk, 1, D)
    k[:, 0, d + D // 2 if partner else d] = b
    v = torch.zeros(Lk, 1, D)
    for j in range(Lk):
        v[j, 0, j] = 1.0
    w = _one_sample(q, k, v, act="silu", scale=scale)
    o = oracle_fwd(w)["o"]
    theta = BASE ** (-2.0 * d / D)
    for i in range(Lq):
        for j in range(Lk):
            ang = (i - j) * theta
            x = scale * a * b * (math.sin(ang) if partner else math.cos(ang))
            want = x / (1.0 + math.exp(-x))
            assert abs(o[i, 0, j] - want) <= 1e-13, (i, j, o[i, 0, j], want)


def test_partner_sign_fixes_the_turn_direction():
    """A turn by +angle of a query at position 1 against the key at position 0: the
    score of e_0 against e_{D/2} is +sin(theta_0) = +sin(1)."""
    D = 8
    q = torch.zeros(2, 1, D)
    q[1, 0, 0] = 1.0
    k = torch.zeros(1, 1, D)
    k[0, 0, D // 2] = 1.0
    v = torch.ones(1, 1, D)
    w = _one_sample(q, k, v, mode="jfa", causal=False)
    # JFA with one key: LSE is the score itself
    lse = oracle_fwd(w)["lse"]
    assert abs(lse[1, 0] - math.sin(1.0)) <= 1e-15
    assert lse[0, 0] == 0.0


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
def test_one_row_samples_are_the_unrotated_result_bitwise(mode):
    w = synth.custom(mode=mode, lq=[1, 1, 1], lk=[1, 1, 1], H=2, D=32, dtype=torch.float32,
                     seed=5, rope_base=BASE)
    plain = synth.Workload(**{**w.__dict__, "rope_base": 0.0})
    a, b = oracle_fwd(w), oracle_fwd(plain)
    assert np.array_equal(a["o"], b["o"])
    ga, gb = oracle_bwd(w), oracle_bwd(plain)
    for n in ("dq", "dk", "dv"):
        assert np.array_equal(ga[n], gb[n]), n


@pytest.mark.parametrize("act", ["silu", "gelu_tanh", "gelu_erf"])
def test_zero_prefix_shifts_positions_and_changes_nothing(act):
    """GDPA depends on positions only through i - j: n zero rows in front of the
    sample's queries, keys and values shift every position by n, the zero keys add
    act(0) v = 0, and rows n.. of the longer sample equal the original rows."""
    g = torch.Generator().manual_seed(3)
    L, n, D = 23, 9, 32
    q, k, v = (torch.randn(L, 2, D, generator=g) for _ in range(3))
    z = torch.zeros(n, 2, D)
    w1 = synth.custom(mode="gdpa", lq=[L], H=2, D=D, dtype=torch.float32, act=act, rope_base=BASE)
    w1 = synth.Workload(**{**w1.__dict__, "q": q, "k": k, "v": v})
    w2 = synth.custom(mode="gdpa", lq=[L + n], H=2, D=D, dtype=torch.float32, act=act,
                      rope_base=BASE)
    w2 = synth.Workload(**{**w2.__dict__, "q": torch.cat([z, q]), "k": torch.cat([z, k]),
                           "v": torch.cat([z, v])})
    o1, o2 = oracle_fwd(w1)["o"], oracle_fwd(w2)["o"]
    assert max_rel(o2[n:], o1) <= 1e-12
    # the rotation is not the identity here
    plain = oracle_fwd(synth.Workload(**{**w1.__dict__, "rope_base": 0.0}))["o"]
    assert max_rel(plain, o1) > 1e-2


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
def test_positions_are_sample_local(mode):
    """Samples with different query and key offsets: each equals itself run alone."""
    w = synth.custom(mode=mode, lq=[5, 17, 0, 30], lk=[12, 3, 8, 30], H=2, D=32,
                     dtype=torch.float32, seed=8, rope_base=BASE, causal=(mode == "jfa"))
    full = oracle_fwd(w)
    fb = oracle_bwd(w)
    for b in range(w.B):
        alone = w.subset([b])
        fa, ga = oracle_fwd(alone), oracle_bwd(alone)
        q0, q1 = int(w.q_off[b]), int(w.q_off[b + 1])
        k0, k1 = int(w.kv_off[b]), int(w.kv_off[b + 1])
        assert np.array_equal(full["o"][q0:q1], fa["o"])
        assert np.array_equal(fb["dq"][q0:q1], ga["dq"])
        assert np.array_equal(fb["dk"][k0:k1], ga["dk"])


def _loss(w, q, k, v):
    w2 = synth.Workload(**{**w.__dict__, "q": q, "k": k, "v": v})
    return float((oracle_fwd(w2)["o"] * w.dout.double().numpy()).sum())


@pytest.mark.parametrize("mode,act,causal,bias", [
    ("gdpa", "silu", False, "none"), ("gdpa", "gelu_tanh", True, "rel"), ("jfa", "silu", True, "none"),
    ("jfa", "silu", False, "keypos")])
def test_rope_gradients_match_central_differences(mode, act, causal, bias):
    w = synth.custom(mode=mode, lq=[9, 4, 13], lk=[9, 7, 13], H=2, D=16, dtype=torch.bfloat16,
                     seed=21, act=act, causal=causal, bias_kind=bias,
                     bias_lo=-3 if bias == "rel" else 0, bias_hi=5, rope_base=100.0)
    # bf16-valued inputs held in float32, so x +- 2^-14 is exact in float32.
    # (held as float32 inputs: the exact turn, no bf16 rounding of the turned rows)
    q, k, v = (t.float() for t in (w.q, w.k, w.v))
    w = synth.Workload(**{**w.__dict__, "q": q, "k": k, "v": v, "dout": w.dout.float(),
                          "dtype": torch.float32})
    g = oracle_bwd(w)
    rng = np.random.default_rng(7)
    h = 2.0 ** -14
    for name, base in (("dq", q), ("dk", k), ("dv", v)):
        for _ in range(2):
            d = torch.from_numpy(rng.integers(-1, 2, size=tuple(base.shape)).astype(np.float32) * h)
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name[1]] = base + d
            args_m[name[1]] = base - d
            fd = (_loss(w, **args_p) - _loss(w, **args_m)) / 2.0
            an = float((g[name] * d.double().numpy()).sum())
            assert abs(fd - an) <= 1e-7 * max(abs(an), 1e-3), (name, fd, an)


@pytest.mark.parametrize("seed", range(12))
def test_rope_matches_dense_complex_form(seed):
    rng = np.random.default_rng(500 + seed)
    B = int(rng.integers(1, 5))
    D = [16, 32, 64, 128][seed % 4]
    mode = "jfa" if seed % 2 else "gdpa"
    lq = rng.integers(0, 30, size=B)
    lk = rng.integers(0, 30, size=B) if seed % 3 == 0 else lq.copy()
    bias = ["none", "rel", "keypos"][seed % 3]
    w = synth.custom(mode=mode, lq=lq, lk=lk, H=2, D=D, dtype=torch.float32, seed=seed,
                     act=["silu", "gelu_tanh", "gelu_erf"][seed % 3], causal=bool(seed % 4 == 1),
                     bias_kind=bias, bias_lo=-5 if bias == "rel" else 0, bias_hi=11,
                     window=3 if seed % 5 == 2 else 0, rope_base=[10000.0, 500.0, 1e6][seed % 3])
    want = dense(w)
    got = {**oracle_fwd(w), **oracle_bwd(w)}
    for n in ("o", "dq", "dk", "dv"):
        assert max_rel(got[n], want[n]) <= 1e-12, n
    if bias != "none":
        assert max_rel(oracle_dbias(w), want["dbias"]) <= 1e-12


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
def test_rope_shared_query_block_matches_dense(mode):
    w = synth.custom(mode=mode, lq=None, lk=[3, 20, 0, 9], H=2, D=32, dtype=torch.float32,
                     seed=4, shared_q=6, with_dout=False, rope_base=BASE)
    want = dense(w, grads=False)
    assert max_rel(oracle_fwd(w)["o"], want["o"]) <= 1e-12


def _jagged(seed, D=64, H=3):
    w = synth.custom(mode="gdpa", lq=[40, 0, 1, 300, 17], lk=[5, 9, 1, 300, 2000], H=H, D=D,
                     dtype=torch.bfloat16, seed=seed, rope_base=BASE)
    return w


@pytest.mark.parametrize("D", [32, 128])
def test_turn_keeps_pair_lengths_and_position_zero(D):
    w = _jagged(1, D=D)
    x = w.k.float().numpy().astype(np.float64)
    y = ref.rope(w.k, w.kv_off, rope_base=BASE)
    h = D // 2
    assert np.allclose(y[..., :h] ** 2 + y[..., h:] ** 2, x[..., :h] ** 2 + x[..., h:] ** 2,
                       rtol=1e-13, atol=1e-13)
    starts = w.kv_off[:-1][np.diff(w.kv_off) > 0]
    assert np.array_equal(y[starts], x[starts])  # position 0 of every sample
    assert not np.array_equal(y, x)


def _bf16_step(x):
    """The spacing of bf16 values at |x| (8 significant bits; below 2^-126 a fixed
    2^-133)."""
    e = np.frexp(np.abs(x))[1]  # 2^(e-1) <= |x| < 2^e
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def test_bf16_turn_is_the_rounded_exact_turn():
    """Each element of the bf16 variant is the bf16 value nearest to the exact turn
    (ties to even): a bf16 value, within half a bf16 step of the exact turn, and on
    an exact tie the one with an even last significand bit."""
    w = _jagged(2, D=128)
    ex = ref.rope(w.k, w.kv_off, rope_base=BASE)
    rd = ref.rope(w.k, w.kv_off, rope_base=BASE, rope_bf16=True)
    # bf16 values: float32 with the low 16 bits clear
    bits = rd.astype(np.float32).view(np.uint32)
    assert np.array_equal(rd.astype(np.float32).astype(np.float64), rd)
    assert not (bits & 0xFFFF).any()
    step = _bf16_step(ex)
    err = np.abs(rd - ex)
    assert (err <= 0.5 * step).all(), float((err / step).max())
    tie = err == 0.5 * step
    assert not ((bits[tie] >> 16) & 1).any()
    # a nearest-value rounding, not a truncation: about half the elements rounded up
    up = (np.abs(rd) > np.abs(ex)).mean()
    assert 0.4 < up < 0.6, up
    # torch's double -> bf16 cast rounds through float32 first, which moves a value by up
    # to half a float32 step (2^-17 of a bf16 step); away from bf16 midpoints by more than
    # that the two agree
    mid = np.abs(err - 0.5 * step) <= 2.0 ** -16 * step
    rne = torch.from_numpy(ex).to(torch.bfloat16).double().numpy()
    assert np.array_equal(rd[~mid], rne[~mid])


def test_bf16_nearest_on_constructed_values():
    """Rounding of float32 values placed on and beside bf16 midpoints and in the
    subnormal range.  Position 0 turns by a zero angle, so one-row samples give the
    bf16 variant of the rows themselves."""
    odd = 1.0 + 2.0 ** -7  # a bf16 value whose last significand bit is odd
    cases = [(1.0 + 2.0 ** -8, 1.0),                    # tie between 1 and odd: to the even 1
             (odd + 2.0 ** -8, 1.0 + 2.0 ** -6),        # tie between odd and 1 + 2^-6: up, to even
             (1.0 + 2.0 ** -8 + 2.0 ** -20, odd),       # just above the tie: up
             (-(1.0 + 2.0 ** -8 - 2.0 ** -20), -1.0),   # just below the tie, negative: to -1
             (3.0 * 2.0 ** -134, 2.0 ** -132),          # subnormal, 1.5 steps of 2^-133: tie, to even 2
             (2.0 ** -135, 0.0)]                        # a quarter of the subnormal step: to 0
    vals = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases])
    assert np.array_equal(vals.astype(np.float32).astype(np.float64), vals)
    x = torch.from_numpy(vals.astype(np.float32)).view(-1, 1, 1).repeat(1, 1, 2)
    off = np.arange(x.shape[0] + 1, dtype=np.int32)  # one-row samples: position 0
    rd = ref.rope(x, off, rope_base=BASE, rope_bf16=True)
    assert np.array_equal(rd[:, 0, 0], want), rd[:, 0, 0]
    assert np.array_equal(rd[:, 0, 1], want), rd[:, 0, 1]


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
def test_bf16_turn_feeds_attention_as_plain_rows(mode):
    w = synth.custom(mode=mode, lq=[40, 0, 1, 130], lk=[5, 9, 1, 130], H=2, D=64,
                     dtype=torch.bfloat16, seed=3, rope_base=BASE, causal=(mode == "jfa"))
    qr = torch.from_numpy(ref.rope(w.q, w.q_off, rope_base=BASE, rope_bf16=True)).float()
    kr = torch.from_numpy(ref.rope(w.k, w.kv_off, rope_base=BASE, rope_bf16=True)).float()
    plain = synth.Workload(**{**w.__dict__, "q": qr, "k": kr, "rope_base": 0.0})
    a, b = oracle_fwd(w), oracle_fwd(plain)
    assert np.array_equal(a["o"], b["o"])
    # and the rounding matters on some row (against the exact turn)
    exact = oracle_fwd(synth.Workload(**{**w.__dict__, "dtype": torch.float32}))
    assert not np.array_equal(a["o"], exact["o"])
