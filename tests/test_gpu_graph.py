"""The library's calls under HIP graph capture.

Every entry point allocates nothing, records no memset or copy and resets its
scheduler counters inside its own planner kernel, so a forward + backward step
can be captured once and replayed.  Each replay is checked bit for bit against
eager calls on the same inputs (the path is deterministic), with eager library
work and synchronisations between replays, and with new input values copied
into the captured buffers between replays.
"""
import pytest
import torch

from recsys_jagged_attention_gdpa_amd import _lib, synth
from tests.gpu_helpers import announce, to_dev

pytestmark = pytest.mark.gpu


class Step:
    """Static buffers and one forward + backward step through the C ABI."""

    def __init__(self, w, d):
        self.w, self.d = w, d
        self.p = _lib.make_problem(
            batch=w.B, heads=w.H, head_dim=w.D, dtype=w.dtype, total_q=w.total_q,
            total_k=w.total_k, q_offsets=d["q_off"], kv_offsets=d["kv_off"], causal=w.causal,
            scale=w.scale, act=w.act, bias_kind=w.bias_kind, bias_table=d["bias"],
            bias_lo=w.bias_lo, bias_hi=w.bias_hi, window=w.window, rope_base=w.rope_base)
        dev = d["q"].device
        self.o = torch.empty_like(d["q"])
        self.lse = torch.empty((w.H, w.total_q), dtype=torch.float32, device=dev)
        self.o_res = torch.empty_like(self.o) if w.mode == "jfa" else None
        self.dq, self.dk, self.dv = (torch.empty_like(d[n]) for n in ("q", "k", "v"))
        self.db = torch.empty_like(d["bias"]) if d["bias"] is not None else None
        pass_b = _lib.PASS_BWD_DBIAS if self.db is not None else _lib.PASS_BWD
        self.ws_f = torch.empty(_lib.ja_workspace_size(self.p, _lib.PASS_FWD), dtype=torch.uint8, device=dev)
        self.ws_b = torch.empty(_lib.ja_workspace_size(self.p, pass_b), dtype=torch.uint8, device=dev)

    def run(self):
        d, p = self.d, self.p
        if self.w.mode == "gdpa":
            _lib.jagged_gdpa_fwd(p, d["q"], d["k"], d["v"], self.o, self.ws_f)
            _lib.jagged_gdpa_bwd(p, d["q"], d["k"], d["v"], d["dout"], self.dq, self.dk, self.dv, self.db,
                                 self.ws_b)
        else:
            _lib.jagged_attn_fwd(p, d["q"], d["k"], d["v"], self.o, self.lse, self.o_res, self.ws_f)
            _lib.jagged_attn_bwd(p, d["q"], d["k"], d["v"], self.o, self.o_res, d["dout"], self.lse, self.dq,
                                 self.dk, self.dv, self.db, self.ws_b)

    def outputs(self):
        out = [self.o, self.dq, self.dk, self.dv]
        if self.w.mode == "jfa":
            out += [self.lse, self.o_res]
        if self.db is not None:
            out.append(self.db)
        return [t.clone() for t in out]


CASES = [
    dict(mode="gdpa", act="gelu_erf", bias_kind="rel", bias_lo=-40, bias_hi=40, rope_base=10000.0),
    dict(mode="jfa", causal=True, window=50),
    dict(mode="jfa", bias_kind="keypos", bias_lo=0, bias_hi=300, rope_base=500.0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_captured_step_replays_match_eager(case):
    kw = CASES[case]
    # short (<= 32 keys) and long samples, empty samples, ragged tails
    w = synth.custom(lq=[1, 70, 300, 0, 129, 5, 260, 33], lk=[32, 1, 17, 0, 300, 65, 129, 500], H=2,
                     D=128, seed=31 + case, **kw)
    announce(f"graph capture case {case}: {kw}")
    d = to_dev(w)
    step = Step(w, d)
    step.run()
    torch.cuda.synchronize()
    eager = step.outputs()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step.run()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in (step.o, step.dq, step.dk, step.dv):  # the replay must write every element
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = step.outputs()
        for a, b in zip(got, eager):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        step.run()  # eager library work between replays
        torch.cuda.synchronize()

    # new input values in the captured buffers: replays read them
    gen = torch.Generator(device="cpu").manual_seed(5)
    for n in ("q", "k", "v", "dout"):
        d[n].copy_(torch.randn(d[n].shape, generator=gen).to(d[n].dtype))
    step.run()
    torch.cuda.synchronize()
    eager2 = step.outputs()
    assert not torch.equal(eager2[0], eager[0])
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(step.outputs(), eager2):
            assert torch.equal(a, b), f"replay {rep} on new inputs differs from the eager step"


@pytest.mark.parametrize("mode", ["gdpa", "jfa"])
def test_captured_mxfp8_forward_replays_match_eager(mode):
    w = synth.custom(mode=mode, lq=[1, 70, 300, 0, 129, 5, 260, 33], lk=[32, 1, 17, 0, 300, 65, 129, 500], H=2,
                     D=128, seed=41, act="gelu_erf", causal=(mode == "jfa"), with_dout=False,
                     mx=("q", "k", "v"))
    announce(f"graph capture mxfp8 forward {mode}")
    d = to_dev(w)
    p = _lib.make_problem(batch=w.B, heads=w.H, head_dim=w.D, dtype=torch.bfloat16, total_q=w.total_q,
                          total_k=w.total_k, q_offsets=d["q_off"], kv_offsets=d["kv_off"], causal=w.causal,
                          scale=w.scale, act=w.act)
    o = torch.empty((w.total_q, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.H, w.total_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(_lib.ja_workspace_size(p, _lib.PASS_FWD), dtype=torch.uint8, device="cuda")

    def run():
        if mode == "gdpa":
            _lib.jagged_gdpa_fwd_mx(p, d["q"], d["q_sc"], d["k"], d["k_sc"], d["v"], d["v_sc"], o, ws)
        else:
            _lib.jagged_attn_fwd_mx(p, d["q"], d["q_sc"], d["k"], d["k_sc"], d["v"], d["v_sc"], o, lse, None, ws)

    run()
    torch.cuda.synchronize()
    eager = (o.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager[0]), f"replay {rep}: O differs from the eager call"
        if mode == "jfa":
            assert torch.equal(lse, eager[1]), f"replay {rep}: LSE differs from the eager call"
        run()
        torch.cuda.synchronize()
