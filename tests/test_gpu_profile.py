"""The scheduler's measurement aid (per-workgroup busy stamps of the persistent
kernels) records without changing any result."""
import pytest
import torch

from recsys_jagged_attention_gdpa_amd import _lib, synth
from tests.gpu_helpers import announce, gpu_bwd, gpu_fwd, to_dev

pytestmark = pytest.mark.gpu

KERNELS = ("fwd", "bwd_kv", "bwd_q")


def _run(w, d):
    f = gpu_fwd(w, d)
    out = dict(f)
    out.update(gpu_bwd(w, d, f))
    torch.cuda.synchronize()
    return out


def test_busy_stamps_fill_one_entry_per_workgroup_and_change_nothing():
    w = synth.make("jfa_causal_self", B=8, max_len=1500)
    announce(f"busy stamps: jfa B={w.B} H={w.H} Tq={w.total_q}")
    d = to_dev(w)
    want = _run(w, d)
    bufs = {k: torch.zeros(4096, dtype=torch.int64, device="cuda") for k in KERNELS}
    try:
        for k in KERNELS:
            _lib.ja_profile_busy(k, bufs[k])
        got = _run(w, d)
    finally:
        for k in KERNELS:
            _lib.ja_profile_busy(k, None)
    for name, t in want.items():
        if t is not None:
            assert torch.equal(got[name], t), name
    for k, b in bufs.items():
        b = b.cpu()
        n = int((b > 0).sum())
        # persistent grid: workgroups 0 .. n-1 each stamped once, the rest untouched
        assert 0 < n < b.numel(), (k, n)
        assert (b[:n] > 0).all() and (b[n:] == 0).all(), k
    # stamps off again: a further call writes nothing
    for b in bufs.values():
        b.zero_()
    _run(w, d)
    assert all(int(b.abs().sum()) == 0 for b in bufs.values())
