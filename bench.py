#!/usr/bin/env python3
"""Throughput of the jagged attention hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
planning, forward and backward (by default JFA causal self-attention over a
jagged batch, B=64, H=8, D=128, lengths uniform in 1..8192: the
sparsity-0.5, MFMA-bound workload the metric names).  Inputs are resident in
HBM before the timed region.  Prints ONE JSON line on stdout; details go to
stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Metric: useful (unpadded) TFLOP/s of forward + backward.  Useful work counts
only valid (query, key) pairs P: forward 4 D P, backward 10 D P (five
GEMM-sized products per pair).  The dominant kernel is also placed on its
roofline (HBM bytes or MFMA FLOPs per launch / its average duration).  Every
kernel's duration comes from HIP events that the library records around its
launches during the timed steps, on the stream it runs on.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from recsys_jagged_attention_gdpa_amd import _lib, synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
KERNEL_SOURCES = ["ja_fwd.hip", "ja_fwd_gdpa.hip", "ja_fwd_mx.hip", "ja_fwd_kernels.h", "ja_bwd.hip",
                  "ja_bwd_kv.hip", "ja_bwd_kernels.h", "ja_dbias_fold.h", "ja_plan.hip", "ja_tiles.h",
                  "ja_device.h", "ja_kernels.h"]

# Workloads: which roofline bounds them (short K/V streams Q / dO / O through HBM;
# long sequences are MFMA work).
BOUND = {"gdpa_xattn_short_kv": "hbm", "pma_gdpa_fwd": "hbm", "jfa_causal_self": "mfma",
         "longtail_gdpa": "mfma", "tiny_gdpa_fp32": "alu", "jfa_swa_causal_self": "mfma",
         "jfa_rope_causal_self": "mfma", "pma_gdpa_fwd_mxfp8": "hbm", "gdpa_xattn_short_kv_mxfp8": "hbm",
         "jfa_causal_self_fwd_mxfp8": "mfma"}
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector (the plain fp32 kernels are ALU loops)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ accounting
def pairs_per_sample(w) -> np.ndarray:
    """Valid (query, key) pairs of each sample (per head)."""
    lq = w.lq.astype(np.int64)
    lk = w.lk.astype(np.int64)
    if not w.causal and not w.window:
        return lq * lk
    out = np.zeros(len(lq), dtype=np.int64)
    for n, (a, b) in enumerate(zip(lq, lk)):
        ia = np.arange(a, dtype=np.int64) + b - a  # aligned positions
        end = np.clip(ia + 1, 0, b) if w.causal else (np.clip(ia + w.window, 0, b) if w.window else b)
        beg = np.clip(ia - w.window + 1, 0, b) if w.window else 0
        out[n] = int(np.maximum(end - beg, 0).sum())
    return out


def valid_pairs(w) -> int:
    """P summed over samples (per head); heads multiply it."""
    return int(pairs_per_sample(w).sum())


SHORT_KV = 32  # samples with at most this many keys go to the short-K/V (fused) units


def kernel_cost(w, kernel: str) -> tuple[float, float]:
    """Algorithmic (bytes, flops) one launch of `kernel` processes for workload w:
    only the samples that kernel handles (bf16: at most SHORT_KV keys -> the
    short / fused units, more -> the tile units; fp32: every sample)."""
    e = w.q.element_size()
    HD = w.H * w.D
    if w.dtype == torch.float32:
        sel = np.ones(w.B, dtype=bool)
    elif kernel in ("fwd_short", "bwd_fused"):
        sel = w.lk <= SHORT_KV
    elif kernel in ("fwd", "bwd_kv", "bwd_q"):
        sel = w.lk > SHORT_KV
    else:
        sel = np.ones(w.B, dtype=bool)
    P = float(pairs_per_sample(w)[sel].sum()) * w.H
    lq = w.lq.astype(np.int64)
    tq_out = tq = int(lq[sel].sum())
    tk = int(w.lk.astype(np.int64)[sel].sum())
    q_rows = tq if w.q_off is not None else w.q.shape[0]  # shared queries are read once
    if kernel in ("fwd", "fwd_short"):
        if w.mx:  # codes (1 byte) and a scale code per 32 elements in; bf16 out
            b = HD * (q_rows + 2 * tk) * (1 + 1 / 32) + 2 * HD * tq_out
        else:
            b = e * HD * (q_rows + tq_out + 2 * tk)
        b += 4 * w.H * tq_out if w.mode == "jfa" else 0
        return b, 4.0 * w.D * P
    if kernel == "bwd_fused":  # read Q, dO, K, V; write dQ, dK, dV; five GEMMs per pair
        return e * HD * (3 * tq + 4 * tk), 10.0 * w.D * P
    if kernel == "bwd_kv":     # read Q, dO, K, V; write dK, dV; four GEMMs per pair
        return e * HD * (2 * tq + 4 * tk), 8.0 * w.D * P
    if kernel == "bwd_q":      # read Q, dO, K, V; write dQ; three GEMMs per pair
        return e * HD * (3 * tq + 2 * tk), 6.0 * w.D * P
    if kernel == "bwd_delta":
        return e * HD * 2 * tq + 4 * w.H * tq, 2.0 * HD * tq
    if kernel == "bwd_dbias":  # read Q, dO, K, V; recompute S and dP (two GEMMs per pair)
        return e * HD * (2 * tq + 2 * tk), 4.0 * w.D * P
    if kernel == "rope":  # read and write every row of q and k
        return e * HD * 2 * (w.q.shape[0] + w.total_k), 0.0
    if kernel == "rope_back":  # bf16: read and write every row of dk; fp32: of dq and dk
        return e * HD * 2 * (w.total_k + (w.q.shape[0] if w.dtype == torch.float32 else 0)), 0.0
    return 0.0, 0.0


# ------------------------------------------------------------------ HIP events
class HipEvents:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
        self.made.append(ev)
        return ev

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        assert rc == 0, rc
        return float(ms.value)

    def close(self):
        for ev in self.made:
            self.hip.hipEventDestroy(ev)
        self.made = []


# ------------------------------------------------------------------ the step
class Runner:
    def __init__(self, w, device="cuda", bias_grad=False):
        self.w = w
        dev = torch.device(device)
        self.q = w.q.to(dev)
        self.k = w.k.to(dev)
        self.v = w.v.to(dev)
        self.dout = None if w.dout is None else w.dout.to(dev)
        self.sc = {n: t.to(dev) for n, t in (w.mx_scales or {}).items()}
        self.q_off = None if w.q_off is None else torch.from_numpy(w.q_off).to(dev)
        self.kv_off = torch.from_numpy(w.kv_off).to(dev)
        self.bias = None if w.bias_table is None else w.bias_table.to(dev)
        # the longest key sequence is known when the batch is formed: passing it
        # lets the library leave out its long-sequence kernels when none can have work
        self.max_kv_len = int(w.lk.max()) if w.B > 0 else 0
        self.prob = _lib.make_problem(
            batch=w.B, heads=w.H, head_dim=w.D, dtype=torch.bfloat16 if w.mx else w.dtype, total_q=w.q.shape[0],
            total_k=w.total_k, q_offsets=self.q_off, kv_offsets=self.kv_off,
            lq_fixed=w.lq_fixed, causal=w.causal, scale=w.scale, act=w.act,
            bias_kind=w.bias_kind, bias_table=self.bias, bias_lo=w.bias_lo, bias_hi=w.bias_hi,
            max_kv_len=self.max_kv_len, window=w.window, rope_base=w.rope_base,
            rope_inputs_turned=w.rope_base > 0)
        # rotary embedding: q and k turned once per step (the rope call), the turned
        # rows serving the forward and the backward
        self.qt = torch.empty_like(self.q) if w.rope_base > 0 else self.q
        self.kt = torch.empty_like(self.k) if w.rope_base > 0 else self.k
        rows = w.total_q_out
        self.o = torch.empty((rows, w.H, w.D), dtype=torch.bfloat16 if w.mx else w.dtype, device=dev)
        self.lse = torch.empty((w.H, rows), dtype=torch.float32, device=dev)
        self.o_res = torch.empty_like(self.o) if (w.mode == "jfa" and w.dtype == torch.bfloat16) else None
        self.ws_f = torch.empty(_lib.ja_workspace_size(self.prob, _lib.PASS_FWD), dtype=torch.uint8, device=dev)
        self.backward = bool(w.backward and w.q_off is not None and self.dout is not None)
        self.bias_grad = bool(bias_grad and self.backward and self.bias is not None)
        if bias_grad and not self.bias_grad:
            raise SystemExit("--bias-grad needs a workload with a backward pass and a bias table")
        self.db = torch.empty_like(self.bias) if self.bias_grad else None
        if self.backward:
            self.dq = torch.empty_like(self.q)
            self.dk = torch.empty_like(self.k)
            self.dv = torch.empty_like(self.v)
            pass_b = _lib.PASS_BWD_DBIAS if self.bias_grad else _lib.PASS_BWD
            self.ws_b = torch.empty(_lib.ja_workspace_size(self.prob, pass_b), dtype=torch.uint8, device=dev)

    def kernels(self):
        rope = ["rope"] if self.w.rope_base else []
        # the turn back of dk (fp32: dq and dk); the bf16 dQ units turn dq back themselves
        rope_back = ["rope_back"] if (self.w.rope_base and self.backward) else []
        if self.w.dtype == torch.float32:  # plain fp32 kernels: no planner, no short / fused units
            ks = rope + ["fwd"]
            if self.backward:
                ks += (["bwd_delta"] if self.w.mode == "jfa" else []) + ["bwd_q", "bwd_kv"]
                ks += ["bwd_dbias"] if self.bias_grad else []
            return ks + rope_back
        long_units = not (0 < self.max_kv_len <= SHORT_KV)  # else those kernels are not launched
        ks = rope + ["plan", "fwd_short"] + (["fwd"] if long_units else [])
        if self.backward:
            ks += ["bwd_fused"] + (["bwd_kv", "bwd_q"] if long_units else [])
            ks += ["bwd_delta"] if self.w.mode == "jfa" else []
            ks += ["bwd_dbias"] if self.bias_grad else []
        return ks + rope_back

    def step(self):
        p, w = self.prob, self.w
        if w.rope_base > 0:
            _lib.jagged_rope(p, self.q, self.k, self.qt, self.kt)
        q, k = self.qt, self.kt
        if w.mx:  # MXFP8 forward (no backward)
            sc = self.sc
            if w.mode == "gdpa":
                _lib.jagged_gdpa_fwd_mx(p, self.q, sc["q"], self.k, sc["k"], self.v, sc["v"], self.o, self.ws_f)
            else:
                _lib.jagged_attn_fwd_mx(p, self.q, sc["q"], self.k, sc["k"], self.v, sc["v"], self.o, self.lse,
                                        self.o_res, self.ws_f)
            return
        if w.mode == "gdpa":
            _lib.jagged_gdpa_fwd(p, q, k, self.v, self.o, self.ws_f)
            if self.backward:
                _lib.jagged_gdpa_bwd(p, q, k, self.v, self.dout, self.dq, self.dk, self.dv, self.db, self.ws_b)
        else:
            _lib.jagged_attn_fwd(p, q, k, self.v, self.o, self.lse, self.o_res, self.ws_f)
            if self.backward:
                _lib.jagged_attn_bwd(p, q, k, self.v, self.o, self.o_res, self.dout, self.lse,
                                     self.dq, self.dk, self.dv, self.db, self.ws_b)


# ------------------------------------------------------------------ traffic
def sources_digest():
    """Digest of the measured kernels' sources and of the compiler configuration."""
    from recsys_jagged_attention_gdpa_amd import build as _build
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "recsys_jagged_attention_gdpa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    h.update(repr(_build.compile_config()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch from committed rocprofv3 counters, if taken on these sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("sources_digest") != sources_digest():
        return None
    return t.get("hbm_bytes_per_launch")


# Device-side kernel names of the library's kernels, as profilers list them.
KERNEL_SYMBOLS = {"plan": "plan_kernel", "fwd": "ja::fwd_kernel<", "fwd_short": "fwd_short_kernel",
                  "bwd_fused": "ja::fused_kernel<", "bwd_kv": "dkdv_kernel<", "bwd_q": "dq_kernel<",
                  "bwd_delta": "delta_kernel<", "bwd_dbias": "dbias_kernel<", "rope": "rope_kernel<",
                  "rope_back": "rope_kernel<"}


def write_traffic(workload, kernel, fetch_csv, write_csv, copy_mib, command):
    """Turn two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) into
    profiles/traffic_<kernel>_<workload>.json.  Both counters are scaled by what they
    read for the calibration copy kernel (an element-wise kernel that reads and writes
    copy_mib MiB), the largest element-wise dispatch in the same runs."""
    import csv
    import collections

    def per_kernel(path, counter):
        vals = collections.defaultdict(list)
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return vals

    copy_bytes = copy_mib * (1 << 20)
    out = {"workload": workload, "kernel": kernel, "sources_digest": sources_digest(),
           "command": command}
    total = 0.0
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = per_kernel(path, counter)
        ours = [v for n, vs in vals.items() if KERNEL_SYMBOLS[kernel] in n for v in vs]
        copies = [max(vs) for n, vs in vals.items() if "elementwise" in n]
        if not ours or not copies:
            raise SystemExit(f"{path}: no {counter} rows for {kernel} or for the copy kernel")
        factor = copy_bytes / (max(copies) * 1024.0)
        kib = sum(ours) / len(ours)
        out[counter] = {"kib_per_dispatch": round(kib, 1), "dispatches": len(ours),
                        "copy_kib": max(copies), "factor": round(factor, 4)}
        total += kib * 1024.0 * factor
    out["hbm_bytes_per_launch"] = int(round(total))
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    log(f"[bench] wrote {path}: {out['hbm_bytes_per_launch']} B per launch")


# ------------------------------------------------------------------ CPU oracle
def cpu_baseline(w, target_s=15.0):
    """Time the fp64 oracle (forward + backward) on a bounded random sample of samples.

    The oracle's rate (valid pairs per second) is first measured on one
    median-size sample; samples are then taken in a seeded random order,
    skipping any that alone would take over half the budget, until the
    predicted time reaches the budget, and that subset is timed."""
    from oracle import ref  # test infrastructure: only this leg of the benchmark uses it
    from tests.helpers import oracle_bwd, oracle_fwd

    rng = np.random.default_rng(7)
    order = [int(b) for b in rng.permutation(w.B)]
    cores = ref.max_threads()
    bwd = w.backward and w.q_off is not None
    pairs = pairs_per_sample(w).astype(np.float64) * w.H

    def run(idx):
        s = w.subset(sorted(idx))
        log(f"[bench] oracle on {len(idx)} sample(s), {int(pairs[idx].sum())} pairs ...")
        t0 = time.perf_counter()
        oracle_fwd(s)
        if bwd:
            oracle_bwd(s)
        return time.perf_counter() - t0

    nz = [b for b in order if pairs[b] > 0]
    if not nz:
        return None
    med = float(np.median(pairs[nz]))
    probe = next(b for b in nz if pairs[b] <= med)
    rate = pairs[probe] / max(run([probe]), 1e-6)  # pairs per second
    chosen, t_pred = [], 0.0
    for b in nz:
        t_b = pairs[b] / rate
        if t_b > target_s / 2:
            continue
        chosen.append(b)
        t_pred += t_b
        if t_pred >= target_s:
            break
    dt = run(chosen)
    useful = (4.0 + (10.0 if bwd else 0.0)) * w.D * float(pairs[chosen].sum())
    return {"value": useful / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(chosen)} of {w.B} samples (seeded random order, samples predicted to take "
                      f"over {target_s / 2:.0f} s alone skipped), all heads, forward"
                      f"{' + backward' if bwd else ''}, fp64, {dt:.1f} s"}


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="jfa_causal_self", choices=sorted(synth.CATALOGUE))
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration runs)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the dominant kernel's measured HBM traffic from two rocprofv3 "
                         "counter_collection.csv files (needs --kernel and --calibrate-copy-mib); "
                         "uses no GPU")
    ap.add_argument("--kernel", default=None, choices=sorted(KERNEL_SYMBOLS))
    ap.add_argument("--command", default="", help="the rocprofv3 command the csv files came from")
    ap.add_argument("--bias-grad", action="store_true",
                    help="also compute the bias table's gradient in every backward pass")
    ap.add_argument("--balance", action="store_true",
                    help="also report the persistent kernels' per-workgroup busy time (max / mean) "
                         "in one extra step after the timed ones")
    ap.add_argument("--roofline-kernel", default=None, choices=sorted(KERNEL_SYMBOLS),
                    help="place this kernel on the roofline instead of the slowest one")
    args = ap.parse_args()

    if args.traffic_from:
        if not args.kernel or not args.calibrate_copy_mib:
            ap.error("--traffic-from needs --kernel and --calibrate-copy-mib")
        write_traffic(args.workload, args.kernel, *args.traffic_from, args.calibrate_copy_mib,
                      args.command)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(samples shard across GPUs with no exchange; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    _lib.load()

    t0 = time.perf_counter()
    w = synth.make(args.workload, args.seed)
    log(f"[bench] workload {args.workload}: B={w.B} H={w.H} D={w.D} Tq={w.total_q} Tk={w.total_k} "
        f"generated in {time.perf_counter() - t0:.1f}s")
    runner = Runner(w, bias_grad=args.bias_grad)
    ev = HipEvents()

    for _ in range(args.warmup):
        runner.step()
    torch.cuda.synchronize()

    if args.calibrate_copy_mib:
        # one element-wise kernel that reads n bytes and writes n bytes
        n = args.calibrate_copy_mib * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy kernel: read {n} bytes, wrote {n} bytes")

    # timed region: exactly K steps; the library records an event pair around every
    # kernel it launches, on the stream it launches it on
    names = runner.kernels()
    pairs = [{k: (ev.create(), ev.create()) for k in names} for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for step_pairs in pairs:
        for k, (a, b) in step_pairs.items():
            _lib.ja_profile_kernel(k, a, b)
        runner.step()
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    for k in names:
        _lib.ja_profile_kernel(k, None, None)
    durs = {k: sum(ev.elapsed_ms(*sp[k]) for sp in pairs) / args.steps for k in names}
    ev.close()
    dominant = max(durs, key=durs.get)
    if args.roofline_kernel:
        if args.roofline_kernel not in durs:
            raise SystemExit(f"kernel {args.roofline_kernel} does not run in this workload")
        dominant = args.roofline_kernel
    dom_ms = durs[dominant]
    log("[bench] kernel ms (timed steps): " + ", ".join(f"{k}={v:.4f}" for k, v in durs.items()))

    balance = None
    if args.balance:
        # one more step, outside the timed region, with every persistent kernel's
        # workgroups stamping their busy cycles
        persistent = [k for k in ("fwd", "fwd_short", "bwd_kv", "bwd_q", "bwd_fused", "bwd_dbias") if k in names]
        bufs = {k: torch.zeros(8192, dtype=torch.int64, device="cuda") for k in persistent}
        for k in persistent:
            _lib.ja_profile_busy(k, bufs[k])
        runner.step()
        torch.cuda.synchronize()
        for k in persistent:
            _lib.ja_profile_busy(k, None)
        balance = {}
        for k, b in bufs.items():
            v = b[b > 0].double().cpu().numpy()
            if v.size:
                balance[k] = {"workgroups": int(v.size), "max_over_mean": round(float(v.max() / v.mean()), 4),
                              "min_over_mean": round(float(v.min() / v.mean()), 4),
                              "mean_cycles": round(float(v.mean()))}
        log(f"[bench] balance: {balance}")

    ms_per_step = (t_end - t_start) * 1e3 / args.steps
    P = valid_pairs(w) * w.H
    useful = (4.0 + (10.0 if runner.backward else 0.0)) * w.D * P
    value = useful / (ms_per_step * 1e-3) / 1e12
    dom_bytes, dom_flops = kernel_cost(w, dominant)
    bound = BOUND.get(args.workload, "hbm")
    if bound == "hbm":
        achieved, peak, unit = dom_bytes / (dom_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    elif bound == "alu":
        achieved, peak, unit = dom_flops / (dom_ms * 1e-3) / 1e12, PEAK_FP32_VALU_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = dom_flops / (dom_ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    traffic = measured_traffic(args.workload, dominant)
    lq = w.lq.astype(np.int64)
    sparsity = 1.0 - float(lq.sum()) / (w.B * max(int(lq.max()), 1))

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(w, args.cpu_seconds)

    line = {
        "metric": "useful (unpadded) TFLOP/s fwd+bwd and % bf16 MFMA peak, sparsity-0.5 jagged",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp8-in/bf16" if w.mx else ("bf16" if w.dtype == torch.bfloat16 else "f32"),
        "data": "synthetic",
        "config": {"workload": args.workload, "B": w.B, "H": w.H, "D": w.D,
                   "total_q": w.total_q, "total_k": w.total_k, "act": w.act if w.mode == "gdpa" else "softmax",
                   "causal": w.causal, "window": w.window, "rope_base": w.rope_base, "bias": w.bias_kind, "jagged_sparsity": round(sparsity, 4),
                   "useful_pairs": P, "backward": runner.backward, "bias_grad": runner.bias_grad},
        "pct_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 3),
        "roofline": {"bound": bound, "kernel": dominant, "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic, "algorithmic_bytes": dom_bytes,
                     "algorithmic_flops": dom_flops, "avg_ms": round(dom_ms, 5)},
        "kernel_ms": {k: round(v, 5) for k, v in durs.items()},
        "cpu_baseline": cpu,
    }
    if balance is not None:
        line["balance"] = balance
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
