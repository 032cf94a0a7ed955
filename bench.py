"""Throughput benchmark of the Gated Delta Rule-2 operator (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = gdr2_fwd(save_for_bwd=1) + gdr2_bwd(fwd_saved=1) over one batch of
synthetic inputs already resident in HBM (the default workload: B=2, H=16,
T=4096, d_k=d_v=128, bf16 inputs, fp32 state, chunk 64). Prints one JSON line.

value            : whole-job tokens/s, tokens = B*T (all heads), over exactly K steps
                   bracketed by device synchronisation.
roofline         : the kernel with the largest average duration (from a pass of K steps
                   before the timed ones, with HIP events at every stage boundary:
                   kernels_avg_ms), its algorithmic HBM bytes per launch (the operator
                   inputs and outputs it must move; no intermediates) over its average
                   duration in the K timed steps, where the library attaches HIP events
                   to the launches at that kernel's two boundaries only.
                   "traffic" is that kernel's measured HBM bytes per launch (rocprofv3
                   FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size), read
                   from the summary under profiles/ when it was taken on the current
                   kernel sources (same digest), else null.
step_roofline    : algorithmic bytes of the whole step (each operator input and output
                   counted once) over 8 TB/s, divided by the measured step time.
cpu_baseline     : the fp64 oracle (test infrastructure, untuned) timed on the host
                   cores over a bounded sample of the same workload's sequences:
                   passes over the first B*H sequences at full length until about
                   10 s have elapsed.

    python bench.py --all-configs [--table PATH]

times every workload of gated_delta_rule_gdr2_amd.inputs.WORKLOADS (the forward-only ones
as gdr2_fwd steps, the training ones as fwd+bwd steps), each right after a 512 MiB write
that evicts the Infinity Cache and also back to back, next to one oracle pass over a
sample of its sequences at full length, with the GPU's normwise relative error against
that pass per output tensor; one JSON line per workload, and with --table a markdown
table at PATH.

    python bench.py --summarize-profile DIR

reads the rocprofv3 output of a profiling run (DIR/trace, DIR/pmc_FETCH_SIZE,
DIR/pmc_WRITE_SIZE, made with --copy-calibration) and writes the per-kernel
summary under profiles/.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(HERE, "profiles")
CSRC = os.path.join(HERE, "gated_delta_rule_gdr2_amd", "csrc")
KERNELS = ("fwd_intra", "fwd_chain", "bwd_chain", "bwd_intra")

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, published
MFMA_F32_PEAK_TFLOPS = 157.3    # dense fp32 MFMA, published
METRIC = "GDR-2 fwd+bwd tokens/s at H=16,d=128,T=4K; % of MFMA/HBM roofline"


def algorithmic_bytes(wl, esz):
    """Per-kernel algorithmic bytes for one launch over the whole workload."""
    th = wl.B * wl.T * wl.H                     # token-heads
    state = wl.B * wl.H * wl.DK * wl.DV * 4     # one fp32 state tensor
    fwd_intra = th * (4 * wl.DK + 2 * wl.DV) * esz           # reads q, k, g, b, v, w
    fwd_chain = th * wl.DV * esz + state * (2 if wl.h0_std > 0 else 1)  # writes o, ht (+ reads h0)
    bwd_chain = th * wl.DV * esz + (state if wl.h0_std > 0 else 0)      # reads dout (+ writes dh0)
    bwd_intra = th * ((4 * wl.DK + 2 * wl.DV) + wl.DV + (4 * wl.DK + 2 * wl.DV)) * esz  # in + dout + grads
    return {"fwd_intra": fwd_intra, "fwd_chain": fwd_chain, "bwd_chain": bwd_chain, "bwd_intra": bwd_intra}


def step_algorithmic_bytes(wl, esz):
    """Operator-level bytes of one fwd+bwd step, each input and output counted once."""
    th = wl.B * wl.T * wl.H
    state = wl.B * wl.H * wl.DK * wl.DV * 4
    fwd = th * (4 * wl.DK + 2 * wl.DV + wl.DV) * esz + state              # in, o, ht
    bwd = th * (4 * wl.DK + 2 * wl.DV + wl.DV + 4 * wl.DK + 2 * wl.DV) * esz  # in, dout, grads
    if wl.h0_std > 0:
        fwd += state      # h0
        bwd += state      # dh0
    return fwd + bwd


def source_digest():
    """sha256 over the kernel sources; a profile summary is valid only for this digest."""
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_summary_path(workload):
    return os.path.join(PROFILES, "hbm_traffic_%s.json" % workload)


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None."""
    p = traffic_summary_path(workload)
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        d = json.load(fh)
    if d.get("source_digest") != source_digest():
        return None
    k = d["kernels"].get(kernel)
    return None if k is None else k["fetch_bytes"] + k["write_bytes"]


def algorithmic_flops(wl, C=64, backward=True):
    """Chunkwise flops (triangular products at half cost, no recompute)."""
    th = wl.B * wl.T * wl.H
    d = wl.DK
    fwd = C * (3 * wl.DK + 2 * wl.DV) + 6 * wl.DK * wl.DV
    bwd = 14 * C * d + 12 * wl.DK * wl.DV
    return th * (fwd + (bwd if backward else 0))


def forward_algorithmic_bytes(wl, esz):
    """Operator-level bytes of one forward call: inputs, o and the final state (+ h0)."""
    th = wl.B * wl.T * wl.H
    state = wl.B * wl.H * wl.DK * wl.DV * 4
    return th * (4 * wl.DK + 2 * wl.DV + wl.DV) * esz + state * (2 if wl.h0_std > 0 else 1)


class HipEvents:
    """Minimal ctypes access to HIP events (created here, recorded by libgdr2)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        evs = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            st = self.hip.hipEventCreate(ctypes.byref(e))
            if st != 0:
                raise RuntimeError("hipEventCreate failed: %d" % st)
            evs[i] = e.value
        return evs

    def record(self, e, stream):
        st = self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError("hipEventRecord failed: %d" % st)

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        st = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if st != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % st)
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def cpu_baseline(wl, inputs, min_seconds=10.0):
    """Time the fp64 oracle (fwd + bwd) in passes over the first n (batch, head) sequences at
    full length (n = the oracle's thread count, at most B*H) until min_seconds have elapsed."""
    import numpy as np
    import oracle
    cores = oracle.num_threads()
    NS = wl.B * wl.H
    n = min(NS, cores)
    sel = [(s // wl.H, s % wl.H) for s in range(n)]

    def take(x, state=False):
        if x is None:
            return None
        a = x.float().cpu().double().numpy()
        if state:
            return np.concatenate([a[b:b + 1, h:h + 1] for b, h in sel], axis=1)
        return np.concatenate([a[b:b + 1, :, h:h + 1] for b, h in sel], axis=2)

    args = [take(inputs[k]) for k in ("q", "k", "v", "g", "b", "w")]
    h0 = take(inputs["h0"], True)
    do = take(inputs["do"])
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.fwd(*args, h0)
        if wl.backward:
            oracle.bwd(*args, h0, do)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    tokens = passes * n * wl.T / wl.H
    return {"value": tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d pass(es) over %d of %d (batch, head) sequences at full length T=%d, fwd+bwd, "
                      "fp64, %.1f s; tokens counted as sequences*T/H" % (passes, n, NS, wl.T, dt)}


def _short(name):
    """The step kernel a dispatch name belongs to (k_<name> with its template arguments next,
    so that k_fwd_chain_sum is not k_fwd_chain), the device copy, or None."""
    for k in KERNELS:
        if "k_" + k + "I" in name:
            return k
    return "copyBuffer" if "copyBuffer" in name else None


def summarize_profile(d, workload, copy_mib, command):
    """Write profiles/ summaries from a rocprofv3 run: kernel trace stats and HBM traffic."""
    stats = {}
    for r in csv.DictReader(open(os.path.join(d, "trace", "run_kernel_stats.csv"))):
        k = _short(r["Name"])
        if k:
            stats[k] = {"name": r["Name"], "calls": int(r["Calls"]), "avg_ms": float(r["AverageNs"]) / 1e6,
                        "min_ms": float(r["MinNs"]) / 1e6, "max_ms": float(r["MaxNs"]) / 1e6}
    ctr = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        vals = {}
        for r in csv.DictReader(open(os.path.join(d, "pmc_" + c, "run_counter_collection.csv"))):
            k = _short(r["Kernel_Name"])
            if k and r["Counter_Name"] == c:
                vals.setdefault(k, []).append(float(r["Counter_Value"]))
        ctr[c] = {k: sum(v) / len(v) for k, v in vals.items()}
    copy_kib = copy_mib * 1024.0
    cal_f = copy_kib / ctr["FETCH_SIZE"]["copyBuffer"]
    cal_w = copy_kib / ctr["WRITE_SIZE"]["copyBuffer"]
    kern = {}
    for k in KERNELS:
        fb = ctr["FETCH_SIZE"][k] * cal_f * 1024
        wb = ctr["WRITE_SIZE"][k] * cal_w * 1024
        kern[k] = {"fetch_bytes": fb, "write_bytes": wb, "avg_ms": stats[k]["avg_ms"],
                   "gbs": (fb + wb) / (stats[k]["avg_ms"] * 1e-3) / 1e9}
    summary = {"workload": workload, "source_digest": source_digest(), "command": command,
               "calibration": {"copy_bytes": copy_mib << 20, "fetch_factor": cal_f, "write_factor": cal_w,
                               "note": "FETCH_SIZE/WRITE_SIZE are KiB per dispatch; each is scaled by "
                                       "the factor that makes a plain device copy of copy_bytes read and "
                                       "write exactly copy_bytes"},
               "kernels": kern}
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_summary_path(workload), "w") as fh:
        json.dump(summary, fh, indent=1)
    tot = sum(v["avg_ms"] for k, v in stats.items() if k in KERNELS)
    lines = ["# Kernel trace and HBM traffic: fwd+bwd step, workload %s" % workload, "",
             "Command (repository root, one MI355X):", "", "    " + command.replace("\n", "\n    "), "",
             "Kernel trace (rocprofv3 --kernel-trace --stats), per dispatch:", "",
             "| kernel | calls | average (ms) | min (ms) | max (ms) | share |", "|---|---|---|---|---|---|"]
    for k in KERNELS:
        v = stats[k]
        lines.append("| `%s` | %d | %.4f | %.4f | %.4f | %.1f%% |" % (v["name"], v["calls"], v["avg_ms"],
                                                                   v["min_ms"], v["max_ms"],
                                                                   100 * v["avg_ms"] / tot))
    lines += ["", "Sum of the four kernel averages: %.4f ms per step." % tot, "",
              "HBM traffic per dispatch (FETCH_SIZE x %.3f, WRITE_SIZE x %.3f; factors from a %d MiB "
              "device copy in the same runs):" % (cal_f, cal_w, copy_mib), "",
              "| kernel | fetched (MB) | written (MB) | GB/s at the trace average |", "|---|---|---|---|"]
    for k in KERNELS:
        v = kern[k]
        lines.append("| %s | %.1f | %.1f | %.0f |" % (k, v["fetch_bytes"] / 1e6, v["write_bytes"] / 1e6, v["gbs"]))
    lines += ["", "Kernel source digest (sha256 over gated_delta_rule_gdr2_amd/csrc): `%s`" % summary["source_digest"]]
    with open(os.path.join(PROFILES, "kernels_%s.md" % workload), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("wrote", traffic_summary_path(workload), "and the kernel table")


def summarize_mfma(d, workload, command):
    """Write profiles/mfma_<workload>.md from a rocprofv3 run with the derived counters
    MfmaUtil, MfmaFlopsBF16 and MfmaFlopsF32 (pmc_mfma/) and a kernel trace (trace/)."""
    stats = {}
    for r in csv.DictReader(open(os.path.join(d, "trace", "run_kernel_stats.csv"))):
        k = _short(r["Name"])
        if k in KERNELS:
            stats[k] = float(r["AverageNs"]) / 1e6
    vals = {}
    for r in csv.DictReader(open(os.path.join(d, "pmc_mfma", "run_counter_collection.csv"))):
        k = _short(r["Kernel_Name"])
        if k in KERNELS:
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    lines = ["# MFMA use per kernel: fwd+bwd step, workload %s" % workload, "",
             "Command (repository root, one MI355X):", "", "    " + command.replace("\n", "\n    "), "",
             "MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs), as rocprofv3 derives it;",
             "MFMA TFLOP/s = MfmaFlopsBF16 (or F32) per dispatch / the kernel-trace average duration,",
             "against the dense peaks (bf16 %.0f, fp32 %.1f TFLOP/s)." % (MFMA_BF16_PEAK_TFLOPS, MFMA_F32_PEAK_TFLOPS), "",
             "| kernel | avg ms | MfmaUtil % | bf16 MFMA TFLOP/s | of bf16 peak | fp32 MFMA TFLOP/s | of fp32 peak |",
             "|---|---|---|---|---|---|---|"]
    for k in KERNELS:
        v = {c: sum(x) / len(x) for c, x in vals.get(k, {}).items()}
        ms = stats[k]
        bf = v.get("MfmaFlopsBF16", 0.0) / (ms * 1e-3) / 1e12
        f32 = v.get("MfmaFlopsF32", 0.0) / (ms * 1e-3) / 1e12
        lines.append("| %s | %.4f | %.1f | %.1f | %.3f | %.2f | %.4f |" % (
            k, ms, v.get("MfmaUtil", float("nan")), bf, bf / MFMA_BF16_PEAK_TFLOPS, f32, f32 / MFMA_F32_PEAK_TFLOPS))
    lines += ["", "Kernel source digest (sha256 over gated_delta_rule_gdr2_amd/csrc): `%s`" % source_digest()]
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, "mfma_%s.md" % workload)
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("wrote", out)


def decode_step_measurement(torch, g2, reps=50):
    """Recurrent step (gdr2_step, decoding): one token per call for B = 512 sequences of H = 16
    heads at d_k = d_v = 128, bf16, state fp32 and updated in place. Algorithmic bytes per call:
    the state read and written (2 x 64 KB per head) plus the token's q, k, g, b, v, w and o."""
    B, H, D = 512, 16, 128  # a 512 MB state, twice the Infinity Cache: every call streams HBM
    gen = torch.Generator(device="cuda").manual_seed(11)
    def rnd(*shape):
        return torch.randn(*shape, device="cuda", generator=gen)
    q, k = (torch.nn.functional.normalize(rnd(B, 1, H, D), dim=-1).bfloat16() for _ in range(2))
    v = rnd(B, 1, H, D).bfloat16()
    g = (-torch.nn.functional.softplus(rnd(B, 1, H, D)) * 0.1).bfloat16()
    b, w = (torch.sigmoid(rnd(B, 1, H, D)).bfloat16() for _ in range(2))
    state = rnd(B, H, D, D) * 0.02
    o = torch.empty(B, 1, H, D, dtype=torch.bfloat16, device="cuda")
    for _ in range(10):
        g2.gdr2_step(q, k, v, g, b, w, state, o=o)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        g2.gdr2_step(q, k, v, g, b, w, state, o=o)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = B * H * (2 * D * D * 4 + 7 * D * 2)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": "decode_bf16_b512h16d128_t1", "us_per_call": us, "tokens_per_s": B / (us * 1e-6),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_call": nbytes}}


def seg_step_ms(torch, g2, wl, segments, K, stream, x=None):
    """Median over K event-timed fwd+bwd steps of gdr2_fwd_seg / gdr2_bwd_seg, with the
    median of each stage (intra-chunk and chain kernels as the library's events split them)."""
    from gated_delta_rule_gdr2_amd.inputs import make_inputs
    if x is None:
        x = {k: (None if v is None else v.cuda()) for k, v in make_inputs(wl).items()}
    names = ("q", "k", "v", "g", "b", "w")
    ws = g2.workspace(wl.B, wl.T, wl.H, wl.DK, wl.DV, x["q"].dtype, True, "cuda", segments)
    grads = {n: torch.empty_like(x[n[1:]]) for n in ("dq", "dk", "dv", "dg", "db", "dw")}
    hip = HipEvents()
    evs = hip.create(6 * K)
    arrs = [((ctypes.c_void_p * 3)(*evs[6 * i:6 * i + 3]), (ctypes.c_void_p * 3)(*evs[6 * i + 3:6 * i + 6]))
            for i in range(K)]

    def step(i):
        fe = None if i is None else ctypes.cast(arrs[i][0], ctypes.c_void_p)
        be = None if i is None else ctypes.cast(arrs[i][1], ctypes.c_void_p)
        g2.gdr2_fwd_seg(*(x[n] for n in names), x["h0"], segments=segments, save_for_bwd=True, ws=ws,
                        stream=stream, stage_events=fe)
        g2.gdr2_bwd_seg(*(x[n] for n in names), x["h0"], x["do"], segments=segments, ws=ws, fwd_saved=True,
                        grads=grads, need_dh0=x["h0"] is not None, stream=stream, stage_events=be)

    for _ in range(2):
        step(None)
    torch.cuda.synchronize()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()

    def med(a, b):
        return sorted(hip.elapsed_ms(evs[6 * i + a], evs[6 * i + b]) for i in range(K))[K // 2]

    out = {"segments": segments, "ms_per_step": med(0, 2) + med(3, 5), "fwd_intra": med(0, 1),
           "fwd_chain": med(1, 2), "bwd_chain": med(3, 4), "bwd_intra": med(4, 5)}
    hip.destroy(evs)
    return out


def scan_workloads():
    from dataclasses import replace
    from gated_delta_rule_gdr2_amd.inputs import WORKLOADS
    long_wl = WORKLOADS["fwdbwd_bf16_b1h16t16384d128_h0"]
    return [long_wl, replace(long_wl, H=4, name="fwdbwd_bf16_b1h4t16384d128_h0"),
            replace(long_wl, H=1, name="fwdbwd_bf16_b1h1t16384d128_h0"), WORKLOADS["fwdbwd_bf16_b2h16t4096d128"]]


def scan_sweep(torch, g2, K=10, table=None):
    """Chunk-parallel scan: fwd+bwd step time against the segment count on the long-sequence
    workload, the same with 4 and 1 heads, and the training shape. One JSON line each, and
    with `table` a markdown table there."""
    from gated_delta_rule_gdr2_amd.inputs import make_inputs
    stream = torch.cuda.current_stream()
    rows = []
    for wl in scan_workloads():
        x = {k: (None if v is None else v.cuda()) for k, v in make_inputs(wl).items()}
        auto = next(s for s in range(1, 33) if g2.gdr2_seg_workspace_bytes(
            wl.B, wl.T, wl.H, wl.DK, wl.DV, 64, s, g2.DTYPE_BF16, True) ==
            g2.gdr2_bwd_workspace_bytes(wl.B, wl.T, wl.H, wl.DK, wl.DV, 64, g2.DTYPE_BF16))
        for segments in (1, 2, 4, 8, 16, 32):
            r = seg_step_ms(torch, g2, wl, segments, K, stream, x)
            r.update({"workload": wl.name, "automatic_segments": auto})
            rows.append(r)
            print(json.dumps(r), flush=True)
        del x
    if table:
        lines = ["# Chunk-parallel scan: fwd+bwd step time against the chain segment count", "",
                 "Kernel source digest: `%s`." % source_digest()[:16],
                 "Command (MI355X, one GPU): `python bench.py --scan-sweep --table PATH`", "",
                 "Each line: median of %d fwd+bwd steps (`gdr2_fwd_seg(save_for_bwd=1)` + "
                 "`gdr2_bwd_seg(fwd_saved=1)`), bf16, d_k = d_v = 128, stage times from the library's HIP "
                 "events on the launch stream (the chain stages include the summary and scan kernels). "
                 "`auto` = the count `gdr2_fwd` / `gdr2_bwd` pick for the shape." % K, "",
                 "| workload | segments | step ms | fwd_intra | fwd chain stage | bwd chain stage | bwd_intra | auto |",
                 "|---|---|---|---|---|---|---|---|"]
        for r in rows:
            lines.append("| %s | %d | %.3f | %.3f | %.3f | %.3f | %.3f | %d |" % (
                r["workload"], r["segments"], r["ms_per_step"], r["fwd_intra"], r["fwd_chain"], r["bwd_chain"],
                r["bwd_intra"], r["automatic_segments"]))
        with open(table, "w") as fh:
            fh.write("\n".join(lines) + "\n")


def chain_scan_measurement(torch, g2, K, stream):
    """The long-sequence workload with 4 heads instead of 16 (32 chain workgroups): fwd+bwd
    step with the chains walked whole, and with the segment count the plain entry points
    pick."""
    wl = scan_workloads()[1]
    from gated_delta_rule_gdr2_amd.inputs import make_inputs
    x = {k: (None if v is None else v.cuda()) for k, v in make_inputs(wl).items()}
    one = seg_step_ms(torch, g2, wl, 1, K, stream, x)
    best = seg_step_ms(torch, g2, wl, 8, K, stream, x)
    return {"workload": wl.name, "ms_per_step_one_segment": one["ms_per_step"],
            "ms_per_step_8_segments": best["ms_per_step"], "chains_ms_one_segment": one["fwd_chain"] +
            one["bwd_chain"], "chains_ms_8_segments": best["fwd_chain"] + best["bwd_chain"]}


def gate_logits_measurement(torch, g2, wl, K, stream):
    """Fused gate activations: forward+backward steps with the gates passed as logits
    (activated inside the kernels), against the same steps with the activations and their
    chain rule done as separate elementwise passes in torch around the plain entry points.
    Median of K event-timed steps each."""
    from gated_delta_rule_gdr2_amd.inputs import make_inputs
    x = {k: (None if v is None else v.cuda()) for k, v in make_inputs(wl, gates="logits").items()}
    names = ("q", "k", "v", "zg", "zb", "zw")
    sc = dict(g_scale=wl.g_scale, b_scale=wl.b_scale)
    ws = g2.workspace(wl.B, wl.T, wl.H, wl.DK, wl.DV, x["q"].dtype, True, "cuda")
    grads = {n: torch.empty_like(x[m]) for n, m in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dg", "zg"),
                                                     ("db", "zb"), ("dw", "zw"))}

    def fused():
        g2.gdr2_fwd_logits(*(x[n] for n in names), x["h0"], save_for_bwd=True, ws=ws, stream=stream, **sc)
        g2.gdr2_bwd_logits(*(x[n] for n in names), x["h0"], x["do"], ws=ws, fwd_saved=True, grads=grads,
                           need_dh0=False, stream=stream, **sc)

    def separate():
        zg, zb, zw = (x[n].float() for n in ("zg", "zb", "zw"))
        g = (-wl.g_scale * torch.nn.functional.softplus(zg)).to(x["q"].dtype)
        sb, w = torch.sigmoid(zb), torch.sigmoid(zw)
        b = (wl.b_scale * sb).to(x["q"].dtype)
        wq = w.to(x["q"].dtype)
        g2.gdr2_fwd(x["q"], x["k"], x["v"], g, b, wq, x["h0"], save_for_bwd=True, ws=ws, stream=stream)
        gr = g2.gdr2_bwd(x["q"], x["k"], x["v"], g, b, wq, x["h0"], x["do"], ws=ws, fwd_saved=True,
                         need_dh0=False, stream=stream)
        (gr["dg"].float() * (-wl.g_scale * torch.sigmoid(zg))).to(x["q"].dtype)
        (gr["db"].float() * (wl.b_scale * sb * (1 - sb))).to(x["q"].dtype)
        (gr["dw"].float() * (w * (1 - w))).to(x["q"].dtype)

    hip = HipEvents()
    res = {}
    for name, fn in (("fused", fused), ("separate_torch_passes", separate)):
        fn()
        torch.cuda.synchronize()
        ev = hip.create(2 * K)
        for i in range(K):
            hip.record(ev[2 * i], stream)
            fn()
            hip.record(ev[2 * i + 1], stream)
        torch.cuda.synchronize()
        res[name] = sorted(hip.elapsed_ms(ev[2 * i], ev[2 * i + 1]) for i in range(K))[K // 2]
        hip.destroy(ev)
    return {"workload": wl.name + "_logits", "ms_per_step": res["fused"],
            "ms_per_step_separate_torch_passes": res["separate_torch_passes"]}


CONFIG_ORDER = ("fwd_f32_b1h2t256d64", "fwd_bf16_b1h16t2048d128_h0", "fwdbwd_bf16_b2h16t4096d128",
                "fwdbwd_bf16_b2h16t4096d128_tied", "fwdbwd_bf16_b8h16t2048d128_g05",
                "fwdbwd_bf16_b1h16t16384d128_h0")


def _normwise(gpu, ref):
    import numpy as np
    den = float(np.linalg.norm(ref))
    return float(np.linalg.norm(gpu - ref)) / (den if den > 0 else 1.0)


def measure_config(torch, g2, wl, K, W, stream, hip, with_oracle=True):
    """One workload: cache-evicted and back-to-back step times, step roofline, and one oracle
    pass over min(cores, B*H) of its sequences at full length with the GPU's error against it."""
    import numpy as np
    from gated_delta_rule_gdr2_amd.inputs import make_inputs
    host = make_inputs(wl)
    x = {k: (None if v is None else v.cuda()) for k, v in host.items()}
    B, T, H, DK, DV = wl.B, wl.T, wl.H, wl.DK, wl.DV
    esz = 2 if wl.dtype == "bf16" else 4
    names = ("q", "k", "v", "g", "b", "w")
    train = wl.backward
    ws = g2.workspace(B, T, H, DK, DV, x["q"].dtype, train, "cuda")
    o = torch.empty(B, T, H, DV, dtype=x["q"].dtype, device="cuda")
    grads = {n: torch.empty_like(x[n[1:]]) for n in ("dq", "dk", "dv", "dg", "db", "dw")} if train else None
    res = {}

    def step():
        _, ht, _ = g2.gdr2_fwd(*(x[n] for n in names), x["h0"], save_for_bwd=train, ws=ws, o=o, stream=stream)
        res["ht"] = ht
        if train:
            res["grads"] = g2.gdr2_bwd(*(x[n] for n in names), x["h0"], x["do"], ws=ws, fwd_saved=True,
                                       grads=grads, need_dh0=x["h0"] is not None, stream=stream)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t0) / K * 1e3
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    ev = hip.create(2 * K)
    for i in range(K):
        flush.fill_(i & 255)
        hip.record(ev[2 * i], stream)
        step()
        hip.record(ev[2 * i + 1], stream)
    torch.cuda.synchronize()
    cold_ms = sorted(hip.elapsed_ms(ev[2 * i], ev[2 * i + 1]) for i in range(K))[K // 2]
    hip.destroy(ev)
    del flush
    nbytes = step_algorithmic_bytes(wl, esz) if train else forward_algorithmic_bytes(wl, esz)
    flops = algorithmic_flops(wl, backward=train)
    peak_tf = MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    t_hbm, t_mfma = nbytes / (HBM_PEAK_GBS * 1e9) * 1e3, flops / (peak_tf * 1e12) * 1e3
    out = {"workload": wl.name, "path": "fwd+bwd" if train else "fwd", "dtype": wl.dtype,
           "B": B, "H": H, "T": T, "d_k": DK, "d_v": DV, "h0": x["h0"] is not None, "tied": wl.tied,
           "ms_cache_evicted": cold_ms, "ms_back_to_back": warm_ms,
           "tokens_per_s": B * T / (cold_ms * 1e-3), "tokens_per_s_back_to_back": B * T / (warm_ms * 1e-3),
           "roofline": {"bound": "hbm" if t_hbm >= t_mfma else "mfma", "algorithmic_bytes": nbytes,
                        "algorithmic_flops": flops, "t_roofline_ms": max(t_hbm, t_mfma),
                        "frac": max(t_hbm, t_mfma) / cold_ms}}
    if with_oracle:
        import oracle
        cores = oracle.num_threads()
        n = min(B * H, cores)
        sel = [(q // H, q % H) for q in range(n)]

        def take(t, state=False):
            if t is None:
                return None
            a = t.float().cpu().double().numpy()
            if state:
                return np.concatenate([a[bb:bb + 1, hh:hh + 1] for bb, hh in sel], axis=1)
            return np.concatenate([a[bb:bb + 1, :, hh:hh + 1] for bb, hh in sel], axis=2)

        args = [take(host[k]) for k in names]
        h0 = take(host["h0"], True)
        t0 = time.perf_counter()
        ro, rht = oracle.fwd(*args, h0)
        rg = oracle.bwd(*args, h0, take(host["do"])) if train else None
        dt = time.perf_counter() - t0
        err = {"o": _normwise(take(o), ro), "ht": _normwise(take(res["ht"], True), rht)}
        if train:
            for k in ("dq", "dk", "dv", "dg", "db", "dw"):
                err[k] = _normwise(take(res["grads"][k]), rg[k])
            if x["h0"] is not None:
                err["dh0"] = _normwise(take(res["grads"]["dh0"], True), rg["dh0"])
        out["parity_normwise_rel_err"] = err
        out["parity_tolerance"] = 2e-2 if wl.dtype == "bf16" else 1e-5
        out["cpu_baseline"] = {"value": n * T / H / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                               "seconds": dt, "sample": "one %s pass over %d of %d (batch, head) sequences at "
                               "full length T=%d, fp64; tokens counted as sequences*T/H"
                               % ("fwd+bwd" if train else "fwd", n, B * H, T)}
    del x, ws, o, grads
    torch.cuda.empty_cache()
    return out


def write_table(rows, path, digest):
    lines = ["# Every workload on one MI355X", "",
             "Kernel source digest: `%s`." % digest[:16],
             "Produced by `python bench.py --all-configs --steps %d --warmup %d --table PATH`; each time is the "
             "median over the steps, each after a 512 MiB write that evicts the Infinity Cache (\"cache evicted\"), "
             "and the mean of the same number of calls back to back." % (rows[0]["steps"], rows[0]["warmup"]), "",
             "| workload | path | ms (cache evicted) | ms (back to back) | tokens/s (evicted) | roofline | "
             "frac | max normwise err (tol) | oracle tokens/s (cores, s) |",
             "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        e = r.get("parity_normwise_rel_err")
        emax = "%.2e (%g)" % (max(e.values()), r["parity_tolerance"]) if e else "-"
        cb = r.get("cpu_baseline")
        cbs = "%.3g (%d, %.3g)" % (cb["value"], cb["cores"], cb["seconds"]) if cb else "-"
        rf = r["roofline"]
        lines.append("| %s | %s | %.4f | %.4f | %.4g | %s %.4f ms | %.3f | %s | %s |" % (
            r["workload"], r["path"], r["ms_cache_evicted"], r["ms_back_to_back"], r["tokens_per_s"],
            rf["bound"], rf["t_roofline_ms"], rf["frac"], emax, cbs))
    lines += ["", "Per-tensor errors (normwise relative, GPU vs the fp64 oracle on the sampled sequences):", ""]
    for r in rows:
        e = r.get("parity_normwise_rel_err")
        if e:
            lines.append("- %s: %s" % (r["workload"], ", ".join("%s %.2e" % kv for kv in e.items())))
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def all_configs(torch, g2, K, W, table, with_oracle):
    from gated_delta_rule_gdr2_amd.inputs import WORKLOADS
    stream = torch.cuda.current_stream()
    hip = HipEvents()
    rows = []
    for name in CONFIG_ORDER:
        print("# %s" % name, file=sys.stderr, flush=True)
        r = measure_config(torch, g2, WORKLOADS[name], K, W, stream, hip, with_oracle)
        r.update(steps=K, warmup=W)
        rows.append(r)
        print(json.dumps(r), flush=True)
    if table:
        write_table(rows, table, source_digest())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="also run one plain device-to-device copy of MB MiB (outside the timed region), "
                         "the reference that HBM byte counters are scaled by")
    ap.add_argument("--summarize-profile", metavar="DIR", default=None,
                    help="summarise a rocprofv3 run (no GPU needed) into profiles/")
    ap.add_argument("--profile-command", default="", help="the command line recorded with --summarize-profile")
    ap.add_argument("--summarize-mfma", metavar="DIR", default=None,
                    help="summarise a rocprofv3 MfmaUtil/MfmaFlops run (pmc_mfma/, trace/) into profiles/")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the step alone (no decode, gate-logit or chain-scan side measurements): "
                         "the run that rocprofv3 traces")
    ap.add_argument("--all-configs", action="store_true",
                    help="time every workload (forward-only ones as forward steps), each next to an oracle pass")
    ap.add_argument("--table", default=None, help="with --all-configs or --scan-sweep: write a markdown table here")
    ap.add_argument("--scan-sweep", action="store_true",
                    help="print fwd+bwd step times against the chain segment count (chunk-parallel scan) and exit")
    args = ap.parse_args()
    if args.summarize_mfma:
        from gated_delta_rule_gdr2_amd.inputs import HEADLINE
        summarize_mfma(args.summarize_mfma, args.workload or HEADLINE, args.profile_command)
        return
    if args.summarize_profile:
        from gated_delta_rule_gdr2_amd.inputs import HEADLINE
        summarize_profile(args.summarize_profile, args.workload or HEADLINE, args.copy_calibration or 256,
                          args.profile_command)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this operator build has no multi-GPU path "
              "(each GPU would run the same kernels on its share of the batch*head sequences). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_gdr2_amd as g2
    from gated_delta_rule_gdr2_amd.inputs import HEADLINE, WORKLOADS, make_inputs

    if args.scan_sweep:
        scan_sweep(torch, g2, table=args.table)
        return
    if args.all_configs:
        all_configs(torch, g2, args.steps, args.warmup, args.table, not args.no_cpu_baseline)
        return

    wl = WORKLOADS[args.workload or HEADLINE]
    if not wl.backward:
        raise SystemExit("bench.py times forward+backward steps; pick a training workload")
    host = make_inputs(wl)
    x = {k: (None if v is None else v.cuda()) for k, v in host.items()}
    B, T, H, DK, DV = wl.B, wl.T, wl.H, wl.DK, wl.DV
    esz = 2 if wl.dtype == "bf16" else 4
    ws = g2.workspace(B, T, H, DK, DV, x["q"].dtype, True, "cuda")
    o = torch.empty(B, T, H, DV, dtype=x["q"].dtype, device="cuda")
    grads = {n: torch.empty_like(x[n[1:]]) for n in ("dq", "dk", "dv", "dg", "db", "dw")}
    names = ("q", "k", "v", "g", "b", "w")
    stream = torch.cuda.current_stream()
    hip = HipEvents()
    K, W = args.steps, args.warmup
    # Stage boundaries as (call, event index): the library's events mark the start of a
    # call's first stage (index 0) and the end of each stage (1, 2), so a kernel's interval
    # runs from the end of the stage before it to its own end.
    kern = {"fwd_intra": (("fwd", 0), ("fwd", 1)), "fwd_chain": (("fwd", 1), ("fwd", 2)),
            "bwd_chain": (("bwd", 0), ("bwd", 1)), "bwd_intra": (("bwd", 1), ("bwd", 2))}

    def ev_arrays(n, pool, only=None):
        """n steps' event arrays (fwd, bwd), 3 slots each, filled from the event list pool;
        with `only` set, just that kernel's two boundaries get events and the other slots
        stay NULL."""
        arrs, it = [], iter(pool)
        for _ in range(n):
            slots = {("fwd", i): None for i in range(3)}
            slots.update({("bwd", i): None for i in range(3)})
            for key in (kern[only] if only else list(slots)):
                slots[key] = next(it)
            arrs.append(slots)
        return arrs

    def c_array(slots, call):
        return ctypes.cast((ctypes.c_void_p * 3)(*(slots[(call, i)] for i in range(3))), ctypes.c_void_p)

    def step(slots):
        fe = None if slots is None else c_array(slots, "fwd")
        be = None if slots is None else c_array(slots, "bwd")
        g2.gdr2_fwd(*(x[n] for n in names), x["h0"], save_for_bwd=True, ws=ws, o=o, stream=stream,
                    stage_events=fe)
        g2.gdr2_bwd(*(x[n] for n in names), x["h0"], x["do"], ws=ws, fwd_saved=True, grads=grads,
                    need_dh0=x["h0"] is not None, stream=stream, stage_events=be)

    def kernel_ms(arrs, k):
        a, b = kern[k]
        return sum(hip.elapsed_ms(sl[a], sl[b]) for sl in arrs) / len(arrs)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # Every event is created here, before any timing, and destroyed after the last read
    # (creating or destroying events between the passes has stalled the launches that follow).
    pool_brk, pool_timed = list(hip.create(6 * K)), list(hip.create(2 * K))
    brk = ev_arrays(K, pool_brk)
    for _ in range(W):
        step(None)
    # Per-kernel breakdown (every stage boundary carries an event), before the timed steps;
    # it also names the dominant kernel.
    for i in range(K):
        step(brk[i])
    torch.cuda.synchronize()
    avg_ms = {k: kernel_ms(brk, k) for k in kern}
    dom = max(avg_ms, key=avg_ms.get)
    # The timed steps: events only at the two boundaries of the dominant kernel, whose
    # average duration over these steps gives roofline.achieved (a few untimed steps with
    # the same events first).
    arrs = ev_arrays(K, pool_timed, only=dom)
    for i in range(min(W, K)):
        step(arrs[i])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(arrs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_ms = kernel_ms(arrs, dom)
    hip.destroy(pool_brk + pool_timed)

    # The same steps once more, each after a 512 MiB write that evicts the 256 MB Infinity
    # Cache, timed by events around the step alone (the write is outside): HBM-honest step time.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    ev_f = hip.create(2 * K)
    for i in range(K):
        flush.fill_(i & 255)
        hip.record(ev_f[2 * i], stream)
        step(None)
        hip.record(ev_f[2 * i + 1], stream)
    torch.cuda.synchronize()
    flushed_ms = sorted(hip.elapsed_ms(ev_f[2 * i], ev_f[2 * i + 1]) for i in range(K))[K // 2]
    hip.destroy(ev_f)
    del flush

    abytes = algorithmic_bytes(wl, esz)
    achieved = abytes[dom] / (dom_ms * 1e-3) / 1e9
    ms_step = elapsed / K * 1e3
    step_bytes = step_algorithmic_bytes(wl, esz)
    t_roof_ms = max(step_bytes / (HBM_PEAK_GBS * 1e9), algorithmic_flops(wl) / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e3

    out = {
        "metric": METRIC,
        "value": B * T * K / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "H": H, "T": T, "d_k": DK, "d_v": DV, "chunk": wl.chunk,
                   "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(wl.name, dom), "kernel": dom,
                     "algorithmic_bytes_per_launch": abytes[dom], "avg_launch_ms": dom_ms},
        "step_roofline": {"bound": "hbm", "algorithmic_bytes": step_bytes, "t_roofline_ms": t_roof_ms,
                          "frac": t_roof_ms / ms_step},
        "kernels_avg_ms": avg_ms,
        "ms_per_step_cache_evicted": flushed_ms,
    }
    if not args.headline_only:
        out["decode_step"] = decode_step_measurement(torch, g2)
        out["gate_logits"] = gate_logits_measurement(torch, g2, wl, K, stream)
        out["chain_scan"] = chain_scan_measurement(torch, g2, K, stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, host)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
