"""Throughput benchmark of the Gated Delta Rule-2 operator (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = gdr2_fwd(save_for_bwd=1) + gdr2_bwd(fwd_saved=1) over one batch of
synthetic inputs already resident in HBM (the default workload: B=2, H=16,
T=4096, d_k=d_v=128, bf16 inputs, fp32 state, chunk 64). Prints one JSON line.

value            : whole-job tokens/s, tokens = B*T (all heads), over exactly K steps
                   bracketed by device synchronisation.
roofline         : the kernel with the largest average duration, its algorithmic HBM
                   bytes per launch (the operator inputs and outputs it must move; no
                   intermediates) over its average duration, timed with HIP events that
                   the library records on the launch stream around each kernel.
step_roofline    : algorithmic bytes of the whole step over 8 TB/s, divided by the
                   measured step time (the fraction of the HBM roofline for fwd+bwd).
cpu_baseline     : the fp64 oracle (test infrastructure, untuned) timed on the host
                   cores over a bounded sample of the same workload's sequences.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, published
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


def algorithmic_flops(wl, C=64):
    """Chunkwise flops (triangular products at half cost, no recompute)."""
    th = wl.B * wl.T * wl.H
    d = wl.DK
    fwd = C * (3 * wl.DK + 2 * wl.DV) + 6 * wl.DK * wl.DV
    bwd = 14 * C * d + 12 * wl.DK * wl.DV
    return th * (fwd + bwd)


class HipEvents:
    """Minimal ctypes access to HIP events (created here, recorded by libgdr2)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            st = self.hip.hipEventCreate(ctypes.byref(e))
            if st != 0:
                raise RuntimeError("hipEventCreate failed: %d" % st)
            evs[i] = e.value
        return evs

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        st = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if st != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % st)
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def cpu_baseline(wl, inputs, budget_seqs=None):
    """Time the fp64 oracle (fwd + bwd) on the first n (batch, head) sequences at full length."""
    import numpy as np
    import oracle
    cores = oracle.num_threads()
    NS = wl.B * wl.H
    n = min(NS, budget_seqs or cores)
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
    t0 = time.perf_counter()
    oracle.fwd(*args, h0)
    if wl.backward:
        oracle.bwd(*args, h0, do)
    dt = time.perf_counter() - t0
    tokens = n * wl.T / wl.H
    return {"value": tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d of %d (batch, head) sequences at full length T=%d, fwd+bwd, fp64, %.1f s"
                      % (n, NS, wl.T, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="also run one plain device-to-device copy of MB MiB (outside the timed region), "
                         "the reference that HBM byte counters are scaled by")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this operator build has no multi-GPU path "
              "(each GPU would run the same kernels on its share of the batch*head sequences). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_gdr2_amd as g2
    from gated_delta_rule_gdr2_amd.inputs import HEADLINE, WORKLOADS, make_inputs

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
    evs = hip.create(6 * K)

    ev_arrays = [((ctypes.c_void_p * 3)(*evs[6 * i:6 * i + 3]), (ctypes.c_void_p * 3)(*evs[6 * i + 3:6 * i + 6]))
                 for i in range(K)]

    def step(i):
        fe = None if i is None else ctypes.cast(ev_arrays[i][0], ctypes.c_void_p)
        be = None if i is None else ctypes.cast(ev_arrays[i][1], ctypes.c_void_p)
        g2.gdr2_fwd(*(x[n] for n in names), x["h0"], save_for_bwd=True, ws=ws, o=o, stream=stream,
                    stage_events=fe)
        g2.gdr2_bwd(*(x[n] for n in names), x["h0"], x["do"], ws=ws, fwd_saved=True, grads=grads,
                    need_dh0=x["h0"] is not None, stream=stream, stage_events=be)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(W):
        step(None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    kern = {"fwd_intra": (0, 1), "fwd_chain": (1, 2), "bwd_chain": (3, 4), "bwd_intra": (4, 5)}
    avg_ms = {k: sum(hip.elapsed_ms(evs[6 * i + a], evs[6 * i + b]) for i in range(K)) / K
              for k, (a, b) in kern.items()}
    hip.destroy(evs)
    abytes = algorithmic_bytes(wl, esz)
    dom = max(avg_ms, key=avg_ms.get)
    achieved = abytes[dom] / (avg_ms[dom] * 1e-3) / 1e9
    ms_step = elapsed / K * 1e3
    step_bytes = sum(abytes.values())
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
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": dom,
                     "algorithmic_bytes_per_launch": abytes[dom], "avg_launch_ms": avg_ms[dom]},
        "step_roofline": {"bound": "hbm", "algorithmic_bytes": step_bytes, "t_roofline_ms": t_roof_ms,
                          "frac": t_roof_ms / ms_step},
        "kernels_avg_ms": avg_ms,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, host)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
