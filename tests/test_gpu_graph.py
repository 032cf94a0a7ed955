"""The entry points under HIP graph capture (torch.cuda.graph): a whole training step
(gdr2_fwd(save_for_bwd) + gdr2_bwd(fwd_saved)) on preallocated buffers, and the forward
without a workspace argument (gdr2_fwd_noalloc, meant for callers that capture). The library
enqueues only kernels (no memset or copy commands), so a captured call must replay exactly:
each graph is replayed several times, with eager work in between that overwrites every
buffer the graph writes (and, for the no-allocation forward, the library's shared scratch
array), and every replay is compared bitwise with the eager call."""
import pytest
import torch

import gated_delta_rule_gdr2_amd as g2
from gated_delta_rule_gdr2_amd.inputs import make_inputs, small

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "b", "w")
REPLAYS = 3


def _inputs(wl):
    x = {k: (None if v is None else v.cuda()) for k, v in make_inputs(wl).items()}
    return [x[n] for n in NAMES] + [x["h0"]], x["do"]


def test_training_step_replays_bitwise():
    wl = small(DK=128, DV=128, T=1000, dtype="bf16", B=2, H=4, h0_std=0.05, seed=91)
    args, do = _inputs(wl)
    print("graph: fwd+bwd B=2 H=4 T=1000 d=128 bf16", flush=True)
    ws = g2.workspace(wl.B, wl.T, wl.H, 128, 128, torch.bfloat16, True)
    o = torch.empty(wl.B, wl.T, wl.H, 128, dtype=torch.bfloat16, device="cuda")
    grads = {n: torch.empty_like(args[i]) for i, n in enumerate(("dq", "dk", "dv", "dg", "db", "dw"))}
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        def step():
            _, ht, _ = g2.gdr2_fwd(*args, save_for_bwd=True, ws=ws, o=o, stream=stream)
            gr = g2.gdr2_bwd(*args, do, ws=ws, fwd_saved=True, grads=grads, stream=stream)
            return ht, gr["dh0"]

        ht, dh0 = step()  # eager, also before capture so that every first-call setup is done
        torch.cuda.synchronize()
        ref = [o.clone(), ht.clone(), dh0.clone()] + [grads[k].clone() for k in sorted(grads)]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            ht_g, dh0_g = step()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for t in [o, ws, ht_g, dh0_g] + list(grads.values()):
            t.fill_(255 if t.dtype == torch.uint8 else float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o, ht_g, dh0_g] + [grads[k] for k in sorted(grads)]
        for a, b in zip(got, ref):
            assert torch.equal(a, b), "replay %d" % r


def test_noalloc_forward_replays_bitwise():
    wl = small(DK=128, DV=128, T=700, dtype="bf16", B=1, H=6, h0_std=0.05, backward=False, seed=92)
    other = small(DK=64, DV=128, T=1500, dtype="bf16", B=2, H=3, backward=False, seed=93)
    args, _ = _inputs(wl)
    oargs, _ = _inputs(other)
    print("graph: gdr2_fwd_noalloc B=1 H=6 T=700 d=128 bf16", flush=True)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        o_ref, h_ref = g2.gdr2_fwd_noalloc(*args, stream=stream)  # eager; looks up the scratch array
        torch.cuda.synchronize()
        o_ref, h_ref = o_ref.clone(), h_ref.clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            o_g, h_g = g2.gdr2_fwd_noalloc(*args, stream=stream)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        o_g.fill_(float("nan"))
        h_g.fill_(float("nan"))
        g2.gdr2_fwd_noalloc(*oargs)  # another shape through the same scratch array, eagerly
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_ref) and torch.equal(h_g, h_ref), "replay %d" % r
