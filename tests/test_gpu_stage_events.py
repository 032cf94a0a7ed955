"""Per-stage timing events of gdr2_fwd / gdr2_bwd (the stage_events argument): element 0
at the start of the first stage and element i at the end of the i-th, attached to the
kernel launches. gdr2_fwd and gdr2_bwd(fwd_saved = 1) take 3 events, gdr2_bwd(fwd_saved
= 0) 5 (the two forward stages, then the two backward ones). Checked: every stage has a
positive duration, the stages add up to the whole call, and timing does not change the
results."""
import ctypes

import pytest
import torch

import gated_delta_rule_gdr2_amd as g2
from bench import HipEvents
from gated_delta_rule_gdr2_amd.inputs import make_inputs, small

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "b", "w")


def _stages(hip, evs, n):
    return [hip.elapsed_ms(evs[i], evs[i + 1]) for i in range(n - 1)], hip.elapsed_ms(evs[0], evs[n - 1])


@pytest.mark.parametrize("segments", [1, 4])
def test_stage_events_cover_the_stages(segments):
    wl = small(DK=128, DV=128, T=1000, dtype="bf16", B=1, H=2, h0_std=0.05, seed=51)
    x = {k: (None if v is None else v.cuda()) for k, v in make_inputs(wl).items()}
    args = [x[n] for n in NAMES] + [x["h0"]]
    hip = HipEvents()
    evs = hip.create(11)
    arrays = [(ctypes.c_void_p * n)(*evs[a:a + n]) for a, n in ((0, 3), (3, 3), (6, 5))]
    fe, be, re = (ctypes.cast(arr, ctypes.c_void_p) for arr in arrays)
    stream = torch.cuda.current_stream()
    try:
        o, ht, ws = g2.gdr2_fwd_seg(*args, segments=segments, save_for_bwd=True, stream=stream, stage_events=fe)
        gr = g2.gdr2_bwd_seg(*args, x["do"], segments=segments, ws=ws, fwd_saved=True, stream=stream,
                             stage_events=be)
        gr = {k: v.clone() for k, v in gr.items()}
        gr_re = g2.gdr2_bwd_seg(*args, x["do"], segments=segments, fwd_saved=False, stream=stream, stage_events=re)
        torch.cuda.synchronize()
        for name, base, n in (("fwd", 0, 3), ("bwd", 3, 3), ("bwd recompute", 6, 5)):
            parts, whole = _stages(hip, evs[base:base + n], n)
            print(name, ["%.4f" % p for p in parts], "whole %.4f ms" % whole, flush=True)
            assert all(p > 0 for p in parts), (name, parts)
            assert abs(sum(parts) - whole) <= 1e-3 * whole + 1e-4, (name, parts, whole)
        o2, ht2, _ = g2.gdr2_fwd_seg(*args, segments=segments, save_for_bwd=True, stream=stream)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(ht, ht2)
        for key in gr:
            assert torch.equal(gr[key], gr_re[key]), key
    finally:
        hip.destroy(evs)


def test_stage_events_with_null_slots():
    """Elements of the event array may be NULL: only the given boundaries carry events (how
    bench.py times the dominant kernel alone). Here only the backward intra-chunk stage's two
    boundaries (elements 1 and 2 of the backward's array) have events; the interval is
    positive and no longer than the whole call timed outside, and the results are unchanged."""
    wl = small(DK=128, DV=128, T=700, dtype="bf16", B=2, H=2, h0_std=0.05, seed=52)
    x = {k: (None if v is None else v.cuda()) for k, v in make_inputs(wl).items()}
    args = [x[n] for n in NAMES] + [x["h0"]]
    hip = HipEvents()
    evs = hip.create(4)
    arr = (ctypes.c_void_p * 3)(None, evs[0], evs[1])
    stream = torch.cuda.current_stream()
    try:
        o, ht, ws = g2.gdr2_fwd(*args, save_for_bwd=True, stream=stream)
        ref = {k: v.clone() for k, v in g2.gdr2_bwd(*args, x["do"], ws=ws, fwd_saved=True, stream=stream).items()
               if v is not None}
        hip.record(evs[2], stream)
        gr = g2.gdr2_bwd(*args, x["do"], ws=ws, fwd_saved=True, stream=stream,
                         stage_events=ctypes.cast(arr, ctypes.c_void_p))
        hip.record(evs[3], stream)
        torch.cuda.synchronize()
        intra, whole = hip.elapsed_ms(evs[0], evs[1]), hip.elapsed_ms(evs[2], evs[3])
        print("intra stage %.4f ms of %.4f ms" % (intra, whole), flush=True)
        assert 0 < intra <= whole
        for key, v in ref.items():
            assert torch.equal(gr[key], v), key
    finally:
        hip.destroy(evs)
