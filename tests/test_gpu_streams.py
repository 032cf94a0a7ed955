"""Independent calls on two streams at once (each with its own workspace and outputs) give
bitwise the results of the same calls made one after the other: the library keeps no device
state of its own between or across calls."""
import pytest
import torch

import gated_delta_rule_gdr2_amd as g2
from gated_delta_rule_gdr2_amd.inputs import make_inputs, small

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "b", "w")


def _call(x, stream):
    args = [x[n] for n in NAMES] + [x["h0"]]
    o, ht, ws = g2.gdr2_fwd(*args, save_for_bwd=True, stream=stream)
    gr = g2.gdr2_bwd(*args, x["do"], ws=ws, fwd_saved=True, stream=stream)
    out = {"o": o, "ht": ht}
    out.update(gr)
    return out


def test_two_streams_match_sequential_calls():
    xs = []
    for seed, T in ((71, 700), (72, 1300)):
        wl = small(DK=128, DV=128, T=T, dtype="bf16", B=2, H=4, h0_std=0.05, seed=seed)
        xs.append({k: (None if v is None else v.cuda()) for k, v in make_inputs(wl).items()})
    ref = []
    for x in xs:
        r = _call(x, torch.cuda.current_stream())
        torch.cuda.synchronize()
        ref.append({k: v.clone() for k, v in r.items()})
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    torch.cuda.synchronize()
    for _ in range(3):
        outs = []
        for x, s in zip(xs, streams):
            with torch.cuda.stream(s):
                outs.append(_call(x, s))
        torch.cuda.synchronize()
        for r, o in zip(ref, outs):
            for key in r:
                assert torch.equal(r[key], o[key]), key
