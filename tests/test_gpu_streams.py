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


def test_non_current_stream_with_library_allocations():
    """Kernels enqueued on a stream that is not torch's current one, with every output and the
    workspace allocated by the binding (ws=None, fwd_saved=False: the workspace is dropped when
    the call returns while the kernels may still run). The current stream then allocates and
    writes memory at once; with the allocations recorded on the kernels' stream the allocator
    cannot hand their memory out before the kernels are done, so the results are bitwise those
    of a plain call."""
    wl = small(DK=128, DV=128, T=900, dtype="bf16", B=2, H=4, h0_std=0.05, seed=73)
    x = {k: (None if v is None else v.cuda()) for k, v in make_inputs(wl).items()}
    args = [x[n] for n in NAMES] + [x["h0"]]
    o_ref, h_ref, _ = g2.gdr2_fwd(*args)
    g_ref = g2.gdr2_bwd(*args, x["do"], fwd_saved=False)
    torch.cuda.synchronize()
    g_ref = {k: v.clone() for k, v in g_ref.items()}
    side = torch.cuda.Stream()  # default priority
    torch.cuda.synchronize()
    for _ in range(3):
        # a long kernel first on the side stream, so the library's kernels start late
        side.wait_stream(torch.cuda.current_stream())
        busy = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
        busy.record_stream(side)
        with torch.cuda.stream(side):
            for _ in range(4):
                busy.fill_(7)
        o, h, _ = g2.gdr2_fwd(*args, stream=side)
        gr = g2.gdr2_bwd(*args, x["do"], fwd_saved=False, stream=side)
        # the current stream reuses freed memory right away and scribbles on it
        junk = [torch.full((8 << 20,), 3.0, device="cuda") for _ in range(8)]
        del junk
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(h, h_ref)
        for key in g_ref:
            assert torch.equal(gr[key], g_ref[key]), key
