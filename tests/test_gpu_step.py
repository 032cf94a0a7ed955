"""Parity of the recurrent step (gdr2_step, for decoding) with the fp64 oracle and with
the chunkwise forward, through the C ABI.

The oracle's forward is the token-by-token recurrence itself, so the step must give its
o and final state from any start state: fp32 inputs max|X - R| / max|R| <= 1e-5, bf16
inputs ||X - R||_F / ||R||_F <= 2e-2 (o rounded to bf16, state fp32)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_gdr2_amd as g2
import oracle
from gated_delta_rule_gdr2_amd.inputs import make_inputs, small

pytestmark = pytest.mark.gpu

TOL = {"f32": ("inf", 1e-5), "bf16": ("fro", 2e-2)}


def err(x, r, kind):
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if kind == "inf":
        return np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-30)
    return np.linalg.norm(x - r) / max(np.linalg.norm(r), 1e-30)


def np64(t):
    return t.detach().float().cpu().double().numpy()


CASES = [
    dict(DK=128, DV=128, T=1, dtype="bf16", B=3, H=4),
    dict(DK=128, DV=128, T=5, dtype="bf16", B=1, H=2, g_scale=2.0),
    dict(DK=64, DV=128, T=33, dtype="bf16", B=2, H=2),
    dict(DK=128, DV=64, T=2, dtype="bf16", B=2, H=3),
    dict(DK=64, DV=64, T=70, dtype="bf16", B=1, H=2),
    dict(DK=64, DV=64, T=1, dtype="f32", B=2, H=2),
    dict(DK=64, DV=64, T=40, dtype="f32", B=1, H=3),
]


@pytest.mark.parametrize("p", CASES, ids=lambda p: "-".join("%s%s" % kv for kv in p.items()))
def test_step_matches_oracle(p):
    kw = dict(p)
    wl = small(DK=kw.pop("DK"), DV=kw.pop("DV"), T=kw.pop("T"), dtype=kw.pop("dtype"), B=kw.pop("B"),
               H=kw.pop("H"), backward=False, h0_std=0.1, **kw)
    inp = make_inputs(wl)
    names = ["q", "k", "v", "g", "b", "w"]
    x = {n: inp[n].cuda() for n in names}
    state = inp["h0"].clone().cuda()
    o = g2.gdr2_step(*(x[n] for n in names), state)
    torch.cuda.synchronize()
    ro, rh = oracle.fwd(*(np64(inp[n]) for n in names), np64(inp["h0"]))
    kind, tol = TOL[wl.dtype]
    eo, eh = err(np64(o), ro, kind), err(np64(state), rh, kind)
    print("o %s err %.3e, state %s err %.3e (tol %.0e)" % (kind, eo, kind, eh, tol))
    assert eo <= tol and eh <= tol


def test_step_continues_across_calls_and_matches_the_chunkwise_forward():
    """Only the state is carried: steps over T1 then T2 tokens equal one call over T1 + T2
    (bitwise: the same operations in the same order), and both agree with the chunkwise
    forward from the same start state."""
    wl = small(DK=128, DV=128, T=96, dtype="bf16", B=2, H=3, backward=False, h0_std=0.05)
    inp = make_inputs(wl)
    names = ["q", "k", "v", "g", "b", "w"]
    x = {n: inp[n].cuda() for n in names}
    h0 = inp["h0"].cuda()
    s_all = h0.clone()
    o_all = g2.gdr2_step(*(x[n] for n in names), s_all)
    s_part = h0.clone()
    o1 = g2.gdr2_step(*(x[n][:, :40].contiguous() for n in names), s_part)
    o2 = g2.gdr2_step(*(x[n][:, 40:].contiguous() for n in names), s_part)
    oc, hc, _ = g2.gdr2_fwd(*(x[n] for n in names), h0)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([o1, o2], 1), o_all) and torch.equal(s_part, s_all)
    assert err(np64(o_all), np64(oc), "fro") <= 2e-2
    assert err(np64(s_all), np64(hc), "fro") <= 2e-2


def test_step_large_state_streaming_stores():
    """A state of 128 MiB or more (here 512 sequences x 16 heads, d = 128: 512 MiB) takes the
    instantiation that writes it back with non-temporal stores. Its o and state must match the
    oracle on sampled (sequence, head) pairs, the last included, and equal bit for bit what the
    plain-store instantiation gives for the same sequences in a small batch."""
    B, H, D = 512, 16, 128
    wl = small(DK=D, DV=D, T=1, dtype="bf16", B=B, H=H, backward=False, h0_std=0.0)
    inp = make_inputs(wl)
    names = ["q", "k", "v", "g", "b", "w"]
    x = {n: inp[n].cuda() for n in names}
    gen = torch.Generator(device="cuda").manual_seed(23)
    state = torch.randn(B, H, D, D, device="cuda", generator=gen) * 0.05
    rows = [0, 137, B - 1]
    start = state[rows].clone()
    o = g2.gdr2_step(*(x[n] for n in names), state)
    # the same sequences as a 3-sequence batch (3 MiB of state: plain stores)
    small_state = start.clone()
    o_small = g2.gdr2_step(*(x[n][rows].contiguous() for n in names), small_state)
    torch.cuda.synchronize()
    assert torch.equal(o[rows], o_small) and torch.equal(state[rows], small_state)
    for b, h in ((0, 0), (137, 5), (B - 1, H - 1)):
        sl = lambda t: np64(t[b:b + 1, :, h:h + 1])
        s0 = np64(start[rows.index(b), h])[None, None]
        ro, rh = oracle.fwd(*(sl(inp[n]) for n in names), s0)
        eo = err(np64(o[b:b + 1, :, h:h + 1]), ro, "fro")
        eh = err(np64(state[b, h])[None, None], rh, "fro")
        print("b %d h %d: o fro err %.3e, state fro err %.3e" % (b, h, eo, eh))
        assert eo <= 2e-2 and eh <= 2e-2
