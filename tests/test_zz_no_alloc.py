"""gdr2_fwd_noalloc -- the inference forward whose workspace is the library's fixed device
array, for callers that cannot allocate -- called through the C ABI against gdr2_fwd, the
entry point it is a variant of: two calls in a row (the second with a smaller input, so the
array holds the first call's contents), then an fp32 call; results bitwise equal to
gdr2_fwd's (same kernels, same workspace layout) and so within the oracle tolerances that
gdr2_fwd meets."""
import pytest
import torch

import gated_delta_rule_gdr2_amd as g2
from gated_delta_rule_gdr2_amd.inputs import WORKLOADS, make_inputs, small

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "b", "w")


def _both(wl):
    x = {k: (None if v is None else v.cuda()) for k, v in make_inputs(wl).items()}
    args = [x[n] for n in NAMES] + [x["h0"]]
    ws_bytes = g2.gdr2_fwd_workspace_bytes(wl.B, wl.T, wl.H, wl.DK, wl.DV, 64, g2._DT[x["q"].dtype], False)
    assert 0 < ws_bytes <= g2.NOALLOC_SCRATCH_BYTES
    o_ref, h_ref, _ = g2.gdr2_fwd(*args)
    torch.cuda.synchronize()
    o, h = g2.gdr2_fwd_noalloc(*args)
    torch.cuda.synchronize()
    return (o_ref, h_ref), (o, h)


def test_noalloc_forward_matches_gdr2_fwd_on_two_calls_in_a_row():
    big = WORKLOADS["fwd_bf16_b1h16t2048d128_h0"]  # B=1, H=16, T=2048, d=128, bf16, h0
    smaller = small(DK=128, DV=128, T=700, dtype="bf16", B=1, H=4, h0_std=0.05, backward=False, seed=81)
    for wl in (big, smaller):
        (o_ref, h_ref), (o, h) = _both(wl)
        assert torch.isfinite(o.float()).all() and torch.isfinite(h).all()
        assert torch.equal(o, o_ref), wl.name
        assert torch.equal(h, h_ref), wl.name


def test_noalloc_forward_fp32_and_without_final_state():
    wl = small(DK=64, DV=64, T=257, dtype="f32", B=2, H=3, h0_std=0.1, backward=False, seed=82)
    (o_ref, h_ref), (o, h) = _both(wl)
    assert torch.equal(o, o_ref) and torch.equal(h, h_ref)
    x = {k: (None if v is None else v.cuda()) for k, v in make_inputs(wl).items()}
    o2, h2 = g2.gdr2_fwd_noalloc(*(x[n] for n in NAMES), None, output_final_state=False)
    o3, _, _ = g2.gdr2_fwd(*(x[n] for n in NAMES), None)
    torch.cuda.synchronize()
    assert h2 is None and torch.equal(o2, o3)


def test_noalloc_rejects_a_call_beyond_the_array():
    wl = small(DK=128, DV=128, T=16384, dtype="bf16", B=2, H=16, backward=False, seed=83)
    need = g2.gdr2_fwd_workspace_bytes(wl.B, wl.T, wl.H, 128, 128, 64, g2.DTYPE_BF16, False)
    assert need > g2.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(wl.B, wl.T, wl.H, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="fixed device array"):
        g2.gdr2_fwd_noalloc(q, q, q, q, q, q)
