"""Calls without tokens (T = 0, or B * H = 0) through the C ABI on the GPU.

A recurrence over no tokens ends where it starts: the oracle's forward returns h_T = h0
and its backward dh0 = dht for T = 0 (checked here against the oracle itself), and the
library must give exactly that -- bitwise, since the state is only copied -- with empty
token outputs, no workspace, and zeros where the start (or end) state is absent."""
import numpy as np
import pytest
import torch

import gated_delta_rule_gdr2_amd as g2
import oracle

pytestmark = pytest.mark.gpu


def tensors(B, T, H, DK, DV, dtype=torch.bfloat16, seed=0):
    gen = torch.Generator().manual_seed(seed)
    tok = lambda d: torch.randn(B, T, H, d, generator=gen).to(dtype).cuda()
    q, k, g, b = tok(DK), tok(DK), tok(DK), tok(DK)
    v, w, do = tok(DV), tok(DV), tok(DV)
    h0 = torch.randn(B, H, DK, DV, generator=gen).cuda()
    dht = torch.randn(B, H, DK, DV, generator=gen).cuda()
    return q, k, v, g, b, w, do, h0, dht


@pytest.mark.parametrize("DK,DV,dtype", [(128, 128, torch.bfloat16), (64, 128, torch.bfloat16),
                                         (64, 64, torch.float32)])
def test_forward_and_backward_without_tokens_pass_the_state(DK, DV, dtype):
    B, H = 2, 3
    q, k, v, g, b, w, do, h0, dht = tensors(B, 0, H, DK, DV, dtype)
    print("T=0 B=%d H=%d dk=%d dv=%d %s" % (B, H, DK, DV, dtype), flush=True)
    # the oracle over no tokens
    z = np.zeros((B, 0, H, DK))
    zv = np.zeros((B, 0, H, DV))
    h0n, dhtn = h0.cpu().double().numpy(), dht.cpu().double().numpy()
    _, rht = oracle.fwd(z, z, zv, z, z, zv, h0n)
    rg = oracle.bwd(z, z, zv, z, z, zv, h0n, zv, dhtn)
    assert np.array_equal(rht, h0n) and np.array_equal(rg["dh0"], dhtn)

    for save in (False, True):
        o, ht, ws = g2.gdr2_fwd(q, k, v, g, b, w, h0, save_for_bwd=save)
        torch.cuda.synchronize()
        assert o.shape == (B, 0, H, DV) and ws.numel() == 0
        assert torch.equal(ht, h0)
    o, ht, _ = g2.gdr2_fwd(q, k, v, g, b, w, None)
    torch.cuda.synchronize()
    assert torch.equal(ht, torch.zeros_like(h0))
    for saved in (False, True):
        ws = g2.workspace(B, 0, H, DK, DV, dtype, True) if saved else None
        gr = g2.gdr2_bwd(q, k, v, g, b, w, h0, do, dht, ws=ws, fwd_saved=saved)
        torch.cuda.synchronize()
        for n in ("dq", "dk", "dg", "db"):
            assert gr[n].shape == (B, 0, H, DK)
        assert torch.equal(gr["dh0"], dht)
    gr = g2.gdr2_bwd(q, k, v, g, b, w, h0, do, None)
    torch.cuda.synchronize()
    assert torch.equal(gr["dh0"], torch.zeros_like(dht))


def test_other_entry_points_without_tokens():
    B, H, DK, DV = 2, 2, 128, 128
    q, k, v, g, b, w, do, h0, dht = tensors(B, 0, H, DK, DV)
    print("T=0 logits / segments / noalloc / step / autograd", flush=True)
    _, ht, _ = g2.gdr2_fwd_logits(q, k, v, g, b, w, h0, g_scale=2.0, b_scale=2.0)
    gr = g2.gdr2_bwd_logits(q, k, v, g, b, w, h0, do, dht, g_scale=2.0, b_scale=2.0)
    torch.cuda.synchronize()
    assert torch.equal(ht, h0) and torch.equal(gr["dh0"], dht)
    _, ht, _ = g2.gdr2_fwd_seg(q, k, v, g, b, w, h0, segments=4, save_for_bwd=True)
    gr = g2.gdr2_bwd_seg(q, k, v, g, b, w, h0, do, dht, segments=4)
    torch.cuda.synchronize()
    assert torch.equal(ht, h0) and torch.equal(gr["dh0"], dht)
    _, ht = g2.gdr2_fwd_noalloc(q, k, v, g, b, w, h0)
    torch.cuda.synchronize()
    assert torch.equal(ht, h0)
    state = h0.clone()
    o = g2.gdr2_step(q, k, v, g, b, w, state)
    torch.cuda.synchronize()
    assert o.shape == (B, 0, H, DV) and torch.equal(state, h0)
    # autograd: o is empty, ht = h0, so dL/dh0 = dL/dht
    h0r = h0.clone().requires_grad_(True)
    o, ht = g2.GDR2Function.apply(q, k, v, g, b, w, h0r)
    (ht * dht).sum().backward()
    torch.cuda.synchronize()
    assert torch.equal(ht.detach(), h0) and torch.equal(h0r.grad, dht)


def test_no_sequences():
    """B = 0 or H = 0: every tensor is empty; the calls succeed and enqueue nothing."""
    for B, H in ((0, 4), (2, 0)):
        print("B=%d H=%d T=64" % (B, H), flush=True)
        q, k, v, g, b, w, do, h0, dht = tensors(B, 64, H, 64, 64)
        o, ht, ws = g2.gdr2_fwd(q, k, v, g, b, w, h0, save_for_bwd=True)
        gr = g2.gdr2_bwd(q, k, v, g, b, w, h0, do, dht, ws=ws, fwd_saved=True)
        torch.cuda.synchronize()
        assert o.numel() == 0 and ht.numel() == 0 and gr["dq"].numel() == 0 and gr["dh0"].numel() == 0
