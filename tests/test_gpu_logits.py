"""Parity of the gate-logit entry points (gdr2_fwd_logits, gdr2_bwd_logits,
gdr2_step_logits) with the fp64 oracle's logit path, through the C ABI.

The kernels activate the gates themselves (b = b_scale sigmoid(zb), w = sigmoid(zw),
g = -g_scale softplus(zg)) and the backward returns the gradients with respect to the
logits. Tolerances as for the plain entry points: fp32 inputs max|X - R| / max|R| <=
1e-5, bf16 inputs ||X - R||_F / ||R||_F <= 2e-2."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import gated_delta_rule_gdr2_amd as g2
import oracle
from gated_delta_rule_gdr2_amd.inputs import WORKLOADS, make_inputs, small
from parity_util import assert_chunks_close, sample_sequences

pytestmark = pytest.mark.gpu

TOL = {"f32": ("inf", 1e-5), "bf16": ("fro", 2e-2)}
GATES = ["zg", "zb", "zw"]


def err(x, r, kind):
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if kind == "inf":
        return np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-30)
    return np.linalg.norm(x - r) / max(np.linalg.norm(r), 1e-30)


def check(name, x, r, dtype):
    kind, tol = TOL[dtype]
    e = err(x, r, kind)
    print("%-4s %s err %.3e (tol %.0e)" % (name, kind, e, tol), flush=True)
    assert e <= tol, (name, e)


def np64(t):
    return None if t is None else t.detach().float().cpu().double().numpy()


def gpu_args(x):
    return [x[n].cuda() for n in ["q", "k", "v"] + GATES]


def oracle_ref(inp, wl, sel=None, backward=True, dht=None):
    """Oracle outputs on all sequences, or on the (b, h) pairs in sel (lists per key)."""
    a = {n: np64(inp[n]) for n in ["q", "k", "v"] + GATES + ["h0", "do"]}
    dh = np64(dht)
    outs = []
    for s in (sel or [None]):
        if s is None:
            cut = lambda x, st=False: x
        else:
            bb, h = s
            cut = lambda x, st=False: None if x is None else (x[bb:bb + 1, h:h + 1] if st else
                                                               x[bb:bb + 1, :, h:h + 1])
        args = [cut(a[n]) for n in ["q", "k", "v"] + GATES]
        o, ht = oracle.fwd_logits(*args, cut(a["h0"], True), g_scale=wl.g_scale, b_scale=wl.b_scale)
        r = {"o": o, "ht": ht}
        if backward:
            r.update(oracle.bwd_logits(*args, cut(a["h0"], True), cut(a["do"]), cut(dh, True),
                                       g_scale=wl.g_scale, b_scale=wl.b_scale))
        outs.append(r)
    if sel is None:
        return outs[0]
    return {k: [r[k] for r in outs] for k in outs[0]}


def pick(x, key, sel):
    if sel is None:
        return x
    parts = []
    for bb, h in sel:
        parts.append((x[bb:bb + 1, h:h + 1] if key in ("ht", "dh0") else x[bb:bb + 1, :, h:h + 1]).ravel())
    return np.concatenate(parts)


def compare(gpu, ref, dtype, keys, sel=None):
    for key in keys:
        r = ref[key] if sel is None else np.concatenate([np.asarray(v).ravel() for v in ref[key]])
        check(key, pick(gpu[key], key, sel), r, dtype)


CASES = [
    dict(DK=64, DV=64, T=100, dtype="bf16"),
    dict(DK=128, DV=128, T=200, dtype="bf16", h0_std=0.1, b_scale=2.0, g_scale=0.5),
    dict(DK=64, DV=128, T=63, dtype="bf16", B=2, H=3, b_mu=1.0, w_mu=-1.0),
    dict(DK=128, DV=64, T=64, dtype="bf16", B=2, H=2, g_scale=2.0),
    dict(DK=128, DV=128, T=191, dtype="bf16", B=2, H=4, b_scale=1.5),
    dict(DK=64, DV=64, T=130, dtype="f32", h0_std=0.1),
    dict(DK=64, DV=64, T=257, dtype="f32", b_scale=2.0, g_scale=0.5, B=2, H=1),
]


def _id(p):
    return "-".join("%s%s" % (k, v) for k, v in p.items())


def _wl(p, backward=True):
    kw = dict(p)
    return small(DK=kw.pop("DK"), DV=kw.pop("DV"), T=kw.pop("T"), dtype=kw.pop("dtype"),
                 B=kw.pop("B", 1), H=kw.pop("H", 2), backward=backward, seed=17, **kw)


@pytest.mark.parametrize("p", CASES, ids=_id)
def test_logits_forward_and_backward_small(p):
    wl = _wl(p)
    inp = make_inputs(wl, gates="logits")
    if inp["h0"] is None:
        inp["h0"] = torch.zeros(wl.B, wl.H, wl.DK, wl.DV)
    dht = torch.from_numpy(np.random.default_rng(9).standard_normal((wl.B, wl.H, wl.DK, wl.DV))).float()
    args = gpu_args(inp)
    h0, do = inp["h0"].cuda(), inp["do"].cuda()
    sc = dict(g_scale=wl.g_scale, b_scale=wl.b_scale)
    o, ht, ws = g2.gdr2_fwd_logits(*args, h0, save_for_bwd=True, **sc)
    gr = g2.gdr2_bwd_logits(*args, h0, do, dht.cuda(), ws=ws, fwd_saved=True, **sc)
    torch.cuda.synchronize()
    gpu = {"o": np64(o), "ht": np64(ht)}
    gpu.update({k: np64(v) for k, v in gr.items()})
    ref = oracle_ref(inp, wl, dht=dht)
    compare(gpu, ref, wl.dtype, ["o", "ht", "dq", "dk", "dv", "dg", "db", "dw", "dh0"])


def test_logits_recompute_path_identical():
    """gdr2_bwd_logits(fwd_saved=0) recomputes the forward with the same activations."""
    wl = _wl(CASES[1])
    x = make_inputs(wl, gates="logits")
    args = gpu_args(x) + [x["h0"].cuda()]
    sc = dict(g_scale=wl.g_scale, b_scale=wl.b_scale)
    _, _, ws = g2.gdr2_fwd_logits(*args, save_for_bwd=True, **sc)
    g1 = g2.gdr2_bwd_logits(*args, x["do"].cuda(), ws=ws, fwd_saved=True, **sc)
    g1 = {k: v.clone() for k, v in g1.items()}
    g2_ = g2.gdr2_bwd_logits(*args, x["do"].cuda(), fwd_saved=False, **sc)
    torch.cuda.synchronize()
    for key in ["dq", "dk", "dv", "dg", "db", "dw", "dh0"]:
        assert torch.equal(g1[key], g2_[key]), key


@pytest.mark.parametrize("p", [CASES[1], CASES[2], CASES[5]], ids=_id)
def test_step_logits_matches_the_oracle(p):
    wl = _wl(p, backward=False)
    inp = make_inputs(wl, gates="logits")
    if inp["h0"] is None:
        inp["h0"] = torch.zeros(wl.B, wl.H, wl.DK, wl.DV)
    state = inp["h0"].cuda().clone()
    o = g2.gdr2_step_logits(*gpu_args(inp), state, g_scale=wl.g_scale, b_scale=wl.b_scale)
    torch.cuda.synchronize()
    ref = oracle_ref(inp, wl, backward=False)
    compare({"o": np64(o), "ht": np64(state)}, ref, wl.dtype, ["o", "ht"])


def test_logits_training_shape_full_size():
    """The B=2, H=16, T=4096, d=128 bf16 training shape with logits in, on two sampled
    sequences that the oracle computes on its own; b in the [0, 2] erase range."""
    wl = replace(WORKLOADS["fwdbwd_bf16_b2h16t4096d128"], seed=41, b_scale=2.0)
    inp = make_inputs(wl, gates="logits")
    args = gpu_args(inp)
    sc = dict(g_scale=wl.g_scale, b_scale=wl.b_scale)
    o, ht, ws = g2.gdr2_fwd_logits(*args, None, save_for_bwd=True, **sc)
    gr = g2.gdr2_bwd_logits(*args, None, inp["do"].cuda(), ws=ws, fwd_saved=True, need_dh0=False, **sc)
    torch.cuda.synchronize()
    gpu = {"o": np64(o), "ht": np64(ht)}
    gpu.update({k: np64(v) for k, v in gr.items() if v is not None})
    sel = sample_sequences(wl)
    ref = oracle_ref(inp, wl, sel=sel)
    compare(gpu, ref, wl.dtype, ["o", "ht", "dq", "dk", "dv", "dg", "db", "dw"], sel=sel)
    for key in ["o", "dq", "dk", "dv", "dg", "db", "dw"]:
        for s, rv in zip(sel, ref[key]):
            bb, h = s
            assert_chunks_close("%s%s" % (key, s), gpu[key][bb, :, h], np.asarray(rv).reshape(wl.T, -1), wl.dtype,
                                wl.T)


@pytest.mark.parametrize("dtype,DK,DV", [("bf16", 128, 128), ("f32", 64, 64)])
def test_logits_strong_decay(dtype, DK, DV):
    """g_scale = 10: g = -10 softplus(zg) runs from about -0.5 to below -30 per token, so
    most 16-token blocks exceed the range of the block-split factors and take the
    per-element diagonal path; forward and backward against the oracle, all finite."""
    wl = small(DK=DK, DV=DV, T=150, dtype=dtype, B=2, H=2, h0_std=0.1, g_scale=10.0, b_scale=2.0, seed=19)
    inp = make_inputs(wl, gates="logits")
    dht = torch.from_numpy(np.random.default_rng(9).standard_normal((wl.B, wl.H, wl.DK, wl.DV))).float()
    args = gpu_args(inp)
    h0, do = inp["h0"].cuda(), inp["do"].cuda()
    sc = dict(g_scale=wl.g_scale, b_scale=wl.b_scale)
    o, ht, ws = g2.gdr2_fwd_logits(*args, h0, save_for_bwd=True, **sc)
    gr = g2.gdr2_bwd_logits(*args, h0, do, dht.cuda(), ws=ws, fwd_saved=True, **sc)
    torch.cuda.synchronize()
    gpu = {"o": np64(o), "ht": np64(ht)}
    gpu.update({k: np64(v) for k, v in gr.items()})
    for k, v in gpu.items():
        assert np.all(np.isfinite(v)), k
    ref = oracle_ref(inp, wl, dht=dht)
    compare(gpu, ref, wl.dtype, ["o", "ht", "dq", "dk", "dv", "dg", "db", "dw", "dh0"])


def test_logits_with_automatic_segments():
    """One sequence of 65 chunks: the logit entry points cut the chains into segments by
    themselves (as gdr2_fwd / gdr2_bwd do), with the gates activated in the kernels."""
    wl = small(DK=128, DV=128, T=4100, dtype="bf16", B=1, H=1, h0_std=0.05, seed=43, b_scale=2.0, g_scale=0.3)
    assert g2.gdr2_fwd_workspace_bytes(1, 4100, 1, 128, 128, 64, g2.DTYPE_BF16, True) == \
        g2.gdr2_seg_workspace_bytes(1, 4100, 1, 128, 128, 64, 4, g2.DTYPE_BF16, True)  # 4 segments
    inp = make_inputs(wl, gates="logits")
    args = gpu_args(inp)
    h0, do = inp["h0"].cuda(), inp["do"].cuda()
    sc = dict(g_scale=wl.g_scale, b_scale=wl.b_scale)
    o, ht, ws = g2.gdr2_fwd_logits(*args, h0, save_for_bwd=True, **sc)
    gr = g2.gdr2_bwd_logits(*args, h0, do, ws=ws, fwd_saved=True, **sc)
    torch.cuda.synchronize()
    gpu = {"o": np64(o), "ht": np64(ht)}
    gpu.update({k: np64(v) for k, v in gr.items()})
    ref = oracle_ref(inp, wl)
    compare(gpu, ref, wl.dtype, ["o", "ht", "dq", "dk", "dv", "dg", "db", "dw", "dh0"])


@pytest.mark.parametrize("p", [CASES[1], CASES[5]], ids=_id)
def test_logits_in_the_tails(p):
    """A fifth of the logits far in the tails: z_b, z_w = +-30 (gates exactly off or fully on,
    zero derivative), z_g from -30 (no decay) to 12 (decay g_scale * 12 per token); the rest
    as drawn. Forward and backward against the oracle."""
    wl = _wl(p)
    inp = make_inputs(wl, gates="logits")
    if inp["h0"] is None:
        inp["h0"] = torch.zeros(wl.B, wl.H, wl.DK, wl.DV)
    rng = np.random.default_rng(77)
    for n, lo, hi in (("zb", None, None), ("zw", None, None), ("zg", -30.0, 12.0)):
        z = inp[n].float().numpy().copy()
        m = rng.random(z.shape) < 0.2
        if lo is None:
            z[m] = np.where(rng.random(int(m.sum())) < 0.5, -30.0, 30.0)
        else:
            z[m] = rng.uniform(lo, hi, int(m.sum()))
        inp[n] = torch.from_numpy(z).to(inp[n].dtype)
    dht = torch.from_numpy(np.random.default_rng(9).standard_normal((wl.B, wl.H, wl.DK, wl.DV))).float()
    args = gpu_args(inp)
    h0, do = inp["h0"].cuda(), inp["do"].cuda()
    sc = dict(g_scale=wl.g_scale, b_scale=wl.b_scale)
    o, ht, ws = g2.gdr2_fwd_logits(*args, h0, save_for_bwd=True, **sc)
    gr = g2.gdr2_bwd_logits(*args, h0, do, dht.cuda(), ws=ws, fwd_saved=True, **sc)
    torch.cuda.synchronize()
    gpu = {"o": np64(o), "ht": np64(ht)}
    gpu.update({k: np64(v) for k, v in gr.items()})
    for k, v in gpu.items():
        assert np.all(np.isfinite(v)), k
    ref = oracle_ref(inp, wl, dht=dht)
    compare(gpu, ref, wl.dtype, ["o", "ht", "dq", "dk", "dv", "dg", "db", "dw", "dh0"])
