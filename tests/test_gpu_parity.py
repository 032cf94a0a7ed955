"""Parity of the HIP path (called through the C ABI) with the fp64 oracle.

Tolerances (per output tensor X against the oracle R computed in fp64 from the
same rounded inputs):
  fp32 inputs : max|X - R| / max|R|  <= 1e-5
  bf16 inputs : ||X - R||_F / ||R||_F <= 2e-2   (fp32 state)
and, for bf16 token tensors of a sampled full-size workload, the same normwise
bound on every 64-token chunk of every sampled sequence, so that an error
confined to a few chunks (a late chain step, the last chunk, a segment boundary)
cannot hide under the whole-tensor norm. Small cases compare every element and
cover several chunks, ragged tails and every supported (dk, dv); the five
benchmark workloads run at full size in the same launch configuration the
benchmark times, and are compared on sampled (batch, head) sequences -- always
the first and the last, plus two more -- which the oracle computes on its own.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import gated_delta_rule_gdr2_amd as g2
import oracle
from gated_delta_rule_gdr2_amd.inputs import WORKLOADS, make_inputs, small

pytestmark = pytest.mark.gpu

from parity_util import TOL, assert_chunks_close, rel_err, sample_sequences


def assert_close(name, x, r, dtype):
    kind, tol = TOL[dtype]
    e = rel_err(x, r, kind)
    print("%-4s %s err %.3e (tol %.0e)" % (name, kind, e, tol), flush=True)
    assert e <= tol, (name, e)


def np64(t):
    return None if t is None else t.detach().float().cpu().double().numpy()


def to_gpu(inp):
    return {k: (None if v is None else v.cuda()) for k, v in inp.items()}


def run_gpu(inp, backward, dht=None, fwd_saved=True):
    x = to_gpu(inp)
    o, ht, ws = g2.gdr2_fwd(x["q"], x["k"], x["v"], x["g"], x["b"], x["w"], x["h0"],
                            save_for_bwd=backward and fwd_saved)
    out = {"o": o, "ht": ht}
    if backward:
        gr = g2.gdr2_bwd(x["q"], x["k"], x["v"], x["g"], x["b"], x["w"], x["h0"], x["do"],
                         None if dht is None else dht.cuda(), ws=ws if fwd_saved else None,
                         fwd_saved=fwd_saved)
        out.update(gr)
    torch.cuda.synchronize()
    return {k: np64(v) for k, v in out.items()}


def run_oracle(inp, backward, dht=None, sel=None):
    """Oracle on the (b, h) sequences listed in sel (all when None). The selected
    sequences are gathered into one call (the oracle runs its sequences in parallel)."""
    names = ["q", "k", "v", "g", "b", "w"]
    arrs = {n: np64(inp[n]) for n in names}
    h0 = np64(inp["h0"])
    do = np64(inp["do"]) if backward else None
    dh = np64(dht)
    if sel is None:
        o, ht = oracle.fwd(*(arrs[n] for n in names), h0)
        res = {"o": o, "ht": ht}
        if backward:
            res.update(oracle.bwd(*(arrs[n] for n in names), h0, do, dh))
        return res

    def gather(x, state=False):
        if x is None:
            return None
        if state:
            return np.concatenate([x[bb:bb + 1, h:h + 1] for bb, h in sel], axis=1)
        return np.concatenate([x[bb:bb + 1, :, h:h + 1] for bb, h in sel], axis=2)

    a = {n: gather(arrs[n]) for n in names}
    hh, dd, dhs = gather(h0, True), gather(do), gather(dh, True)
    o, ht = oracle.fwd(*(a[n] for n in names), hh)
    r = {"o": o, "ht": ht}
    if backward:
        r.update(oracle.bwd(*(a[n] for n in names), hh, dd, dhs))
    # back to per-sequence pieces, in the order of sel
    res = {}
    for key, v in r.items():
        if v is None:
            continue
        res[key] = [v[:, :, i:i + 1] if key not in ("ht", "dh0") else v[:, i:i + 1] for i in range(len(sel))]
    return res


def gpu_slice(x, key, s):
    bb, h = s
    if key in ("ht", "dh0"):
        return x[bb:bb + 1, h:h + 1]
    return x[bb:bb + 1, :, h:h + 1]


TOKEN_KEYS = ("o", "dq", "dk", "dv", "dg", "db", "dw")


def compare(gpu, ref, dtype, backward, sel=None, has_h0=True, keys=None, chunks=None):
    """Whole-tensor bounds; with chunks = T also the bound on every 64-token chunk of every
    sampled sequence (bf16 token tensors)."""
    if keys is None:
        keys = ["o", "ht"] + (["dq", "dk", "dv", "dg", "db", "dw"] + (["dh0"] if has_h0 else []) if backward else [])
    for key in keys:
        if sel is None:
            assert_close(key, gpu[key], ref[key], dtype)
        else:
            x = np.concatenate([gpu_slice(gpu[key], key, s).ravel() for s in sel])
            r = np.concatenate([np.asarray(v).ravel() for v in ref[key]])
            assert_close(key, x, r, dtype)
            if chunks and key in TOKEN_KEYS and dtype == "bf16":
                for s, rv in zip(sel, ref[key]):
                    assert_chunks_close("%s%s" % (key, s), gpu_slice(gpu[key], key, s), rv, dtype, chunks)


SMALL = [
    dict(DK=64, DV=64, T=100, dtype="bf16"),
    dict(DK=128, DV=128, T=200, dtype="bf16", h0_std=0.1),
    dict(DK=64, DV=128, T=130, dtype="bf16"),
    dict(DK=128, DV=64, T=64, dtype="bf16", B=2, H=3),
    dict(DK=128, DV=128, T=1, dtype="bf16", h0_std=0.1),
    dict(DK=128, DV=128, T=63, dtype="bf16", g_scale=2.0),
    dict(DK=64, DV=64, T=100, dtype="f32"),
    dict(DK=64, DV=64, T=257, dtype="f32", h0_std=0.1, B=2, H=1),
    # many sequences whose last chunk is one token short / about half full: the padding
    # rows that the backward kernel stages and zeroes in LDS
    dict(DK=128, DV=128, T=191, dtype="bf16", B=2, H=8),
    dict(DK=64, DV=128, T=100, dtype="bf16", B=4, H=4),
    # the [0, 2] erase range: b = 2 sigmoid(.), negative eigenvalues of the transition
    dict(DK=128, DV=128, T=200, dtype="bf16", b_scale=2.0, h0_std=0.1),
    dict(DK=64, DV=64, T=130, dtype="f32", b_scale=2.0),
]


def _id(p):
    return "-".join("%s%s" % (k, v) for k, v in p.items())


@pytest.mark.parametrize("p", SMALL, ids=_id)
def test_forward_small(p):
    kw = dict(p)
    wl = small(DK=kw.pop("DK"), DV=kw.pop("DV"), T=kw.pop("T"), dtype=kw.pop("dtype"),
               B=kw.pop("B", 1), H=kw.pop("H", 2), backward=False, **kw)
    inp = make_inputs(wl)
    compare(run_gpu(inp, False), run_oracle(inp, False), wl.dtype, False)


@pytest.mark.parametrize("p", SMALL, ids=_id)
def test_backward_small(p):
    kw = dict(p)
    wl = small(DK=kw.pop("DK"), DV=kw.pop("DV"), T=kw.pop("T"), dtype=kw.pop("dtype"),
               B=kw.pop("B", 1), H=kw.pop("H", 2), backward=True, **kw)
    inp = make_inputs(wl)
    if inp["h0"] is None:
        inp["h0"] = torch.zeros(wl.B, wl.H, wl.DK, wl.DV)
    dht = torch.from_numpy(np.random.default_rng(5).standard_normal((wl.B, wl.H, wl.DK, wl.DV))).float()
    compare(run_gpu(inp, True, dht), run_oracle(inp, True, dht), wl.dtype, True)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_full_size(name):
    wl = WORKLOADS[name]
    inp = make_inputs(wl)
    gpu = run_gpu(inp, wl.backward)
    sel = None if wl.B * wl.H * wl.T <= 4096 else sample_sequences(wl)
    ref = run_oracle(inp, wl.backward, sel=sel)
    compare(gpu, ref, wl.dtype, wl.backward, sel=sel, has_h0=inp["h0"] is not None, chunks=wl.T)


def test_erase_range_two_full_size():
    """The headline training shape with the [0, 2] erase range (b = 2 sigmoid(N(0, 1)))."""
    wl = replace(WORKLOADS["fwdbwd_bf16_b2h16t4096d128"], b_scale=2.0, seed=33)
    inp = make_inputs(wl)
    gpu = run_gpu(inp, True)
    sel = sample_sequences(wl)
    ref = run_oracle(inp, True, sel=sel)
    compare(gpu, ref, wl.dtype, True, sel=sel, has_h0=False, chunks=wl.T)


@pytest.mark.parametrize("p", [dict(DK=128, DV=128, T=150, dtype="bf16", B=2, H=3, h0_std=0.1),
                               dict(DK=64, DV=64, T=130, dtype="f32", B=1, H=2, h0_std=0.1)], ids=_id)
def test_recompute_backward_small(p):
    """gdr2_bwd(fwd_saved=0) -- the backward that recomputes the forward inside the call --
    against the oracle on a small ragged case with h0 and dht."""
    kw = dict(p)
    wl = small(DK=kw.pop("DK"), DV=kw.pop("DV"), T=kw.pop("T"), dtype=kw.pop("dtype"),
               B=kw.pop("B"), H=kw.pop("H"), backward=True, seed=71, **kw)
    inp = make_inputs(wl)
    dht = torch.from_numpy(np.random.default_rng(8).standard_normal((wl.B, wl.H, wl.DK, wl.DV))).float()
    gpu = run_gpu(inp, True, dht, fwd_saved=False)
    ref = run_oracle(inp, True, dht)
    compare(gpu, ref, wl.dtype, True, keys=["dq", "dk", "dv", "dg", "db", "dw", "dh0"])


def test_recompute_backward_full_size():
    """gdr2_bwd(fwd_saved=0) at the headline training shape, on sampled sequences."""
    wl = WORKLOADS["fwdbwd_bf16_b2h16t4096d128"]
    inp = make_inputs(wl)
    gpu = run_gpu(inp, True, fwd_saved=False)
    sel = sample_sequences(wl)
    ref = run_oracle(inp, True, sel=sel)
    compare(gpu, ref, wl.dtype, True, sel=sel, has_h0=False, chunks=wl.T,
            keys=["dq", "dk", "dv", "dg", "db", "dw"])


def test_fp32_at_a_streaming_store_size():
    """fp32 at d = 64 with a training workspace past the library's 128 MiB threshold (B2 H16
    T2048 with h0: 163 MiB), so every kernel runs its non-temporal-store instantiation, which
    the small fp32 cases never reach: sampled sequences, the last included, against the
    oracle at the fp32 tolerance."""
    wl = small(name="f32_stream", DK=64, DV=64, T=2048, dtype="f32", B=2, H=16, backward=True, seed=91,
               h0_std=0.1)
    assert g2.gdr2_fwd_workspace_bytes(wl.B, wl.T, wl.H, wl.DK, wl.DV, dtype=g2.DTYPE_F32,
                                       save_for_bwd=True) >= 128 << 20
    inp = make_inputs(wl)
    gpu = run_gpu(inp, True)
    sel = sample_sequences(wl)
    ref = run_oracle(inp, True, sel=sel)
    compare(gpu, ref, wl.dtype, True, sel=sel, has_h0=True)


def test_state_size_matches_the_pages():
    """262,144 state floats per layer for H = 16, d_k = d_v = 128 (LIT-802 takeaway 3)."""
    wl = WORKLOADS["fwd_bf16_b1h16t2048d128_h0"]
    inp = to_gpu(make_inputs(wl))
    _, ht, _ = g2.gdr2_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["b"], inp["w"], inp["h0"])
    assert ht[0].numel() == 262144


def test_deterministic_and_recompute_path_identical():
    wl = small(DK=128, DV=128, T=300, dtype="bf16", B=1, H=3, h0_std=0.05)
    x = to_gpu(make_inputs(wl))
    args = (x["q"], x["k"], x["v"], x["g"], x["b"], x["w"], x["h0"])
    o1, h1, ws = g2.gdr2_fwd(*args, save_for_bwd=True)
    g1 = g2.gdr2_bwd(*args, x["do"], ws=ws, fwd_saved=True)
    o2, h2, _ = g2.gdr2_fwd(*args, save_for_bwd=True)
    g2_ = g2.gdr2_bwd(*args, x["do"], fwd_saved=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    for key in ["dq", "dk", "dv", "dg", "db", "dw", "dh0"]:
        assert torch.equal(g1[key], g2_[key]), key


def test_ragged_backward_repeatable():
    """A partial last chunk gives the same gradients, bitwise, on repeated calls."""
    wl = small(DK=128, DV=128, T=127, dtype="bf16", B=4, H=8, h0_std=0.05)
    x = to_gpu(make_inputs(wl))
    args = (x["q"], x["k"], x["v"], x["g"], x["b"], x["w"], x["h0"])
    _, _, ws = g2.gdr2_fwd(*args, save_for_bwd=True)
    first = g2.gdr2_bwd(*args, x["do"], ws=ws, fwd_saved=True)
    first = {k: v.clone() for k, v in first.items()}
    for _ in range(3):
        again = g2.gdr2_bwd(*args, x["do"], ws=ws, fwd_saved=True)
        torch.cuda.synchronize()
        for key in ["dq", "dk", "dv", "dg", "db", "dw", "dh0"]:
            assert torch.equal(first[key], again[key]), key


def test_split_invariance_on_gpu():
    """Only the state is carried between chunks (digg thread post 9/): two calls chained through
    ht == one call, bitwise when the split falls on a chunk boundary."""
    wl = small(DK=128, DV=128, T=320, dtype="bf16", B=1, H=2, h0_std=0.05, backward=False)
    x = to_gpu(make_inputs(wl))
    names = ["q", "k", "v", "g", "b", "w"]
    o, ht, _ = g2.gdr2_fwd(*(x[n] for n in names), x["h0"])
    T1 = 128
    oa, ha, _ = g2.gdr2_fwd(*(x[n][:, :T1].contiguous() for n in names), x["h0"])
    ob, hb, _ = g2.gdr2_fwd(*(x[n][:, T1:].contiguous() for n in names), ha)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([oa, ob], 1), o) and torch.equal(hb, ht)


def test_gate_product_identity_on_gpu():
    """x = w*v, so dv*v = dw*w (up to the rounding of the two bf16 outputs)."""
    wl = small(DK=128, DV=128, T=192, dtype="bf16", B=1, H=2)
    inp = make_inputs(wl)
    out = run_gpu(inp, True)
    v, w = np64(inp["v"]), np64(inp["w"])
    assert rel_err(out["dv"] * v, out["dw"] * w, "fro") < 1e-2


def test_autograd_function_matches_direct_calls():
    wl = small(DK=64, DV=64, T=96, dtype="bf16", B=1, H=2, h0_std=0.1)
    x = to_gpu(make_inputs(wl))
    ts = [x[n].clone().requires_grad_(True) for n in ["q", "k", "v", "g", "b", "w"]]
    h0 = x["h0"].clone().requires_grad_(True)
    o, ht = g2.GDR2Function.apply(*ts, h0)
    (o.float() * x["do"].float()).sum().backward()
    gr = g2.gdr2_bwd(*(x[n] for n in ["q", "k", "v", "g", "b", "w"]), x["h0"], x["do"])
    torch.cuda.synchronize()
    for t, key in zip(ts + [h0], ["dq", "dk", "dv", "dg", "db", "dw", "dh0"]):
        assert torch.equal(t.grad, gr[key]), key


DEGENERATE = [
    # no erase: decayed linear attention (b = 0)
    ("no_erase", dict(b=0.0)),
    # no decay and the gates fully open (g = 0, b = w = 1): the delta rule that overwrites
    ("overwrite", dict(g=0.0, b=1.0, w=1.0)),
    # strong forgetting at every token and channel, from moderate to far past the point where
    # the block-split factor exp(-15 g) of a 16-token block leaves the fp32 range (g < -5.9):
    # the diagonal blocks take the per-element path there
    ("forget_1p5", dict(g=-1.5)),
    ("forget_5p5", dict(g=-5.5)),
    ("forget_8", dict(g=-8.0)),
    ("forget_20", dict(g=-20.0)),
    ("forget_50", dict(g=-50.0)),
    # zero keys: nothing is written or erased; the state only decays and is read out
    ("zero_keys", dict(k=0.0)),
]


@pytest.mark.parametrize("dtype,DK,DV", [("bf16", 128, 128), ("f32", 64, 64)])
@pytest.mark.parametrize("name,fill", DEGENERATE, ids=[d[0] for d in DEGENERATE])
def test_degenerate_gates(dtype, DK, DV, name, fill):
    """Special cases of the recurrence with closed forms, forward and backward against the oracle."""
    wl = small(DK=DK, DV=DV, T=150, dtype=dtype, B=1, H=2, h0_std=0.1, backward=True, seed=53)
    inp = make_inputs(wl)
    for key, val in fill.items():
        inp[key] = torch.full_like(inp[key], val[dtype] if isinstance(val, dict) else val)
    dht = torch.from_numpy(np.random.default_rng(6).standard_normal((wl.B, wl.H, wl.DK, wl.DV))).float()
    gpu = run_gpu(inp, True, dht)
    for k, v in gpu.items():
        assert v is None or np.all(np.isfinite(v)), k
    ref = run_oracle(inp, True, dht)
    compare(gpu, ref, wl.dtype, True)


@pytest.mark.parametrize("dtype,DK,DV,T", [("bf16", 128, 128, 200), ("f32", 64, 64, 150), ("bf16", 64, 128, 97)])
def test_mixed_strong_and_weak_decay(dtype, DK, DV, T):
    """Some channels forget at g = -30 per token, some at -3, the rest as drawn (weak); a random
    tenth of the tokens decays at -60 on every channel; ragged last chunk. Mixed chunks where
    only some blocks or channels need the per-element diagonal path."""
    wl = small(DK=DK, DV=DV, T=T, dtype=dtype, B=2, H=2, h0_std=0.1, backward=True, seed=57)
    inp = make_inputs(wl)
    g = inp["g"].float().numpy().copy()
    g[..., 0::4] = -30.0
    g[..., 1::8] = -3.0
    rows = np.random.default_rng(58).random(g.shape[:3]) < 0.1
    g[rows] = -60.0
    inp["g"] = torch.from_numpy(g).to(inp["g"].dtype)
    dht = torch.from_numpy(np.random.default_rng(7).standard_normal((wl.B, wl.H, wl.DK, wl.DV))).float()
    gpu = run_gpu(inp, True, dht)
    for k, v in gpu.items():
        assert v is None or np.all(np.isfinite(v)), k
    ref = run_oracle(inp, True, dht)
    compare(gpu, ref, wl.dtype, True)


MANY_SHORT = [
    # many sequences of two or three chunks, the last ragged: large grids, every sequence's
    # last chunk partial, random h0 and dht. With 512 or more 16-column chain walks the chains
    # run 32-column slices (all but the 8 x 8 fp32 case); every d_k / d_v and both dtypes.
    dict(DK=128, DV=128, T=65, dtype="bf16", B=16, H=16, h0_std=0.05),
    dict(DK=64, DV=64, T=70, dtype="f32", B=8, H=8, h0_std=0.05),
    dict(DK=64, DV=64, T=70, dtype="f32", B=8, H=16, h0_std=0.05),
    dict(DK=64, DV=64, T=130, dtype="bf16", B=8, H=16, h0_std=0.05),
    dict(DK=128, DV=64, T=100, dtype="bf16", B=8, H=16),
    dict(DK=64, DV=128, T=100, dtype="bf16", B=4, H=16, h0_std=0.05),
]


@pytest.mark.parametrize("p", MANY_SHORT, ids=lambda p: "-".join("%s%s" % kv for kv in p.items()))
def test_many_short_sequences(p):
    kw = dict(p)
    wl = small(DK=kw.pop("DK"), DV=kw.pop("DV"), T=kw.pop("T"), dtype=kw.pop("dtype"), B=kw.pop("B"),
               H=kw.pop("H"), backward=True, seed=61, **kw)
    inp = make_inputs(wl)
    dht = torch.from_numpy(np.random.default_rng(5).standard_normal((wl.B, wl.H, wl.DK, wl.DV))).float()
    gpu = run_gpu(inp, True, dht)
    rng = np.random.default_rng(wl.seed + 300)
    sel = sorted({(int(rng.integers(wl.B)), int(rng.integers(wl.H))) for _ in range(6)})
    ref = run_oracle(inp, True, dht, sel=sel)
    compare(gpu, ref, wl.dtype, True, sel=sel)
