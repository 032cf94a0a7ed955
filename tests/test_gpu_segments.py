"""Parity of the chunk-parallel scan (gdr2_fwd_seg / gdr2_bwd_seg: the state chains cut
into segments walked at the same time) with the fp64 oracle, through the C ABI.

The segmented path reaches the same quantities as the sequential one through the
composed segment transitions, so it is held to the same tolerances against the oracle:
fp32 inputs max|X - R| / max|R| <= 1e-5, bf16 inputs ||X - R||_F / ||R||_F <= 2e-2."""
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
NAMES = ["q", "k", "v", "g", "b", "w"]
GRADS = ["dq", "dk", "dv", "dg", "db", "dw"]


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


def run_seg(x, segments, dht=None, need_dh0=True):
    args = [x[n] for n in NAMES] + [x["h0"]]
    o, ht, ws = g2.gdr2_fwd_seg(*args, segments=segments, save_for_bwd=True)
    gr = g2.gdr2_bwd_seg(*args, x["do"], dht, segments=segments, ws=ws, fwd_saved=True, need_dh0=need_dh0)
    torch.cuda.synchronize()
    out = {"o": o, "ht": ht}
    out.update(gr)
    return out


def oracle_all(inp, dht, sel=None):
    """Oracle outputs on all sequences, or on the (b, h) pairs in sel, gathered into one call
    (the oracle runs its sequences in parallel) and returned flattened in the order of sel."""
    a = {n: np64(inp[n]) for n in NAMES + ["h0", "do"]}
    dh = np64(dht)
    if sel is None:
        args = [a[n] for n in NAMES]
        h0, do, dhs = a["h0"], a["do"], dh
    else:
        tok = lambda x: np.concatenate([x[bb:bb + 1, :, h:h + 1] for bb, h in sel], axis=2)
        st = lambda x: None if x is None else np.concatenate([x[bb:bb + 1, h:h + 1] for bb, h in sel], axis=1)
        args = [tok(a[n]) for n in NAMES]
        h0, do, dhs = st(a["h0"]), tok(a["do"]), st(dh)
    o, ht = oracle.fwd(*args, h0)
    r = {"o": o, "ht": ht}
    r.update(oracle.bwd(*args, h0, do, dhs))
    if sel is None:
        return r
    # per sequence in the order of sel, flattened and concatenated (as pick() does)
    out = {}
    for k, v in r.items():
        if v is None:
            continue
        v = np.asarray(v)
        parts = [(v[:, i:i + 1] if k in ("ht", "dh0") else v[:, :, i:i + 1]).ravel() for i in range(len(sel))]
        out[k] = np.concatenate(parts)
    return out


def pick(x, key, sel):
    x = np64(x)
    if sel is None:
        return x
    return np.concatenate([(x[bb:bb + 1, h:h + 1] if key in ("ht", "dh0") else x[bb:bb + 1, :, h:h + 1]).ravel()
                           for bb, h in sel])


CASES = [
    # (shape, segments): several chunks per segment, a short last segment, one chunk per
    # segment, more segments than chunks, a ragged last chunk
    (dict(DK=128, DV=128, T=1000, dtype="bf16", B=1, H=2, h0_std=0.1), 3),
    (dict(DK=128, DV=128, T=1000, dtype="bf16", B=1, H=2, h0_std=0.1), 16),
    (dict(DK=64, DV=128, T=700, dtype="bf16", B=2, H=1), 4),
    (dict(DK=128, DV=64, T=512, dtype="bf16", B=1, H=3, g_scale=0.02), 2),
    (dict(DK=64, DV=64, T=300, dtype="bf16", B=1, H=2), 40),
    (dict(DK=64, DV=64, T=1111, dtype="f32", B=1, H=2, h0_std=0.1), 5),
    (dict(DK=64, DV=64, T=640, dtype="f32", B=2, H=1, b_scale=2.0), 10),
]


def _id(c):
    p, seg = c
    return "-".join("%s%s" % (k, v) for k, v in p.items()) + "-seg%d" % seg


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_segmented_matches_the_oracle(case):
    p, segments = case
    kw = dict(p)
    wl = small(DK=kw.pop("DK"), DV=kw.pop("DV"), T=kw.pop("T"), dtype=kw.pop("dtype"), B=kw.pop("B"),
               H=kw.pop("H"), backward=True, seed=23, **kw)
    inp = make_inputs(wl)
    if inp["h0"] is None:
        inp["h0"] = torch.zeros(wl.B, wl.H, wl.DK, wl.DV)
    dht = torch.from_numpy(np.random.default_rng(3).standard_normal((wl.B, wl.H, wl.DK, wl.DV))).float()
    x = {k: v.cuda() for k, v in inp.items()}
    gpu = run_seg(x, segments, dht.cuda())
    ref = oracle_all(inp, dht)
    for key in ["o", "ht"] + GRADS + ["dh0"]:
        check(key, np64(gpu[key]), ref[key], wl.dtype)


def test_one_segment_is_the_plain_path_bitwise():
    wl = small(DK=128, DV=128, T=600, dtype="bf16", B=1, H=2, h0_std=0.05)
    x = {k: v.cuda() for k, v in make_inputs(wl).items()}
    args = [x[n] for n in NAMES] + [x["h0"]]
    o1, h1, ws1 = g2.gdr2_fwd(*args, save_for_bwd=True)
    g1 = g2.gdr2_bwd(*args, x["do"], ws=ws1, fwd_saved=True)
    s = run_seg(x, 1)
    for key, a in [("o", o1), ("ht", h1)] + [(k, g1[k]) for k in GRADS + ["dh0"]]:
        assert torch.equal(a, s[key]), key


def test_segmented_repeatable_and_recompute_identical():
    wl = small(DK=128, DV=128, T=900, dtype="bf16", B=2, H=2, h0_std=0.05)
    x = {k: v.cuda() for k, v in make_inputs(wl).items()}
    args = [x[n] for n in NAMES] + [x["h0"]]
    a = run_seg(x, 4)
    a = {k: v.clone() for k, v in a.items()}
    b = run_seg(x, 4)
    r = g2.gdr2_bwd_seg(*args, x["do"], segments=4, fwd_saved=False)
    torch.cuda.synchronize()
    for key in ["o", "ht"] + GRADS + ["dh0"]:
        assert torch.equal(a[key], b[key]), key
    for key in GRADS + ["dh0"]:
        assert torch.equal(a[key], r[key]), key


def test_segmented_long_sequence_full_size():
    """The B=1, H=16, T=16384 long-sequence workload (h0, dh0) cut into 8 segments of 32
    chunks, on four sampled sequences (the first and the last among them) that the oracle
    computes on its own; every 64-token chunk of each is held to the bound too, so that an
    error at a segment boundary cannot hide under the whole-tensor norm."""
    wl = WORKLOADS["fwdbwd_bf16_b1h16t16384d128_h0"]
    inp = make_inputs(wl)
    x = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    gpu = run_seg(x, 8)
    sel = sample_sequences(wl, seed_offset=200)
    ref = oracle_all(inp, None, sel=sel)
    for key in ["o", "ht"] + GRADS + ["dh0"]:
        check(key, pick(gpu[key], key, sel), ref[key], wl.dtype)
        if key not in ("ht", "dh0"):
            rs = np.asarray(ref[key]).reshape(len(sel), wl.T, -1)
            for i, (bb, h) in enumerate(sel):
                assert_chunks_close("%s%s" % (key, (bb, h)), np64(gpu[key])[bb, :, h], rs[i], wl.dtype, wl.T)


def test_plain_entry_points_segment_few_sequences():
    """gdr2_fwd / gdr2_bwd cut the chains by themselves when the sequences are few: one
    sequence of 65 chunks takes 4 segments, bitwise the same as gdr2_fwd_seg(4), and
    matches the oracle."""
    wl = small(DK=128, DV=128, T=4100, dtype="bf16", B=1, H=1, h0_std=0.05, seed=29)
    assert g2.gdr2_fwd_workspace_bytes(1, 4100, 1, 128, 128, 64, g2.DTYPE_BF16, True) == \
        g2.gdr2_seg_workspace_bytes(1, 4100, 1, 128, 128, 64, 4, g2.DTYPE_BF16, True)
    inp = make_inputs(wl)
    x = {k: v.cuda() for k, v in inp.items()}
    args = [x[n] for n in NAMES] + [x["h0"]]
    o, ht, ws = g2.gdr2_fwd(*args, save_for_bwd=True)
    gr = g2.gdr2_bwd(*args, x["do"], ws=ws, fwd_saved=True)
    torch.cuda.synchronize()
    plain = {"o": o, "ht": ht}
    plain.update(gr)
    seg = run_seg(x, 4)
    for key in ["o", "ht"] + GRADS + ["dh0"]:
        assert torch.equal(plain[key], seg[key]), key
    ref = oracle_all(inp, None)
    for key in ["o", "ht"] + GRADS + ["dh0"]:
        check(key, np64(plain[key]), ref[key], wl.dtype)


def test_segmented_inference_forward_without_initial_state():
    """An inference forward (no backward arrays in the workspace) with 6 segments and no h0,
    then a training forward + backward with no h0 and no dht: both against the oracle."""
    wl = small(DK=128, DV=128, T=1300, dtype="bf16", B=1, H=2, seed=37)
    inp = make_inputs(wl)
    x = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    args = [x[n] for n in NAMES] + [None]
    ws = torch.empty(g2.gdr2_seg_workspace_bytes(1, 1300, 2, 128, 128, 64, 6, g2.DTYPE_BF16, False),
                     dtype=torch.uint8, device="cuda")
    o, ht, _ = g2.gdr2_fwd_seg(*args, segments=6, save_for_bwd=False, ws=ws)
    torch.cuda.synchronize()
    ref = oracle_all(inp, None)
    check("o", np64(o), ref["o"], wl.dtype)
    check("ht", np64(ht), ref["ht"], wl.dtype)
    tr = run_seg(x, 6, None, need_dh0=False)
    for key in ["o", "ht"] + GRADS:
        check(key, np64(tr[key]), ref[key], wl.dtype)
