"""Pins for the fp64 oracle, each tied to something other than the oracle itself.

Every test here runs on the CPU. The operator is the Gated Delta Rule-2
recurrence (anthology record LIT-802, "Key takeaways", first bullet; paper
Sec. 3.1 Eqs. 8-10). The pins are:
  * a hand-worked scalar example (tests/golden/scalar_worked_example.json);
  * the reductions the pages state: tied gates b = w = beta*1 give KDA exactly,
    a scalar decay on top gives Gated DeltaNet (LIT-802 takeaway 1, App. A.5;
    chatpaper abstract), and g = 0 gives the delta rule
    S <- (I - beta k k^T) S + beta k v^T (digg thread, post 7/);
  * the overwrite property of the delta rule (digg thread, posts 7/-8/: the
    step reads what the key returns and writes the difference; at full
    strength it overwrites);
  * closed forms: with b = 0 the erase vanishes and the operator is decayed
    linear attention, with g = 0 a masked matrix product;
  * invariants: linearity in (v, h0), dependence on v and w through w*v only,
    split invariance (only the state is carried between chunks, digg thread
    post 9/), zero-token padding;
  * brute force with dense transition matrices for T <= 8;
  * for the backward: central finite differences, a torch-autograd token loop
    written separately, the KDA gradient identity and the w*v product identity.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_inputs(rng, B, T, H, DK, DV, gscale=0.3, h0=True, normalize=True):
    q = rng.standard_normal((B, T, H, DK))
    k = rng.standard_normal((B, T, H, DK))
    if normalize:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, DV))
    g = -np.logaddexp(0, rng.standard_normal((B, T, H, DK))) * gscale
    b = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, DK))))
    w = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, DV))))
    hh = rng.standard_normal((B, H, DK, DV)) * 0.3 if h0 else None
    return q, k, v, g, b, w, hh


def relerr(x, r):
    return np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-300)


# ----------------------------------------------------------------------------- forward pins

def test_scalar_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "scalar_worked_example.json")))
    toks = ex["tokens"]
    T = len(toks)
    arr = lambda key: np.array([t[key] for t in toks], dtype=np.float64).reshape(1, T, 1, 1)
    g = np.log(arr("alpha"))
    o, ht = oracle.fwd(arr("q"), arr("k"), arr("v"), g, arr("b"), arr("w"))
    np.testing.assert_allclose(o.reshape(-1), ex["o"], rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(ht.reshape(()), ex["S_final"], rtol=1e-15)


def brute_force(q, k, v, g, b, w, h0):
    """Dense transition matrices E_t = (I - k_t (b_t*k_t)^T) diag(exp g_t) for one sequence:
    S_t = E_t S_{t-1} + k_t (w_t*v_t)^T, expanded as products of E's."""
    T, DK = q.shape
    DV = v.shape[1]
    E = [(np.eye(DK) - np.outer(k[t], b[t] * k[t])) @ np.diag(np.exp(g[t])) for t in range(T)]
    Wr = [np.outer(k[t], w[t] * v[t]) for t in range(T)]
    o = np.zeros((T, DV))
    for t in range(T):
        prod = np.eye(DK)
        St = np.zeros((DK, DV))
        for i in range(t, -1, -1):  # S_t = sum_i (E_t ... E_{i+1}) Wr_i + (E_t ... E_1) h0
            St += prod @ Wr[i]
            prod = prod @ E[i]
        St += prod @ h0
        o[t] = St.T @ q[t]
    return o, St


@pytest.mark.parametrize("DK,DV,T", [(3, 2, 7), (8, 8, 8), (1, 4, 5)])
def test_brute_force_unrolled_products(DK, DV, T):
    rng = np.random.default_rng(100 + DK * 10 + DV)
    q, k, v, g, b, w, h0 = rand_inputs(rng, 1, T, 1, DK, DV, normalize=False)
    o, ht = oracle.fwd(q, k, v, g, b, w, h0)
    ob, Sb = brute_force(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], b[0, :, 0], w[0, :, 0], h0[0, 0])
    assert relerr(o[0, :, 0], ob) < 1e-13
    assert relerr(ht[0, 0], Sb) < 1e-13


def kda_reference(q, k, v, g, beta, h0):
    """Kimi Delta Attention written in its own form: S <- (I - beta k k^T) diag(alpha) S + beta k v^T."""
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    o = np.zeros((B, T, H, DV))
    S_all = np.zeros((B, H, DK, DV))
    for bb in range(B):
        for h in range(H):
            S = h0[bb, h].copy() if h0 is not None else np.zeros((DK, DV))
            for t in range(T):
                kt, bt = k[bb, t, h], beta[bb, t, h]
                S = (np.eye(DK) - bt * np.outer(kt, kt)) @ (np.exp(g[bb, t, h])[:, None] * S) \
                    + bt * np.outer(kt, v[bb, t, h])
                o[bb, t, h] = S.T @ q[bb, t, h]
            S_all[bb, h] = S
    return o, S_all


def test_reduces_to_kda_with_tied_gates():
    rng = np.random.default_rng(1)
    B, T, H, DK, DV = 2, 37, 2, 6, 5
    q, k, v, g, _, _, h0 = rand_inputs(rng, B, T, H, DK, DV)
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    b = np.repeat(beta[..., None], DK, -1)
    w = np.repeat(beta[..., None], DV, -1)
    o, ht = oracle.fwd(q, k, v, g, b, w, h0)
    ok, Sk = kda_reference(q, k, v, g, beta, h0)
    assert relerr(o, ok) < 1e-13 and relerr(ht, Sk) < 1e-13


def gdn_reference(q, k, v, a, beta, h0):
    """Gated DeltaNet in its own form: S <- a (I - beta k k^T) S + beta k v^T, scalar a per token."""
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    o = np.zeros((B, T, H, DV))
    S_all = np.zeros((B, H, DK, DV))
    for bb in range(B):
        for h in range(H):
            S = h0[bb, h].copy() if h0 is not None else np.zeros((DK, DV))
            for t in range(T):
                kt, bt = k[bb, t, h], beta[bb, t, h]
                S = a[bb, t, h] * (S - bt * np.outer(kt, kt @ S)) + bt * np.outer(kt, v[bb, t, h])
                o[bb, t, h] = S.T @ q[bb, t, h]
            S_all[bb, h] = S
    return o, S_all


def test_reduces_to_gated_deltanet_with_scalar_decay():
    rng = np.random.default_rng(2)
    B, T, H, DK, DV = 1, 41, 3, 7, 4
    q, k, v, _, _, _, h0 = rand_inputs(rng, B, T, H, DK, DV)
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    a = np.exp(-np.logaddexp(0, rng.standard_normal((B, T, H))) * 0.3)
    g = np.repeat(np.log(a)[..., None], DK, -1)
    o, ht = oracle.fwd(q, k, v, g, np.repeat(beta[..., None], DK, -1), np.repeat(beta[..., None], DV, -1), h0)
    og, Sg = gdn_reference(q, k, v, a, beta, h0)
    assert relerr(o, og) < 1e-13 and relerr(ht, Sg) < 1e-13


def test_reduces_to_delta_rule_without_decay():
    rng = np.random.default_rng(3)
    B, T, H, DK, DV = 1, 30, 1, 5, 5
    q, k, v, _, _, _, _ = rand_inputs(rng, B, T, H, DK, DV)
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    g = np.zeros((B, T, H, DK))
    o, ht = oracle.fwd(q, k, v, g, np.repeat(beta[..., None], DK, -1), np.repeat(beta[..., None], DV, -1))
    S = np.zeros((DK, DV))
    for t in range(T):  # S <- (I - beta k k^T) S + beta k v^T
        kt, bt = k[0, t, 0], beta[0, t, 0]
        S = S - bt * np.outer(kt, kt @ S) + bt * np.outer(kt, v[0, t, 0])
        assert relerr(o[0, t, 0], S.T @ q[0, t, 0]) < 1e-13
    assert relerr(ht[0, 0], S) < 1e-13


def test_overwrite_property():
    """When sum_c b_c k_c^2 = 1 the read along b*k after the step returns exactly w*v."""
    rng = np.random.default_rng(4)
    B, T, H, DK, DV = 1, 25, 2, 8, 6
    _, k, v, g, b, w, h0 = rand_inputs(rng, B, T, H, DK, DV, normalize=False)
    b = b / np.sum(b * k * k, axis=-1, keepdims=True)  # sum_c b_c k_c^2 = 1 (b may leave [0,1])
    q = b * k
    o, _ = oracle.fwd(q, k, v, g, b, w, h0)
    assert relerr(o, w * v) < 1e-12


def test_erase_strength_two_is_a_householder_reflection():
    """The [0, 2] erase range (LIT-802 takeaway 5 / Table 5): with b = 2*1, a unit key, no
    decay and no write, the transition I - 2 k k^T is a reflection: it keeps the state's
    Frobenius norm, negates the state's component along k, and twice the same key restores
    the state exactly."""
    rng = np.random.default_rng(12)
    B, T, H, DK, DV = 1, 2, 1, 5, 3
    q, k, v, g, b, w, h0 = rand_inputs(rng, B, T, H, DK, DV)
    k[:, 1] = k[:, 0]
    b = np.full_like(b, 2.0)
    g = np.zeros_like(g)
    w = np.zeros_like(w)
    _, h1 = oracle.fwd(q[:, :1], k[:, :1], v[:, :1], g[:, :1], b[:, :1], w[:, :1], h0)
    _, h2 = oracle.fwd(q, k, v, g, b, w, h0)
    kk = k[0, 0, 0]
    assert abs(np.linalg.norm(h1) - np.linalg.norm(h0)) < 1e-13 * np.linalg.norm(h0)
    assert relerr(kk @ h1[0, 0], -(kk @ h0[0, 0])) < 1e-13
    assert relerr(h2, h0) < 1e-13


def test_b_zero_is_decayed_linear_attention():
    """b = 0 removes the erase: o_t = sum_{i<=t} [sum_c q_tc k_ic exp(G_tc - G_ic)] (w_i*v_i)
    + (q_t*exp(G_t))^T h0 with G the running sum of g; with g = 0 it is tril(Q K^T)(W*V) + Q h0."""
    rng = np.random.default_rng(5)
    B, T, H, DK, DV = 1, 33, 2, 6, 7
    q, k, v, g, b, w, h0 = rand_inputs(rng, B, T, H, DK, DV)
    b = np.zeros_like(b)
    o, _ = oracle.fwd(q, k, v, g, b, w, h0)
    for h in range(H):
        G = np.cumsum(g[0, :, h], axis=0)
        Q, K, X = q[0, :, h], k[0, :, h], w[0, :, h] * v[0, :, h]
        L = np.einsum("tc,ic,tic->ti", Q, K, np.exp(G[:, None, :] - G[None, :, :])) * np.tri(T)
        ref = L @ X + (Q * np.exp(G)) @ h0[0, h]
        assert relerr(o[0, :, h], ref) < 1e-12
    g0 = np.zeros_like(g)
    o0, _ = oracle.fwd(q, k, v, g0, b, w, h0)
    for h in range(H):
        Q, K, X = q[0, :, h], k[0, :, h], w[0, :, h] * v[0, :, h]
        ref = np.tril(Q @ K.T) @ X + Q @ h0[0, h]
        assert relerr(o0[0, :, h], ref) < 1e-13


def test_linearity_in_values_and_initial_state():
    rng = np.random.default_rng(6)
    B, T, H, DK, DV = 1, 20, 2, 5, 4
    q, k, v1, g, b, w, h01 = rand_inputs(rng, B, T, H, DK, DV)
    v2 = rng.standard_normal(v1.shape)
    h02 = rng.standard_normal(h01.shape)
    a1, a2 = 0.7, -1.3
    o1, s1 = oracle.fwd(q, k, v1, g, b, w, h01)
    o2, s2 = oracle.fwd(q, k, v2, g, b, w, h02)
    o3, s3 = oracle.fwd(q, k, a1 * v1 + a2 * v2, g, b, w, a1 * h01 + a2 * h02)
    assert relerr(o3, a1 * o1 + a2 * o2) < 1e-13
    assert relerr(s3, a1 * s1 + a2 * s2) < 1e-13
    # v and w enter only through their product
    o4, s4 = oracle.fwd(q, k, v1 * w, g, b, np.ones_like(w), h01)
    assert relerr(o4, o1) < 1e-14 and relerr(s4, s1) < 1e-14


def test_split_invariance():
    rng = np.random.default_rng(7)
    B, T, H, DK, DV = 2, 50, 2, 6, 6
    q, k, v, g, b, w, h0 = rand_inputs(rng, B, T, H, DK, DV)
    o, ht = oracle.fwd(q, k, v, g, b, w, h0)
    T1 = 19
    oa, sa = oracle.fwd(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], b[:, :T1], w[:, :T1], h0)
    ob, sb = oracle.fwd(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], b[:, T1:], w[:, T1:], sa)
    assert relerr(np.concatenate([oa, ob], 1), o) < 1e-13
    assert relerr(sb, ht) < 1e-13


def test_zero_token_padding_is_a_no_op():
    rng = np.random.default_rng(8)
    B, T, H, DK, DV = 1, 23, 2, 4, 5
    q, k, v, g, b, w, h0 = rand_inputs(rng, B, T, H, DK, DV)
    pad = lambda x: np.concatenate([x, np.zeros((B, 9) + x.shape[2:])], 1)
    o, ht = oracle.fwd(q, k, v, g, b, w, h0)
    op, hp = oracle.fwd(*(pad(x) for x in (q, k, v, g, b, w)), h0)
    assert np.array_equal(op[:, :T], o) and np.array_equal(hp, ht)
    assert np.all(op[:, T:] == 0)


# ----------------------------------------------------------------------------- backward pins

def loss(q, k, v, g, b, w, h0, do, dht):
    o, ht = oracle.fwd(q, k, v, g, b, w, h0)
    return np.sum(o * do) + np.sum(ht * dht)


def test_backward_matches_central_finite_differences():
    rng = np.random.default_rng(9)
    B, T, H, DK, DV = 1, 12, 1, 4, 3
    q, k, v, g, b, w, h0 = rand_inputs(rng, B, T, H, DK, DV, normalize=False)
    do = rng.standard_normal(v.shape)
    dht = rng.standard_normal(h0.shape)
    gr = oracle.bwd(q, k, v, g, b, w, h0, do, dht)
    args = dict(q=q, k=k, v=v, g=g, b=b, w=w, h0=h0)
    eps = 1e-6
    for name, key in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("b", "db"), ("w", "dw"),
                      ("h0", "dh0")]:
        x = args[name]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            xp = x.copy(); xp[ix] += eps
            xm = x.copy(); xm[ix] -= eps
            ap = dict(args, **{name: xp}); am = dict(args, **{name: xm})
            fd[ix] = (loss(**ap, do=do, dht=dht) - loss(**am, do=do, dht=dht)) / (2 * eps)
        err = np.max(np.abs(gr[key] - fd)) / np.max(np.abs(fd))
        assert err < 1e-7, (name, err)


def torch_token_loop(q, k, v, g, b, w, h0):
    """A separately written fp64 token loop, differentiated by torch autograd."""
    B, T, H, DK = q.shape
    outs, finals = [], []
    for bb in range(B):
        for h in range(H):
            S = h0[bb, h]
            ot = []
            for t in range(T):
                decayed = torch.exp(g[bb, t, h])[:, None] * S
                read = decayed.T @ (b[bb, t, h] * k[bb, t, h])
                S = decayed + torch.outer(k[bb, t, h], w[bb, t, h] * v[bb, t, h] - read)
                ot.append(S.T @ q[bb, t, h])
            outs.append(torch.stack(ot))
            finals.append(S)
    o = torch.stack(outs).reshape(B, H, T, -1).permute(0, 2, 1, 3)
    return o, torch.stack(finals).reshape(B, H, DK, -1)


def test_backward_matches_torch_autograd_loop():
    rng = np.random.default_rng(10)
    B, T, H, DK, DV = 1, 150, 2, 16, 12   # 150 > one 64-token checkpoint segment, ragged
    q, k, v, g, b, w, h0 = rand_inputs(rng, B, T, H, DK, DV)
    do = rng.standard_normal(v.shape)
    dht = rng.standard_normal(h0.shape)
    gr = oracle.bwd(q, k, v, g, b, w, h0, do, dht)
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, g, b, w, h0)]
    o, ht = torch_token_loop(*ts)
    (o * torch.tensor(do)).sum().add((ht * torch.tensor(dht)).sum()).backward()
    for t, key in zip(ts, ["dq", "dk", "dv", "dg", "db", "dw", "dh0"]):
        assert relerr(gr[key], t.grad.numpy()) < 1e-12, key


def test_kda_gradient_identity():
    """With tied gates, d beta of KDA equals sum_c db + sum_c dw; the other gradients agree."""
    rng = np.random.default_rng(11)
    B, T, H, DK, DV = 1, 40, 1, 6, 5
    q, k, v, g, _, _, h0 = rand_inputs(rng, B, T, H, DK, DV)
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    do = rng.standard_normal((B, T, H, DV))
    gr = oracle.bwd(q, k, v, g, np.repeat(beta[..., None], DK, -1), np.repeat(beta[..., None], DV, -1),
                    h0, do)
    tq, tk, tv, tg, tb, th = [torch.tensor(x, requires_grad=True) for x in (q, k, v, g, beta, h0)]
    S = th[0, 0]
    outs = []
    for t in range(T):  # KDA in its own form
        kt, bt = tk[0, t, 0], tb[0, t, 0]
        S = (torch.eye(DK, dtype=torch.float64) - bt * torch.outer(kt, kt)) @ (torch.exp(tg[0, t, 0])[:, None] * S) \
            + bt * torch.outer(kt, tv[0, t, 0])
        outs.append(S.T @ tq[0, t, 0])
    (torch.stack(outs) * torch.tensor(do[0, :, 0])).sum().backward()
    dbeta = gr["db"].sum(-1) + gr["dw"].sum(-1)
    assert relerr(dbeta, tb.grad.numpy()) < 1e-12
    for t, key in [(tq, "dq"), (tk, "dk"), (tv, "dv"), (tg, "dg"), (th, "dh0")]:
        assert relerr(gr[key], t.grad.numpy()) < 1e-12, key


def test_gradient_product_identity():
    """x = w*v, so dv*v = dw*w elementwise."""
    rng = np.random.default_rng(12)
    q, k, v, g, b, w, h0 = rand_inputs(rng, 1, 30, 2, 5, 4)
    gr = oracle.bwd(q, k, v, g, b, w, h0, rng.standard_normal(v.shape))
    assert relerr(gr["dv"] * v, gr["dw"] * w) < 1e-13


def test_gradient_split_invariance():
    """The first half's gradients, with dht taken from the second half's dh0, equal the full run's."""
    rng = np.random.default_rng(13)
    B, T, H, DK, DV = 1, 90, 2, 6, 5
    q, k, v, g, b, w, h0 = rand_inputs(rng, B, T, H, DK, DV)
    do = rng.standard_normal(v.shape)
    dht = rng.standard_normal(h0.shape)
    full = oracle.bwd(q, k, v, g, b, w, h0, do, dht)
    T1 = 41
    first = lambda x: x[:, :T1]
    second = lambda x: x[:, T1:]
    _, s1 = oracle.fwd(*(first(x) for x in (q, k, v, g, b, w)), h0)
    g2 = oracle.bwd(*(second(x) for x in (q, k, v, g, b, w)), s1, second(do), dht)
    g1 = oracle.bwd(*(first(x) for x in (q, k, v, g, b, w)), h0, first(do), g2["dh0"])
    for key in ["dq", "dk", "dv", "dg", "db", "dw"]:
        assert relerr(np.concatenate([g1[key], g2[key]], 1), full[key]) < 1e-12, key
    assert relerr(g1["dh0"], full["dh0"]) < 1e-12


def test_golden_regression_fixture():
    """Fixture written by tests/golden/make_golden.py, which calls only the oracle."""
    path = os.path.join(GOLDEN, "oracle_small.npz")
    d = np.load(path)
    o, ht = oracle.fwd(d["q"], d["k"], d["v"], d["g"], d["b"], d["w"], d["h0"])
    gr = oracle.bwd(d["q"], d["k"], d["v"], d["g"], d["b"], d["w"], d["h0"], d["do"], d["dht"])
    assert relerr(o, d["o"]) < 1e-14 and relerr(ht, d["ht"]) < 1e-14
    for key in ["dq", "dk", "dv", "dg", "db", "dw", "dh0"]:
        assert relerr(gr[key], d[key]) < 1e-14, key


# ----------------------------------------------------------------------------- gate logits

def test_gate_logit_activations():
    """sigmoid(0) = 1/2, softplus(0) = ln 2, and the activations' limits."""
    g, b, w = oracle.gates_from_logits(np.array([0.0, -40.0, 40.0]), np.array([0.0, -40.0, 40.0]),
                                       np.array([0.0, 3.0, -3.0]), 0.5, 2.0)
    assert np.allclose(g, [-0.5 * np.log(2.0), -0.5 * np.exp(-40.0), -20.0], rtol=1e-12, atol=0)
    assert np.allclose(b, [1.0, 2.0 * np.exp(-40.0), 2.0], rtol=1e-12, atol=0)
    assert np.allclose(w, [0.5, 1.0 / (1.0 + np.exp(-3.0)), 1.0 / (1.0 + np.exp(3.0))], rtol=1e-12, atol=0)


def test_backward_through_gate_logits_matches_finite_differences():
    rng = np.random.default_rng(21)
    B, T, H, DK, DV = 1, 9, 1, 3, 4
    q, k, v, _, _, _, h0 = rand_inputs(rng, B, T, H, DK, DV, normalize=False)
    zg, zb, zw = rng.standard_normal((B, T, H, DK)), rng.standard_normal((B, T, H, DK)), \
        rng.standard_normal((B, T, H, DV))
    do = rng.standard_normal(v.shape)
    dht = rng.standard_normal(h0.shape)
    s = 0.7
    gr = oracle.bwd_logits(q, k, v, zg, zb, zw, h0, do, dht, g_scale=s, b_scale=2.0)

    def lossz(zg, zb, zw):
        o, ht = oracle.fwd_logits(q, k, v, zg, zb, zw, h0, g_scale=s, b_scale=2.0)
        return float(np.sum(o * do) + np.sum(ht * dht))

    args = dict(zg=zg, zb=zb, zw=zw)
    eps = 1e-6
    for name, key in [("zg", "dg"), ("zb", "db"), ("zw", "dw")]:
        x = args[name]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            ix = it.multi_index
            xp = x.copy(); xp[ix] += eps
            xm = x.copy(); xm[ix] -= eps
            fd[ix] = (lossz(**dict(args, **{name: xp})) - lossz(**dict(args, **{name: xm}))) / (2 * eps)
        err = np.max(np.abs(gr[key] - fd)) / np.max(np.abs(fd))
        assert err < 1e-7, (name, err)

