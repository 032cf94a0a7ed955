"""The chunkwise equations the kernels implement equal the token-wise oracle to
machine precision in fp64 (the property the pages report for the chunk form:
anthology record LIT-802, takeaway 2, App. D.6)."""
import numpy as np
import pytest

import oracle
from chunk_mirror import chunk_bwd, chunk_fwd


def rel(x, r):
    return np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-300)


def inputs(seed, T, DK, DV, gscale=0.1, h0=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, DK)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, DK)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, DV))
    g = -np.logaddexp(0, rng.standard_normal((T, DK))) * gscale
    b = 1 / (1 + np.exp(-rng.standard_normal((T, DK))))
    w = 1 / (1 + np.exp(-rng.standard_normal((T, DV))))
    h = rng.standard_normal((DK, DV)) * 0.1 if h0 else None
    do = rng.standard_normal((T, DV))
    dht = rng.standard_normal((DK, DV))
    return q, k, v, g, b, w, h, do, dht


def as4(x):
    return x[None, :, None, :]


@pytest.mark.parametrize("C", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("T,gscale", [(64, 0.1), (150, 0.5), (200, 2.0)])
def test_chunk_forward_equals_oracle(C, T, gscale):
    q, k, v, g, b, w, h0, _, _ = inputs(T + C, T, 16, 12, gscale)
    o, S = chunk_fwd(q, k, v, g, b, w, h0, C)
    oo, So = oracle.fwd(as4(q), as4(k), as4(v), as4(g), as4(b), as4(w), h0[None, None])
    assert rel(o, oo[0, :, 0]) < 1e-12 and rel(S, So[0, 0]) < 1e-12


@pytest.mark.parametrize("C", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("T,gscale", [(64, 0.1), (150, 0.5)])
def test_chunk_backward_equals_oracle(C, T, gscale):
    q, k, v, g, b, w, h0, do, dht = inputs(7 * T + C, T, 16, 12, gscale)
    gr = chunk_bwd(q, k, v, g, b, w, h0, do, dht, C)
    go = oracle.bwd(as4(q), as4(k), as4(v), as4(g), as4(b), as4(w), h0[None, None], as4(do), dht[None, None])
    for key in ["dq", "dk", "dv", "dg", "db", "dw"]:
        assert rel(gr[key], go[key][0, :, 0]) < 1e-12, key
    assert rel(gr["dh0"], go["dh0"][0, 0]) < 1e-12
