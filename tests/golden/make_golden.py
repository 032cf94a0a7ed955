"""Writes tests/golden/oracle_small.npz: a small fp64 case and the oracle's outputs.

Calls only the oracle package. The fixture guards the oracle against silent
drift; the oracle itself is pinned by the other tests in test_oracle_pins.py.
Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def main():
    rng = np.random.default_rng(2024)
    B, T, H, DK, DV = 1, 70, 2, 8, 6
    q = rng.standard_normal((B, T, H, DK)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, T, H, DK)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, DV))
    g = -np.logaddexp(0, rng.standard_normal((B, T, H, DK))) * 0.2
    b = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, DK))))
    w = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, DV))))
    h0 = rng.standard_normal((B, H, DK, DV)) * 0.1
    do = rng.standard_normal((B, T, H, DV))
    dht = rng.standard_normal((B, H, DK, DV))
    o, ht = oracle.fwd(q, k, v, g, b, w, h0)
    gr = oracle.bwd(q, k, v, g, b, w, h0, do, dht)
    np.savez(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.npz"),
             q=q, k=k, v=v, g=g, b=b, w=w, h0=h0, do=do, dht=dht, o=o, ht=ht, **gr)


if __name__ == "__main__":
    main()
