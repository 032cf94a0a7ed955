"""Shared helpers of the GPU parity tests: error measures, sequence sampling and the
per-chunk bound for sampled full-size workloads (no arithmetic of the method)."""
import numpy as np

TOL = {"f32": ("inf", 1e-5), "bf16": ("fro", 2e-2)}


def rel_err(x, r, kind):
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if kind == "inf":
        return np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-30)
    return np.linalg.norm(x - r) / max(np.linalg.norm(r), 1e-30)


def assert_chunks_close(name, x, r, dtype, T, C=64):
    """x, r: one sequence's token tensor (T rows); the tolerance on every C-token chunk, so
    that an error confined to a few chunks cannot hide under the whole-tensor norm."""
    kind, tol = TOL[dtype]
    x = np.asarray(x, dtype=np.float64).reshape(T, -1)
    r = np.asarray(r, dtype=np.float64).reshape(T, -1)
    worst, at = 0.0, -1
    for c0 in range(0, T, C):
        e = rel_err(x[c0:c0 + C], r[c0:c0 + C], kind)
        if e > worst:
            worst, at = e, c0 // C
    print("%-12s worst chunk %d err %.3e (tol %.0e)" % (name, at, worst, tol), flush=True)
    assert worst <= tol, (name, at, worst)


def sample_sequences(wl, n=4, seed_offset=100):
    """(batch, head) pairs of a workload: the first, the last, and n - 2 more at random."""
    rng = np.random.default_rng(wl.seed + seed_offset)
    seqs = {(0, 0), (wl.B - 1, wl.H - 1)}
    while len(seqs) < min(n, wl.B * wl.H):
        seqs.add((int(rng.integers(wl.B)), int(rng.integers(wl.H))))
    return sorted(seqs)
