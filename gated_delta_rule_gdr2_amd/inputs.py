"""Seeded synthetic inputs for the Gated Delta Rule-2 operator.

This module holds the workload definitions and the random-input recipe only;
it contains none of the operator's arithmetic. Both the HIP path (benchmark,
GPU tests) and the fp64 oracle (tests) take their inputs from here.

The five workloads mirror the shapes the Gated DeltaNet-2 pages train and
measure on: 4K training length (anthology record LIT-802, takeaway 3), and
the 2K x 8 and 16K x 1 points of the throughput figure (takeaway 6, Fig. 2),
with H = 16 heads of d_k = d_v = 128, which gives the 262,144-float state per
layer stated in takeaway 3. No dataset is involved: every tensor is drawn
from a seeded numpy PCG64 generator in float64, in the fixed order
q, k, v, g, b, w, h0, do, then rounded once to the working dtype (bf16 with
round-to-nearest-even, or fp32). The oracle consumes exactly the rounded
values, upcast to fp64.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    DK: int
    DV: int
    dtype: str            # "f32" or "bf16"
    backward: bool        # fwd only, or fwd+bwd
    seed: int
    g_scale: float = 0.1  # g = -softplus(N(0,1)) * g_scale per key channel
    b_mu: float = 0.0     # b = b_scale * sigmoid(N(b_mu, 1)) per channel
    b_scale: float = 1.0  # 2.0: the [0, 2] erase range (negative eigenvalues of the transition)
    w_mu: float = 0.0     # w = sigmoid(N(w_mu, 1)) per channel
    h0_std: float = 0.0   # h0 ~ N(0, h0_std) in fp32 (0 -> no initial state)
    tied: bool = False    # b = w = beta * 1, beta = sigmoid(N(0,1)) per token
    chunk: int = 64
    extra: dict = field(default_factory=dict)

    @property
    def tokens(self) -> int:
        return self.B * self.T


WORKLOADS = {
    # small fp32 forward case the oracle finishes instantly
    "fwd_f32_b1h2t256d64": Workload("fwd_f32_b1h2t256d64", 1, 2, 256, 64, 64, "f32", False, seed=1),
    # bf16 forward with a random fp32 initial state
    "fwd_bf16_b1h16t2048d128_h0": Workload("fwd_bf16_b1h16t2048d128_h0", 1, 16, 2048, 128, 128, "bf16",
                                           False, seed=2, h0_std=0.02),
    # training shape: the headline throughput workload
    "fwdbwd_bf16_b2h16t4096d128": Workload("fwdbwd_bf16_b2h16t4096d128", 2, 16, 4096, 128, 128, "bf16",
                                           True, seed=3),
    # the same shape with tied gates b = w = beta (the KDA special case)
    "fwdbwd_bf16_b2h16t4096d128_tied": Workload("fwdbwd_bf16_b2h16t4096d128_tied", 2, 16, 4096, 128, 128,
                                                "bf16", True, seed=31, tied=True),
    # batch-heavy, faster forgetting
    "fwdbwd_bf16_b8h16t2048d128_g05": Workload("fwdbwd_bf16_b8h16t2048d128_g05", 8, 16, 2048, 128, 128,
                                               "bf16", True, seed=4, g_scale=0.5),
    # long sequence, initial state, skewed gates
    "fwdbwd_bf16_b1h16t16384d128_h0": Workload("fwdbwd_bf16_b1h16t16384d128_h0", 1, 16, 16384, 128, 128,
                                               "bf16", True, seed=5, b_mu=1.0, w_mu=-1.0, h0_std=0.02),
}

HEADLINE = "fwdbwd_bf16_b2h16t4096d128"


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


def make_inputs(wl: Workload, device="cpu", gates="act", **overrides) -> dict:
    """Draw the workload's tensors. Returns torch tensors on ``device``:
    q, k, g, b [B,T,H,DK]; v, w [B,T,H,DV] in the working dtype; h0 [B,H,DK,DV]
    fp32 or None; do [B,T,H,DV] in the working dtype (None for fwd-only).
    gates="logits": instead of g, b, w the dict holds the normal draws they are made
    from, zg, zb, zw (zb and zw with their means b_mu, w_mu added), for the entry
    points that take the gates as logits with scales g_scale, b_scale."""
    if overrides:
        wl = replace(wl, **overrides)
    if gates not in ("act", "logits") or (gates == "logits" and wl.tied):
        raise ValueError("gates must be 'act' or 'logits' (logits: untied gates only)")
    rng = np.random.default_rng(wl.seed)
    B, T, H, DK, DV = wl.B, wl.T, wl.H, wl.DK, wl.DV
    q = rng.standard_normal((B, T, H, DK))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, T, H, DK))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, DV))
    zg = rng.standard_normal((B, T, H, DK))
    g = -_softplus(zg) * wl.g_scale
    if wl.tied:
        beta = _sigmoid(rng.standard_normal((B, T, H, 1)))
        b = np.broadcast_to(beta, (B, T, H, DK)).copy()
        w = np.broadcast_to(beta, (B, T, H, DV)).copy()
    else:
        zb = rng.standard_normal((B, T, H, DK)) + wl.b_mu
        b = wl.b_scale * _sigmoid(zb)
        zw = rng.standard_normal((B, T, H, DV)) + wl.w_mu
        w = _sigmoid(zw)
    h0 = rng.standard_normal((B, H, DK, DV)) * wl.h0_std if wl.h0_std > 0 else None
    do = rng.standard_normal((B, T, H, DV)) if wl.backward else None

    dt = torch_dtype(wl.dtype)

    def cast(x, dtype=dt):
        if x is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).to(device)

    if gates == "logits":
        return dict(q=cast(q), k=cast(k), v=cast(v), zg=cast(zg), zb=cast(zb), zw=cast(zw),
                    h0=cast(h0, torch.float32), do=cast(do))
    return dict(q=cast(q), k=cast(k), v=cast(v), g=cast(g), b=cast(b), w=cast(w),
                h0=cast(h0, torch.float32), do=cast(do))


def small(name="tiny", B=1, H=2, T=100, DK=64, DV=64, dtype="bf16", backward=True, seed=7, **kw) -> Workload:
    """A small workload for parity tests (several chunks and a ragged tail by default)."""
    return Workload(name, B, H, T, DK, DV, dtype, backward, seed, **kw)
