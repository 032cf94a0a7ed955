"""fp64 CPU oracle for the Gated Delta Rule-2 operator -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The HIP library never uses it, and the
two share no code.

The arithmetic lives in ``gdr2_oracle.c`` (plain C, fp64, OpenMP over the B*H
sequences); this module only compiles it with gcc and marshals numpy arrays.
What it computes is the token-by-token recurrence of "Gated DeltaNet-2:
Decoupling Erase and Write in Linear Attention" (anthology record LIT-802,
"Key takeaways", first bullet; paper Sec. 3.1 Eqs. 8-10):

    S_t = (I - k_t (b_t * k_t)^T) diag(exp g_t) S_{t-1} + k_t (w_t * v_t)^T
    o_t = S_t^T q_t          (readout after the update; a reading, see C file)

and the hand-derived back-propagation through that loop.

Parity status: every function here is pinned by tests in
``tests/test_oracle_pins.py`` (reductions to KDA / Gated DeltaNet / DeltaNet
stated on the pages, closed forms, invariants, brute force, finite
differences; for the gate-logit functions, finite differences with respect to
the logits and the activation values themselves).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr2_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle into ``oracle/liboracle.so`` with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
               "-shared", "-std=c11", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("GDR2_ORACLE_LIB")  # another build of the same source (sanitizer runs)
        if not path:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            path = _LIB
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.gdr2_oracle_fwd.argtypes = [i, i, i, i, i] + [dp] * 9
        lib.gdr2_oracle_fwd.restype = None
        lib.gdr2_oracle_bwd.argtypes = [i, i, i, i, i] + [dp] * 16
        lib.gdr2_oracle_bwd.restype = None
        lib.gdr2_oracle_num_threads.argtypes = []
        lib.gdr2_oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def num_threads() -> int:
    return int(_load().gdr2_oracle_num_threads())


def fwd(q, k, v, g, b, w, h0=None):
    """Forward recurrence in fp64.

    q, k, g, b: [B, T, H, DK]; v, w: [B, T, H, DV]; h0: [B, H, DK, DV] or None.
    Returns (o [B, T, H, DV], ht [B, H, DK, DV]).
    """
    q, k, v, g, b, w, h0 = (_f64(x) for x in (q, k, v, g, b, w, h0))
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    o = np.zeros((B, T, H, DV))
    ht = np.zeros((B, H, DK, DV))
    _load().gdr2_oracle_fwd(B, T, H, DK, DV, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w),
                            _ptr(h0), _ptr(o), _ptr(ht))
    return o, ht


def bwd(q, k, v, g, b, w, h0, do, dht=None):
    """Backward pass in fp64 (back-propagation through the token loop).

    Returns dict with dq, dk, dv, dg, db, dw (input shapes) and dh0 [B, H, DK, DV].
    """
    q, k, v, g, b, w, h0, do, dht = (_f64(x) for x in (q, k, v, g, b, w, h0, do, dht))
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    out = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("db", b), ("dw", w))}
    out["dh0"] = np.zeros((B, H, DK, DV))
    _load().gdr2_oracle_bwd(B, T, H, DK, DV, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w),
                            _ptr(h0), _ptr(do), _ptr(dht), _ptr(out["dq"]), _ptr(out["dk"]),
                            _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["db"]), _ptr(out["dw"]),
                            _ptr(out["dh0"]))
    return out


# ----------------------------------------------------------------------------- gate logits
# The gates as the pages define them: the erase gate b and the write gate w are each a
# sigmoid of their own projection (Gated DeltaNet-2 record LIT-802, "Key takeaways", first
# bullet); the widened erase range [0, 2] of its Table 5 ablation is b = 2 sigmoid(z_b),
# taken here as b = b_scale * sigmoid(z_b). The pages do not fix how the log-decay is
# parametrised; the reading used here is g = -g_scale * softplus(z_g), g_scale > 0, so
# that alpha = exp g lies in (0, 1). numpy, fp64.

def _sigmoid(z):
    e = np.exp(-np.abs(z))                       # never overflows; exact in both tails
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gates_from_logits(zg, zb, zw, g_scale=1.0, b_scale=1.0):
    """(g, b, w) = (-g_scale softplus(zg), b_scale sigmoid(zb), sigmoid(zw))."""
    zg, zb, zw = (_f64(x) for x in (zg, zb, zw))
    return -g_scale * np.logaddexp(0.0, zg), b_scale * _sigmoid(zb), _sigmoid(zw)


def fwd_logits(q, k, v, zg, zb, zw, h0=None, g_scale=1.0, b_scale=1.0):
    """Forward recurrence with the gates given as logits (see gates_from_logits)."""
    g, b, w = gates_from_logits(zg, zb, zw, g_scale, b_scale)
    return fwd(q, k, v, g, b, w, h0)


def bwd_logits(q, k, v, zg, zb, zw, h0, do, dht=None, g_scale=1.0, b_scale=1.0):
    """Backward with the gates given as logits: the dict holds dL/dzg, dL/dzb, dL/dzw under
    the keys dg, db, dw, the other gradients as bwd(). Chain rule through the activations:
    d sigmoid/dz = sigmoid (1 - sigmoid), d softplus/dz = sigmoid."""
    g, b, w = gates_from_logits(zg, zb, zw, g_scale, b_scale)
    gr = bwd(q, k, v, g, b, w, h0, do, dht)
    sb = _sigmoid(_f64(zb))
    gr["dg"] = gr["dg"] * (-g_scale * _sigmoid(_f64(zg)))
    gr["db"] = gr["db"] * (b_scale * sb * (1.0 - sb))
    gr["dw"] = gr["dw"] * (w * (1.0 - w))
    return gr
