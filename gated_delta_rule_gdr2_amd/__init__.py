"""MI355X-native Gated Delta Rule-2 operator: thin Python binding of libgdr2.

The operator ("Gated DeltaNet-2: Decoupling Erase and Write in Linear
Attention", anthology record LIT-802, takeaway 1; paper Sec. 3.1 Eqs. 8-10)

    S_t = (I - k_t (b_t * k_t)^T) diag(exp g_t) S_{t-1} + k_t (w_t * v_t)^T
    o_t = S_t^T q_t

runs entirely in the HIP kernels of ``libgdr2.so`` (built from ``csrc/`` by
``python -m gated_delta_rule_gdr2_amd.build``); see ``include/gdr2.h`` for the
C ABI. This module only marshals torch tensors (device memory and the current
HIP stream) into those calls. There is no fallback: if the library is missing
every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["gdr2_fwd", "gdr2_bwd", "gdr2_step", "gdr2_fwd_logits", "gdr2_bwd_logits", "gdr2_step_logits",
           "gdr2_fwd_seg", "gdr2_bwd_seg", "gdr2_fwd_noalloc", "gdr2_fwd_workspace_bytes",
           "gdr2_bwd_workspace_bytes", "gdr2_seg_workspace_bytes", "gdr2_strerror", "gdr2_version", "GDR2Function",
           "library_path", "load_library"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDR2_LIB names another build of the same library (e.g. one with host-side sanitizers)
_LIB_PATH = os.environ.get("GDR2_LIB") or os.path.join(_HERE, "libgdr2.so")
_lib = None

DTYPE_F32, DTYPE_BF16 = 0, 1
_DT = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}
EXPORTED = ["gdr2_fwd", "gdr2_bwd", "gdr2_step", "gdr2_fwd_logits", "gdr2_bwd_logits", "gdr2_step_logits",
            "gdr2_fwd_seg", "gdr2_bwd_seg", "gdr2_fwd_noalloc", "gdr2_fwd_workspace_bytes",
            "gdr2_bwd_workspace_bytes", "gdr2_seg_workspace_bytes", "gdr2_strerror", "gdr2_version"]
NOALLOC_SCRATCH_BYTES = 64 << 20  # GDR2_NOALLOC_SCRATCH_BYTES in include/gdr2.h


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libgdr2.so (raises RuntimeError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libgdr2.so not found at %s; build it with "
                           "`python -m gated_delta_rule_gdr2_amd.build`" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.gdr2_fwd_workspace_bytes.argtypes = [i] * 8
    lib.gdr2_fwd_workspace_bytes.restype = sz
    lib.gdr2_bwd_workspace_bytes.argtypes = [i] * 7
    lib.gdr2_bwd_workspace_bytes.restype = sz
    lib.gdr2_fwd.argtypes = [vp] * 9 + [i] * 8 + [vp, sz, vp, vp]
    lib.gdr2_fwd.restype = i
    lib.gdr2_bwd.argtypes = [vp] * 16 + [i] * 8 + [vp, sz, vp, vp]
    lib.gdr2_bwd.restype = i
    lib.gdr2_step.argtypes = [vp] * 8 + [i] * 6 + [vp]
    lib.gdr2_step.restype = i
    f = ctypes.c_float
    lib.gdr2_fwd_logits.argtypes = [vp] * 6 + [f, f] + [vp] * 3 + [i] * 8 + [vp, sz, vp, vp]
    lib.gdr2_fwd_logits.restype = i
    lib.gdr2_bwd_logits.argtypes = [vp] * 6 + [f, f] + [vp] * 10 + [i] * 8 + [vp, sz, vp, vp]
    lib.gdr2_bwd_logits.restype = i
    lib.gdr2_step_logits.argtypes = [vp] * 6 + [f, f] + [vp] * 2 + [i] * 6 + [vp]
    lib.gdr2_step_logits.restype = i
    lib.gdr2_seg_workspace_bytes.argtypes = [i] * 9
    lib.gdr2_seg_workspace_bytes.restype = sz
    lib.gdr2_fwd_seg.argtypes = [vp] * 9 + [i] * 9 + [vp, sz, vp, vp]
    lib.gdr2_fwd_seg.restype = i
    lib.gdr2_bwd_seg.argtypes = [vp] * 16 + [i] * 9 + [vp, sz, vp, vp]
    lib.gdr2_bwd_seg.restype = i
    lib.gdr2_fwd_noalloc.argtypes = [vp] * 9 + [i] * 7 + [vp]
    lib.gdr2_fwd_noalloc.restype = i
    lib.gdr2_strerror.argtypes = [i]
    lib.gdr2_strerror.restype = ctypes.c_char_p
    lib.gdr2_version.argtypes = []
    lib.gdr2_version.restype = i
    _lib = lib
    return lib


def gdr2_strerror(status: int) -> str:
    return load_library().gdr2_strerror(int(status)).decode()


def gdr2_version() -> int:
    return int(load_library().gdr2_version())


def gdr2_fwd_workspace_bytes(B, T, H, dk, dv, chunk=64, dtype=DTYPE_BF16, save_for_bwd=False) -> int:
    return int(load_library().gdr2_fwd_workspace_bytes(B, T, H, dk, dv, chunk, dtype, int(bool(save_for_bwd))))


def gdr2_bwd_workspace_bytes(B, T, H, dk, dv, chunk=64, dtype=DTYPE_BF16) -> int:
    return int(load_library().gdr2_bwd_workspace_bytes(B, T, H, dk, dv, chunk, dtype))


def gdr2_seg_workspace_bytes(B, T, H, dk, dv, chunk=64, segments=1, dtype=DTYPE_BF16, save_for_bwd=False) -> int:
    return int(load_library().gdr2_seg_workspace_bytes(B, T, H, dk, dv, chunk, segments, dtype,
                                                       int(bool(save_for_bwd))))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, dtype, shape):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must have dtype %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _raise(status, what):
    if status != 0:
        raise RuntimeError("%s failed: %s (status %d)" % (what, gdr2_strerror(status), status))


def _dims(q, v):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if q.dtype not in _DT:
        raise ValueError("unsupported dtype %s" % q.dtype)
    return B, T, H, dk, dv, _DT[q.dtype]


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _keep_for(stream, *tensors):
    """Tensors allocated here come from torch's current stream; when the kernels run on
    another stream, tell the caching allocator that this stream uses them too, so that their
    memory is not handed out again (after the caller, or this module, drops them) before the
    work enqueued on that stream has finished with it."""
    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def workspace(B, T, H, dk, dv, dtype, train, device="cuda", segments=None):
    """Allocate a workspace tensor (uint8) big enough for gdr2_fwd(save_for_bwd=train) / gdr2_bwd
    (segments=None), or for their _seg variants with that many segments."""
    dt = _DT[dtype] if isinstance(dtype, torch.dtype) else dtype
    if segments is None:
        n = gdr2_bwd_workspace_bytes(B, T, H, dk, dv, 64, dt) if train else \
            gdr2_fwd_workspace_bytes(B, T, H, dk, dv, 64, dt, False)
    else:
        n = gdr2_seg_workspace_bytes(B, T, H, dk, dv, 64, segments, dt, train)
    if n == 0 and B * T * H > 0:
        raise ValueError("unsupported shape/dtype for gdr2: B=%d T=%d H=%d dk=%d dv=%d" % (B, T, H, dk, dv))
    return torch.empty(n, dtype=torch.uint8, device=device)  # empty for a call without tokens


def gdr2_fwd(q, k, v, g, b, w, h0=None, *, chunk=64, save_for_bwd=False, ws=None, o=None,
             output_final_state=True, stream=None, stage_events=None):
    """Forward pass. q, k, g, b: [B,T,H,dk]; v, w: [B,T,H,dv] (bf16 or fp32, same dtype);
    h0: [B,H,dk,dv] fp32 or None. Returns (o, ht or None, ws). Pass ``ws`` back to
    gdr2_bwd(..., fwd_saved=True) when save_for_bwd is set. ``stage_events``: optional
    ctypes array of hipEvent_t handles recorded around the kernels (see include/gdr2.h)."""
    return _fwd(None, q, k, v, g, b, w, h0, chunk, save_for_bwd, ws, o, output_final_state, stream,
                stage_events)


def gdr2_fwd_seg(q, k, v, g, b, w, h0=None, *, segments, chunk=64, save_for_bwd=False, ws=None, o=None,
                 output_final_state=True, stream=None, stage_events=None):
    """gdr2_fwd with the state chains cut into ``segments`` pieces walked in parallel
    (chunk-parallel scan; see include/gdr2.h). The workspace must be sized for the same segments."""
    return _fwd(None, q, k, v, g, b, w, h0, chunk, save_for_bwd, ws, o, output_final_state, stream,
                stage_events, segments)


def gdr2_fwd_logits(q, k, v, zg, zb, zw, h0=None, *, g_scale=1.0, b_scale=1.0, chunk=64, save_for_bwd=False,
                    ws=None, o=None, output_final_state=True, stream=None, stage_events=None):
    """Forward pass with the gates given as logits, activated inside the kernels:
    g = -g_scale softplus(zg), b = b_scale sigmoid(zb), w = sigmoid(zw). Otherwise as gdr2_fwd."""
    return _fwd((g_scale, b_scale), q, k, v, zg, zb, zw, h0, chunk, save_for_bwd, ws, o, output_final_state,
                stream, stage_events)


def _fwd(scales, q, k, v, g, b, w, h0, chunk, save_for_bwd, ws, o, output_final_state, stream, stage_events,
         segments=None):
    lib = load_library()
    B, T, H, dk, dv, dt = _dims(q, v)
    for t, n, shp in ((q, "q", (B, T, H, dk)), (k, "k", (B, T, H, dk)), (g, "g", (B, T, H, dk)),
                      (b, "b", (B, T, H, dk)), (v, "v", (B, T, H, dv)), (w, "w", (B, T, H, dv))):
        _check(t, n, q.dtype, shp)
    _check(h0, "h0", torch.float32, (B, H, dk, dv))
    new = []
    if o is None:
        o = torch.empty(B, T, H, dv, dtype=q.dtype, device=q.device)
        new.append(o)
    _check(o, "o", q.dtype, (B, T, H, dv))
    ht = torch.empty(B, H, dk, dv, dtype=torch.float32, device=q.device) if output_final_state else None
    new.append(ht)
    if ws is None:
        ws = workspace(B, T, H, dk, dv, dt, save_for_bwd, q.device, segments)
        new.append(ws)
    _keep_for(stream, *new)
    tail = (_ptr(h0), _ptr(o), _ptr(ht), B, T, H, dk, dv, chunk, dt, int(bool(save_for_bwd)), _ptr(ws),
            ws.numel(), _stream(stream), stage_events)
    if segments is not None:
        st = lib.gdr2_fwd_seg(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), *tail[:9], segments,
                              *tail[9:])
        _raise(st, "gdr2_fwd_seg")
        return o, ht, ws
    if scales is None:
        st = lib.gdr2_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), *tail)
    else:
        st = lib.gdr2_fwd_logits(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), *scales, *tail)
    _raise(st, "gdr2_fwd" if scales is None else "gdr2_fwd_logits")
    return o, ht, ws


def gdr2_fwd_noalloc(q, k, v, g, b, w, h0=None, *, chunk=64, o=None, output_final_state=True, stream=None):
    """Inference forward whose workspace is the library's fixed device array (for callers that
    cannot allocate device memory; see include/gdr2.h). The C call allocates nothing; this
    wrapper allocates o and ht only when they are not passed. Calls that overlap on one GPU race
    on the shared array. Returns (o, ht or None)."""
    lib = load_library()
    B, T, H, dk, dv, dt = _dims(q, v)
    for t, n, shp in ((q, "q", (B, T, H, dk)), (k, "k", (B, T, H, dk)), (g, "g", (B, T, H, dk)),
                      (b, "b", (B, T, H, dk)), (v, "v", (B, T, H, dv)), (w, "w", (B, T, H, dv))):
        _check(t, n, q.dtype, shp)
    _check(h0, "h0", torch.float32, (B, H, dk, dv))
    new = []
    if o is None:
        o = torch.empty(B, T, H, dv, dtype=q.dtype, device=q.device)
        new.append(o)
    _check(o, "o", q.dtype, (B, T, H, dv))
    ht = torch.empty(B, H, dk, dv, dtype=torch.float32, device=q.device) if output_final_state else None
    new.append(ht)
    _keep_for(stream, *new)
    st = lib.gdr2_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), _ptr(h0), _ptr(o), _ptr(ht),
                              B, T, H, dk, dv, chunk, dt, _stream(stream))
    _raise(st, "gdr2_fwd_noalloc")
    return o, ht


def gdr2_step(q, k, v, g, b, w, state, *, o=None, stream=None):
    """Recurrent step (decoding): the T tokens of q, k, g, b [B,T,H,dk] and v, w [B,T,H,dv]
    one at a time from ``state`` ([B,H,dk,dv] fp32), which is updated in place. Returns o."""
    return _step(None, q, k, v, g, b, w, state, o, stream)


def gdr2_step_logits(q, k, v, zg, zb, zw, state, *, g_scale=1.0, b_scale=1.0, o=None, stream=None):
    """Recurrent step with the gates given as logits (activations as gdr2_fwd_logits)."""
    return _step((g_scale, b_scale), q, k, v, zg, zb, zw, state, o, stream)


def _step(scales, q, k, v, g, b, w, state, o, stream):
    lib = load_library()
    B, T, H, dk, dv, dt = _dims(q, v)
    for t, n, shp in ((q, "q", (B, T, H, dk)), (k, "k", (B, T, H, dk)), (g, "g", (B, T, H, dk)),
                      (b, "b", (B, T, H, dk)), (v, "v", (B, T, H, dv)), (w, "w", (B, T, H, dv))):
        _check(t, n, q.dtype, shp)
    if state is None:
        raise ValueError("state is required")
    _check(state, "state", torch.float32, (B, H, dk, dv))
    if o is None:
        o = torch.empty(B, T, H, dv, dtype=q.dtype, device=q.device)
        _keep_for(stream, o)
    _check(o, "o", q.dtype, (B, T, H, dv))
    tail = (_ptr(state), _ptr(o), B, T, H, dk, dv, dt, _stream(stream))
    if scales is None:
        st = lib.gdr2_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), *tail)
    else:
        st = lib.gdr2_step_logits(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), *scales, *tail)
    _raise(st, "gdr2_step" if scales is None else "gdr2_step_logits")
    return o


def gdr2_bwd(q, k, v, g, b, w, h0, dout, dht=None, *, chunk=64, ws=None, fwd_saved=False,
             need_dh0=True, grads=None, stream=None, stage_events=None):
    """Backward pass. Returns a dict with dq, dk, dv, dg, db, dw (input dtype) and dh0 (fp32 or None).
    With fwd_saved=True, ``ws`` must be the workspace of a gdr2_fwd(..., save_for_bwd=True) call on
    the same inputs."""
    return _bwd(None, q, k, v, g, b, w, h0, dout, dht, chunk, ws, fwd_saved, need_dh0, grads, stream,
                stage_events)


def gdr2_bwd_seg(q, k, v, g, b, w, h0, dout, dht=None, *, segments, chunk=64, ws=None, fwd_saved=False,
                 need_dh0=True, grads=None, stream=None, stage_events=None):
    """gdr2_bwd with the reverse state chains cut into ``segments`` pieces (chunk-parallel scan).
    With fwd_saved=True, ``ws`` must come from gdr2_fwd_seg(save_for_bwd=True) with the same segments."""
    return _bwd(None, q, k, v, g, b, w, h0, dout, dht, chunk, ws, fwd_saved, need_dh0, grads, stream,
                stage_events, segments)


def gdr2_bwd_logits(q, k, v, zg, zb, zw, h0, dout, dht=None, *, g_scale=1.0, b_scale=1.0, chunk=64, ws=None,
                    fwd_saved=False, need_dh0=True, grads=None, stream=None, stage_events=None):
    """Backward with the gates given as logits: dg, db, dw of the returned dict are the gradients
    with respect to zg, zb, zw. With fwd_saved=True, ``ws`` must come from gdr2_fwd_logits on the
    same inputs and scales."""
    return _bwd((g_scale, b_scale), q, k, v, zg, zb, zw, h0, dout, dht, chunk, ws, fwd_saved, need_dh0, grads,
                stream, stage_events)


def _bwd(scales, q, k, v, g, b, w, h0, dout, dht, chunk, ws, fwd_saved, need_dh0, grads, stream, stage_events,
         segments=None):
    lib = load_library()
    B, T, H, dk, dv, dt = _dims(q, v)
    for t, n, shp in ((q, "q", (B, T, H, dk)), (k, "k", (B, T, H, dk)), (g, "g", (B, T, H, dk)),
                      (b, "b", (B, T, H, dk)), (v, "v", (B, T, H, dv)), (w, "w", (B, T, H, dv)),
                      (dout, "dout", (B, T, H, dv))):
        _check(t, n, q.dtype, shp)
    _check(h0, "h0", torch.float32, (B, H, dk, dv))
    _check(dht, "dht", torch.float32, (B, H, dk, dv))
    new = []
    if grads is None:
        grads = {n: torch.empty_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("db", b),
                                                     ("dw", w))}
        new += list(grads.values())
    grads["dh0"] = torch.empty(B, H, dk, dv, dtype=torch.float32, device=q.device) if need_dh0 else None
    new.append(grads["dh0"])
    if ws is None:
        if fwd_saved:
            raise ValueError("fwd_saved=True needs the forward's workspace")
        ws = workspace(B, T, H, dk, dv, dt, True, q.device, segments)
        new.append(ws)  # dropped on return: its memory must outlive the kernels on `stream`
    _keep_for(stream, *new)
    tail = (_ptr(h0), _ptr(dout), _ptr(dht), _ptr(grads["dq"]), _ptr(grads["dk"]), _ptr(grads["dv"]),
            _ptr(grads["dg"]), _ptr(grads["db"]), _ptr(grads["dw"]), _ptr(grads["dh0"]), B, T, H, dk, dv, chunk,
            dt, int(bool(fwd_saved)), _ptr(ws), ws.numel(), _stream(stream), stage_events)
    if segments is not None:
        st = lib.gdr2_bwd_seg(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), *tail[:16], segments,
                              *tail[16:])
        _raise(st, "gdr2_bwd_seg")
        return grads
    if scales is None:
        st = lib.gdr2_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), *tail)
    else:
        st = lib.gdr2_bwd_logits(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(b), _ptr(w), *scales, *tail)
    _raise(st, "gdr2_bwd" if scales is None else "gdr2_bwd_logits")
    return grads


class GDR2Function(torch.autograd.Function):
    """Autograd wrapper: forward saves the per-chunk states in the workspace, backward reuses them."""

    @staticmethod
    def forward(ctx, q, k, v, g, b, w, h0=None):
        o, ht, ws = gdr2_fwd(q, k, v, g, b, w, h0, save_for_bwd=True)
        ctx.save_for_backward(q, k, v, g, b, w, h0, ws)
        ctx.has_h0 = h0 is not None
        return o, ht

    @staticmethod
    def backward(ctx, do, dht):
        q, k, v, g, b, w, h0, ws = ctx.saved_tensors
        gr = gdr2_bwd(q, k, v, g, b, w, h0, do.contiguous(),
                      None if dht is None else dht.contiguous(), ws=ws, fwd_saved=True,
                      need_dh0=ctx.has_h0)
        return gr["dq"], gr["dk"], gr["dv"], gr["dg"], gr["db"], gr["dw"], gr["dh0"]
