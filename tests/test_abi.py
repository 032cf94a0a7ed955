"""Host-only checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/gdr2.h declares, sizes workspaces, and rejects bad
arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_gdr2_amd as g2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr2.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUP, ERR_ALIGN, ERR_WS, ERR_HIP, ERR_VALUE, ERR_SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(g2.library_path()):
        from gated_delta_rule_gdr2_amd import build
        build.build()
    return g2.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr2_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_exported_api():
    assert declared_functions() == sorted(g2.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    # the dynamic symbol table holds them as plain C names
    out = os.popen("nm -D --defined-only %s" % g2.library_path()).read()
    for name in declared_functions():
        assert re.search(r"\bT %s$" % name, out, flags=re.M), name


def test_version_and_strerror(lib):
    assert g2.gdr2_version() >= 100
    for st in (OK, ERR_NULL, ERR_SHAPE, ERR_UNSUP, ERR_ALIGN, ERR_WS, ERR_HIP, ERR_VALUE, ERR_SCRATCH):
        assert g2.gdr2_strerror(st) and g2.gdr2_strerror(st) != "unknown status"
    assert g2.gdr2_strerror(-99) == "unknown status"


def test_workspace_sizes(lib):
    BF = g2.DTYPE_BF16
    a = g2.gdr2_fwd_workspace_bytes(2, 4096, 16, 128, 128, 64, BF, False)
    b = g2.gdr2_fwd_workspace_bytes(2, 4096, 16, 128, 128, 64, BF, True)
    c = g2.gdr2_bwd_workspace_bytes(2, 4096, 16, 128, 128, 64, BF)
    assert 0 < a < b == c
    # tail chunk rounds up
    assert g2.gdr2_fwd_workspace_bytes(1, 65, 1, 64, 64, 64, BF, False) == \
        g2.gdr2_fwd_workspace_bytes(1, 128, 1, 64, 64, 64, BF, False)
    # unsupported -> 0
    assert g2.gdr2_fwd_workspace_bytes(1, 64, 1, 96, 64, 64, BF, False) == 0
    assert g2.gdr2_fwd_workspace_bytes(1, 64, 1, 64, 64, 32, BF, False) == 0
    assert g2.gdr2_fwd_workspace_bytes(1, 64, 1, 128, 128, 64, g2.DTYPE_F32, False) == 0
    assert g2.gdr2_fwd_workspace_bytes(-1, 64, 1, 64, 64, 64, BF, False) == 0
    # no tokens -> no workspace
    assert g2.gdr2_fwd_workspace_bytes(0, 64, 1, 64, 64, 64, BF, False) == 0
    assert g2.gdr2_fwd_workspace_bytes(1, 0, 1, 64, 64, 64, BF, True) == 0
    assert g2.gdr2_bwd_workspace_bytes(1, 64, 0, 64, 64, 64, BF) == 0
    assert g2.gdr2_seg_workspace_bytes(1, 0, 1, 64, 64, 64, 2, BF, 1) == 0


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def fwd(lib, ptrs=None, B=1, T=64, H=1, dk=64, dv=64, chunk=64, dtype=g2.DTYPE_BF16, save=0,
        ws=FAKE, ws_bytes=1 << 40):
    p = [FAKE] * 9 if ptrs is None else ptrs
    return lib.gdr2_fwd(*[ctypes.c_void_p(x) for x in p], B, T, H, dk, dv, chunk, dtype, save,
                        ctypes.c_void_p(ws), ws_bytes, None, None)


def bwd(lib, ptrs=None, B=1, T=64, H=1, dk=64, dv=64, chunk=64, dtype=g2.DTYPE_BF16, saved=1,
        ws=FAKE, ws_bytes=1 << 40):
    p = [FAKE] * 16 if ptrs is None else ptrs
    return lib.gdr2_bwd(*[ctypes.c_void_p(x) for x in p], B, T, H, dk, dv, chunk, dtype, saved,
                        ctypes.c_void_p(ws), ws_bytes, None, None)


@pytest.mark.parametrize("idx", range(8))
def test_fwd_rejects_null_required_pointers(lib, idx):
    # q k v g b w h0 o ht: h0 (6) and ht (8) are optional
    required = [0, 1, 2, 3, 4, 5, 7]
    if idx >= len(required):
        return
    p = [FAKE] * 9
    p[required[idx]] = 0
    assert fwd(lib, p) == ERR_NULL


def test_bwd_rejects_null_required_pointers(lib):
    # q k v g b w h0 dout dht dq dk dv dg db dw dh0: h0 (6), dht (8), dh0 (15) optional
    for i in [0, 1, 2, 3, 4, 5, 7, 9, 10, 11, 12, 13, 14]:
        p = [FAKE] * 16
        p[i] = 0
        assert bwd(lib, p) == ERR_NULL, i


def test_shape_and_support_errors(lib):
    assert fwd(lib, B=-1) == ERR_SHAPE
    assert fwd(lib, T=-1) == ERR_SHAPE
    assert bwd(lib, T=-64) == ERR_SHAPE
    assert fwd(lib, H=-1) == ERR_SHAPE
    assert fwd(lib, dk=96) == ERR_UNSUP
    assert fwd(lib, dv=32) == ERR_UNSUP
    assert fwd(lib, chunk=32) == ERR_UNSUP
    assert fwd(lib, dtype=7) == ERR_UNSUP
    assert fwd(lib, dk=128, dv=128, dtype=g2.DTYPE_F32) == ERR_UNSUP
    assert bwd(lib, dk=48) == ERR_UNSUP


def test_calls_without_tokens(lib):
    """B, T or H zero: the token tensors are empty (NULL pointers allowed) and no workspace is
    needed. With no state to pass through (ht / dh0 NULL, or B * H = 0) the calls succeed
    without any HIP call, so they run here; state pass-through is a GPU test."""
    none6 = [0] * 6
    assert fwd(lib, none6 + [0, 0, 0], T=0, ws=0, ws_bytes=0) == OK
    assert fwd(lib, none6 + [FAKE, 0, 0], T=0, ws=0, ws_bytes=0, save=1) == OK
    assert fwd(lib, none6 + [FAKE, 0, FAKE], B=0, ws=0, ws_bytes=0) == OK  # B * H = 0: no state
    assert fwd(lib, none6 + [FAKE, 0, FAKE], H=0, ws=0, ws_bytes=0) == OK
    assert bwd(lib, [0] * 16, T=0, ws=0, ws_bytes=0) == OK
    assert bwd(lib, [0] * 15 + [FAKE], B=0, ws=0, ws_bytes=0, saved=0) == OK
    assert step(lib, [0] * 6 + [FAKE, 0], T=0) == OK
    assert step(lib, [0] * 8, T=0) == ERR_NULL  # the state is required whenever B * H > 0
    assert step(lib, [0] * 8, B=0) == OK
    # the other checks still apply
    assert fwd(lib, none6 + [0, 0, 0], T=0, dk=96) == ERR_UNSUP
    assert fwd(lib, none6 + [FAKE + 4, 0, 0], T=0) == ERR_ALIGN
    assert bwd(lib, [0] * 16, T=0, dtype=g2.DTYPE_F32, dk=128, dv=128) == ERR_UNSUP
    assert fwd_logits(lib, none6 + [0, 0, 0], gs=-1.0, T=0) == ERR_VALUE


def test_alignment_errors(lib):
    for i in range(9):
        p = [FAKE] * 9
        p[i] = FAKE + 2
        assert fwd(lib, p) == ERR_ALIGN, i
    assert fwd(lib, ws=FAKE + 8) == ERR_ALIGN
    p = [FAKE] * 16
    p[15] = FAKE + 4
    assert bwd(lib, p) == ERR_ALIGN


def test_workspace_errors(lib):
    need = g2.gdr2_fwd_workspace_bytes(1, 64, 1, 64, 64, 64, g2.DTYPE_BF16, False)
    assert fwd(lib, ws_bytes=need - 1) == ERR_WS
    assert fwd(lib, ws=0) == ERR_WS
    need_t = g2.gdr2_fwd_workspace_bytes(1, 64, 1, 64, 64, 64, g2.DTYPE_BF16, True)
    assert fwd(lib, save=1, ws_bytes=need_t - 1) == ERR_WS
    assert bwd(lib, ws_bytes=g2.gdr2_bwd_workspace_bytes(1, 64, 1, 64, 64, 64, g2.DTYPE_BF16) - 1) == ERR_WS


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(g2, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(g2, "_lib", None)
    with pytest.raises(RuntimeError, match="not found"):
        g2.load_library()


def step(lib, ptrs=None, B=1, T=1, H=1, dk=64, dv=64, dtype=g2.DTYPE_BF16):
    p = [FAKE] * 8 if ptrs is None else ptrs
    return lib.gdr2_step(*[ctypes.c_void_p(x) for x in p], B, T, H, dk, dv, dtype, None)


def test_step_rejects_bad_arguments(lib):
    # q k v g b w state o: all required
    for i in range(8):
        p = [FAKE] * 8
        p[i] = 0
        assert step(lib, p) == ERR_NULL, i
        p[i] = FAKE + 4
        assert step(lib, p) == ERR_ALIGN, i
    assert step(lib, B=-1) == ERR_SHAPE
    assert step(lib, T=-1) == ERR_SHAPE
    assert step(lib, dk=96) == ERR_UNSUP
    assert step(lib, dk=128, dv=128, dtype=g2.DTYPE_F32) == ERR_UNSUP


# ----------------------------------------------------------------------------- gate-logit entry points

def fwd_logits(lib, ptrs=None, gs=1.0, bs=1.0, B=1, T=64, H=1, dk=64, dv=64, ws=FAKE, ws_bytes=1 << 40):
    p = [FAKE] * 9 if ptrs is None else ptrs
    v = [ctypes.c_void_p(x) for x in p]
    return lib.gdr2_fwd_logits(*v[:6], gs, bs, *v[6:], B, T, H, dk, dv, 64, g2.DTYPE_BF16, 1,
                               ctypes.c_void_p(ws), ws_bytes, None, None)


def bwd_logits(lib, ptrs=None, gs=1.0, bs=1.0, B=1, T=64, H=1, dk=64, dv=64, ws=FAKE, ws_bytes=1 << 40):
    p = [FAKE] * 16 if ptrs is None else ptrs
    v = [ctypes.c_void_p(x) for x in p]
    return lib.gdr2_bwd_logits(*v[:6], gs, bs, *v[6:], B, T, H, dk, dv, 64, g2.DTYPE_BF16, 1,
                               ctypes.c_void_p(ws), ws_bytes, None, None)


def step_logits(lib, ptrs=None, gs=1.0, bs=1.0, B=1, T=1, H=1, dk=64, dv=64):
    p = [FAKE] * 8 if ptrs is None else ptrs
    v = [ctypes.c_void_p(x) for x in p]
    return lib.gdr2_step_logits(*v[:6], gs, bs, *v[6:], B, T, H, dk, dv, g2.DTYPE_BF16, None)


@pytest.mark.parametrize("gs,bs", [(0.0, 1.0), (-1.0, 1.0), (float("nan"), 1.0), (float("inf"), 1.0),
                                   (1.0, 0.0), (1.0, 2.5), (1.0, float("nan")), (1.0, -1.0)])
def test_logit_entry_points_reject_bad_scales(lib, gs, bs):
    assert fwd_logits(lib, gs=gs, bs=bs) == ERR_VALUE
    assert bwd_logits(lib, gs=gs, bs=bs) == ERR_VALUE
    assert step_logits(lib, gs=gs, bs=bs) == ERR_VALUE


def test_logit_entry_points_validate_like_the_plain_ones(lib):
    p = [FAKE] * 9
    p[3] = 0  # zg
    assert fwd_logits(lib, p) == ERR_NULL
    p[3] = FAKE + 2
    assert fwd_logits(lib, p) == ERR_ALIGN
    assert fwd_logits(lib, dk=96) == ERR_UNSUP
    assert fwd_logits(lib, ws_bytes=1) == ERR_WS
    p = [FAKE] * 16
    p[14] = 0  # dzw
    assert bwd_logits(lib, p) == ERR_NULL
    assert bwd_logits(lib, B=-1) == ERR_SHAPE
    p = [FAKE] * 8
    p[6] = 0  # state
    assert step_logits(lib, p) == ERR_NULL
    assert step_logits(lib, dv=32) == ERR_UNSUP


# ----------------------------------------------------------------------------- segmented chains

def test_segment_workspace_sizes(lib):
    BF = g2.DTYPE_BF16
    # one segment: the plain sizes
    assert g2.gdr2_seg_workspace_bytes(2, 4096, 16, 128, 128, 64, 1, BF, False) == \
        g2.gdr2_fwd_workspace_bytes(2, 4096, 16, 128, 128, 64, BF, False)
    assert g2.gdr2_seg_workspace_bytes(2, 4096, 16, 128, 128, 64, 1, BF, True) == \
        g2.gdr2_bwd_workspace_bytes(2, 4096, 16, 128, 128, 64, BF)
    # four segments add three fp32 matrices per (sequence, segment)
    extra = g2.gdr2_seg_workspace_bytes(2, 4096, 16, 128, 128, 64, 4, BF, True) - \
        g2.gdr2_seg_workspace_bytes(2, 4096, 16, 128, 128, 64, 1, BF, True)
    assert extra == 32 * 4 * 3 * 128 * 128 * 4
    # more segments than chunks: one per chunk
    assert g2.gdr2_seg_workspace_bytes(1, 200, 1, 64, 64, 64, 9, BF, True) == \
        g2.gdr2_seg_workspace_bytes(1, 200, 1, 64, 64, 64, 4, BF, True)
    assert g2.gdr2_seg_workspace_bytes(1, 200, 1, 64, 64, 64, 0, BF, True) == 0


def test_segment_entry_points_validate(lib):
    v = [ctypes.c_void_p(FAKE)] * 9
    for seg in (0, -3):
        assert lib.gdr2_fwd_seg(*v, 1, 64, 1, 64, 64, 64, seg, g2.DTYPE_BF16, 0, ctypes.c_void_p(FAKE), 1 << 40,
                                None, None) == ERR_VALUE
        assert lib.gdr2_bwd_seg(*([ctypes.c_void_p(FAKE)] * 16), 1, 64, 1, 64, 64, 64, seg, g2.DTYPE_BF16, 1,
                                ctypes.c_void_p(FAKE), 1 << 40, None, None) == ERR_VALUE
    # the workspace check uses the segmented size
    need = g2.gdr2_seg_workspace_bytes(1, 640, 1, 64, 64, 64, 4, g2.DTYPE_BF16, False)
    assert lib.gdr2_fwd_seg(*v, 1, 640, 1, 64, 64, 64, 4, g2.DTYPE_BF16, 0, ctypes.c_void_p(FAKE), need - 1,
                            None, None) == ERR_WS
    v2 = list(v)
    v2[0] = ctypes.c_void_p(0)
    assert lib.gdr2_fwd_seg(*v2, 1, 640, 1, 64, 64, 64, 4, g2.DTYPE_BF16, 0, ctypes.c_void_p(FAKE), 1 << 40,
                            None, None) == ERR_NULL


def test_automatic_segments(lib):
    """The plain entry points size (and run) the chunk-parallel scan by themselves only
    when the chain walks (B * H * dv / 16) are at most 128: 512 / walks segments, at
    most 8, of at least 16 chunks each."""
    BF = g2.DTYPE_BF16

    def auto(B, T, H, dv):
        n = g2.gdr2_bwd_workspace_bytes(B, T, H, 128, dv, 64, BF)
        hits = [s for s in range(1, 17) if g2.gdr2_seg_workspace_bytes(B, T, H, 128, dv, 64, s, BF, True) == n]
        return hits[0]

    assert auto(2, 4096, 16, 128) == 1       # 256 workgroups
    assert auto(1, 16384, 16, 128) == 4      # 128
    assert auto(1, 2048, 16, 128) == 2       # 128, 32 chunks: segments of 16
    assert auto(8, 2048, 16, 128) == 1       # 1024
    assert auto(1, 16384, 4, 128) == 8       # 32
    assert auto(1, 16384, 2, 64) == 8        # 8
    assert auto(1, 4096, 1, 128) == 4        # 64 chunks: segments of 16
    assert auto(1, 2048, 1, 128) == 2        # 32 chunks
    assert auto(1, 1024, 1, 128) == 1        # 16 chunks
    assert auto(1, 500, 1, 128) == 1         # 8 chunks


def test_sizes_that_overflow_are_rejected(lib):
    # more than 2^31 - 1 chunks, or more than 2^40 token rows: invalid shape, nothing enqueued
    assert fwd(lib, B=1 << 16, T=1 << 20, H=1 << 10) == ERR_SHAPE
    assert fwd(lib, B=1 << 20, T=1 << 20, H=1) == ERR_SHAPE
    assert g2.gdr2_fwd_workspace_bytes(1 << 16, 1 << 20, 1 << 10, 64, 64, 64, g2.DTYPE_BF16, False) == 0


def noalloc(lib, ptrs=None, B=1, T=64, H=1, dk=64, dv=64, chunk=64, dtype=g2.DTYPE_BF16):
    p = [FAKE] * 9 if ptrs is None else ptrs
    return lib.gdr2_fwd_noalloc(*[ctypes.c_void_p(x) for x in p], B, T, H, dk, dv, chunk, dtype, None)


def test_noalloc_scratch_size_matches_the_header():
    m = re.search(r"#define GDR2_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == g2.NOALLOC_SCRATCH_BYTES


def test_noalloc_validates_like_the_forward_and_rejects_oversized_calls(lib):
    """Every check happens on the host before any HIP call (so no GPU is needed here): the
    forward's own errors, and GDR2_ERR_SCRATCH for a call whose workspace exceeds the fixed
    array -- the largest that fits and the smallest that does not, from the size query."""
    for idx in range(7):  # q, k, v, g, b, w and o (index 7 of the pointer list) are required
        p = [FAKE] * 9
        p[idx if idx < 6 else 7] = 0
        assert noalloc(lib, p) == ERR_NULL
    assert noalloc(lib, B=-1) == ERR_SHAPE
    # no tokens (B * H = 0, so no state either): nothing to do, no scratch looked up
    assert noalloc(lib, [0] * 9, B=0) == OK
    assert noalloc(lib, dk=96) == ERR_UNSUP
    assert noalloc(lib, dtype=g2.DTYPE_F32, dk=128, dv=128) == ERR_UNSUP
    p = [FAKE] * 9
    p[2] = FAKE + 8
    assert noalloc(lib, p) == ERR_ALIGN
    BF = g2.DTYPE_BF16
    cap = g2.NOALLOC_SCRATCH_BYTES
    # grow T until the inference workspace no longer fits
    T = 64
    while g2.gdr2_fwd_workspace_bytes(1, T + 64, 16, 128, 128, 64, BF, False) <= cap:
        T += 64
    assert g2.gdr2_fwd_workspace_bytes(1, T, 16, 128, 128, 64, BF, False) <= cap
    assert noalloc(lib, B=1, T=T + 64, H=16, dk=128, dv=128) == ERR_SCRATCH
    assert noalloc(lib, B=64, T=65536, H=16, dk=128, dv=128) == ERR_SCRATCH
    # the B=1, H=16, T=2048, d=128 bf16 forward workload fits
    assert g2.gdr2_fwd_workspace_bytes(1, 2048, 16, 128, 128, 64, BF, False) <= cap
