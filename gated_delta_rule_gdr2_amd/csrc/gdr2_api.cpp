// C ABI of libgdr2: argument validation (host only, before any HIP call),
// workspace sizing and kernel dispatch. See include/gdr2.h for the contract.
#include "../../include/gdr2.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdr2_kernels.hpp"

namespace {

bool supported(int dk, int dv, int chunk, int dtype) {
    if (chunk != 64) return false;
    if (dtype == GDR2_DTYPE_BF16) return (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
    if (dtype == GDR2_DTYPE_F32) return dk == 64 && dv == 64;
    return false;
}

int esize(int dtype) { return dtype == GDR2_DTYPE_BF16 ? 2 : 4; }

bool aligned(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(int B, int T, int H, int dk, int dv, int chunk, int dtype) {
    if (B < 0 || T < 0 || H < 0) return GDR2_ERR_SHAPE;
    if (!supported(dk, dv, chunk, dtype)) return GDR2_ERR_UNSUPPORTED;
    // element counts must fit comfortably in 64-bit offsets and the grid in 32 bits
    const long long NT = (T + 63) / 64;
    const long long nc = (long long)B * H * NT;
    if (nc > 0x7fffffffLL || (long long)B * T * H > (1LL << 40)) return GDR2_ERR_SHAPE;
    return GDR2_OK;
}

// No tokens (B, T or H zero): the token tensors are empty and their pointers may be null;
// the calls only pass the state through (see pass_state).
bool no_tokens(int B, int T, int H) { return (long long)B * T * H == 0; }

// The result of a call without tokens: the end state of a recurrence over no tokens is its
// start state (h_T = h0, and zero without h0), and so is the gradient that reaches the start
// (dh0 = dht, and zero without dht). dst (B * H * dk * dv floats) may be null: nothing to do.
int pass_state(float* dst, const float* src, int B, int H, int dk, int dv, void* stream) {
    const long long n = (long long)B * H * dk * dv;
    if (!dst || n == 0) return GDR2_OK;
    return gdr2::launch_state_pass(dst, src, n, (hipStream_t)stream) == hipSuccess ? GDR2_OK : GDR2_ERR_HIP;
}

// Segments of the state chains: `segments` requested (>= 1) -> chunks per segment and
// the number of (non-empty) segments actually used.
void seg_plan(int T, int segments, int& nseg, int& seg_len) {
    const int NT = (T + 63) / 64;
    const int req = segments < NT ? segments : NT;
    seg_len = (NT + req - 1) / req;
    nseg = (NT + seg_len - 1) / seg_len;
}

// The segment count gdr2_fwd / gdr2_bwd use. The chains run one workgroup per (sequence,
// 16 value columns) and a step's cost is set by the operands each walk moves through its
// compute unit, which the scan roughly triples (summaries, transitions, the second walk),
// so it pays only when the walks are too few to fill the 256 compute units: up to 128
// chain walks, 512 / (walks) segments (the main walks then use 32-column slices), at most
// 8, each of at least 16 chunks (shorter segments spend more on the summaries than they
// save). Measured at d = 128: T = 16384 fwd+bwd, 16 heads best with 4 segments (1.12 ms
// against 1.22 with one), 4 heads with 4-8 (0.46-0.47 against 0.73), one head with 8
// (0.30 against 0.63); the forward alone at 16 heads, T = 2048, is faster with 2 segments
// of 16 chunks than with 4 of 8 (0.080 against 0.100 ms).
int auto_segments(int B, int T, int H, int dv) {
    const long long wgs = (long long)B * H * (dv / 16);
    const int NT = (T + 63) / 64;
    if (wgs < 1 || wgs > 128) return 1;
    int n = (int)(512 / wgs);
    if (n > 8) n = 8;
    if (n > NT / 16) n = NT / 16;
    return n < 1 ? 1 : n;
}

gdr2::Layout layout_for(int B, int T, int H, int dk, int dv, int dtype, int segments, bool train) {
    const long long NT = (T + 63) / 64;
    int nseg, seg_len;
    seg_plan(T, segments, nseg, seg_len);
    return gdr2::make_layout((long long)B * H * NT, dk, dv, esize(dtype), (long long)B * H, nseg, train);
}

// gate scales of the logit entry points: finite, g_scale > 0, 0 < b_scale <= 2
bool scales_ok(float g_scale, float b_scale) {
    return g_scale > 0.f && g_scale <= 3.0e38f && b_scale > 0.f && b_scale <= 2.f;
}

// Results that a later kernel reads go out with non-temporal stores once the data they
// belong to passes half the 256 MB Infinity Cache (the workspace of the chunked path, the
// state of the decode step); below that, plain stores leave them cached for the reader.
// Measured: 176 MB and more of workspace -- faster with the hint; 37 MB -- faster without.
constexpr size_t NT_OUT_MIN_BYTES = size_t(128) << 20;

void fill_common(gdr2::Args& a, int B, int T, int H, int dk, int dv, int dtype, void* ws, int segments = 1,
                 bool train = true) {
    a.B = B;
    a.T = T;
    a.H = H;
    a.NT = (T + 63) / 64;
    a.NC = (long long)B * H * a.NT;
    seg_plan(T, segments, a.nseg, a.seg_len);
    a.L = layout_for(B, T, H, dk, dv, dtype, segments, train);
    a.ws = (char*)ws;
    a.nt_out = (train ? a.L.train_bytes : a.L.fwd_infer_bytes) >= NT_OUT_MIN_BYTES;
}

}  // namespace

extern "C" {

size_t gdr2_seg_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int segments, int dtype,
                                int save_for_bwd) {
    if (check_shape(B, T, H, dk, dv, chunk, dtype) != GDR2_OK || segments < 1 || no_tokens(B, T, H)) return 0;
    gdr2::Layout L = layout_for(B, T, H, dk, dv, dtype, segments, save_for_bwd != 0);
    return save_for_bwd ? L.train_bytes : L.fwd_infer_bytes;
}

size_t gdr2_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype, int save_for_bwd) {
    if (check_shape(B, T, H, dk, dv, chunk, dtype) != GDR2_OK) return 0;
    return gdr2_seg_workspace_bytes(B, T, H, dk, dv, chunk, auto_segments(B, T, H, dv), dtype, save_for_bwd);
}

size_t gdr2_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype) {
    if (check_shape(B, T, H, dk, dv, chunk, dtype) != GDR2_OK) return 0;
    return gdr2_seg_workspace_bytes(B, T, H, dk, dv, chunk, auto_segments(B, T, H, dv), dtype, 1);
}

}  // extern "C"

namespace {

// Host validation of a forward call (everything but the workspace) and the workspace
// bytes it needs; no HIP call.
int fwd_check(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
              const float* h0, void* o, float* ht, int B, int T, int H, int dk, int dv, int chunk, int dtype,
              int save_for_bwd, int act, float g_scale, float b_scale, int& segments, size_t& need) {
    int st = check_shape(B, T, H, dk, dv, chunk, dtype);
    if (st != GDR2_OK) return st;
    if (!no_tokens(B, T, H) && (!q || !k || !v || !g || !b || !w || !o)) return GDR2_ERR_NULL;
    if (act && !scales_ok(g_scale, b_scale)) return GDR2_ERR_VALUE;
    if (segments < 0) return GDR2_ERR_VALUE;  // 0: the automatic count
    if (segments == 0) segments = auto_segments(B, T, H, dv);
    const void* ptrs[] = {q, k, v, g, b, w, h0, o, ht};
    for (const void* p : ptrs)
        if (p && !aligned(p)) return GDR2_ERR_ALIGN;
    need = gdr2_seg_workspace_bytes(B, T, H, dk, dv, chunk, segments, dtype, save_for_bwd);
    return GDR2_OK;
}

int fwd_impl(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
             const float* h0, void* o, float* ht, int B, int T, int H, int dk, int dv, int chunk, int dtype,
             int save_for_bwd, void* workspace, size_t workspace_bytes, void* stream,
             void* const* stage_events, int act, float g_scale, float b_scale, int segments) {
    size_t need = 0;
    int st = fwd_check(q, k, v, g, b, w, h0, o, ht, B, T, H, dk, dv, chunk, dtype, save_for_bwd, act, g_scale,
                       b_scale, segments, need);
    if (st != GDR2_OK) return st;
    if (workspace && !aligned(workspace)) return GDR2_ERR_ALIGN;
    if (no_tokens(B, T, H)) return pass_state(ht, h0, B, H, dk, dv, stream);
    if (!workspace || workspace_bytes < need) return GDR2_ERR_WORKSPACE;

    gdr2::Args a = {};
    a.q = q; a.k = k; a.v = v; a.g = g; a.b = b; a.w = w;
    a.h0 = h0; a.o = o; a.ht = ht;
    a.act = act; a.g_scale = g_scale; a.b_scale = b_scale;
    fill_common(a, B, T, H, dk, dv, dtype, workspace, segments, save_for_bwd != 0);
    a.events = (hipEvent_t const*)stage_events;
    hipError_t e = gdr2::launch_fwd(a, dtype == GDR2_DTYPE_BF16, save_for_bwd != 0, (hipStream_t)stream);
    return e == hipSuccess ? GDR2_OK : GDR2_ERR_HIP;
}

int bwd_impl(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
             const float* h0, const void* dout, const float* dht, void* dq, void* dk_, void* dv_, void* dg,
             void* db, void* dw, float* dh0, int B, int T, int H, int dk, int dv, int chunk, int dtype,
             int fwd_saved, void* workspace, size_t workspace_bytes, void* stream,
             void* const* stage_events, int act, float g_scale, float b_scale, int segments) {
    int st = check_shape(B, T, H, dk, dv, chunk, dtype);
    if (st != GDR2_OK) return st;
    if (!no_tokens(B, T, H) &&
        (!q || !k || !v || !g || !b || !w || !dout || !dq || !dk_ || !dv_ || !dg || !db || !dw))
        return GDR2_ERR_NULL;
    if (act && !scales_ok(g_scale, b_scale)) return GDR2_ERR_VALUE;
    if (segments < 0) return GDR2_ERR_VALUE;  // 0: the automatic count
    if (segments == 0) segments = auto_segments(B, T, H, dv);
    const void* ptrs[] = {q, k, v, g, b, w, h0, dout, dht, dq, dk_, dv_, dg, db, dw, dh0, workspace};
    for (const void* p : ptrs)
        if (p && !aligned(p)) return GDR2_ERR_ALIGN;
    if (no_tokens(B, T, H)) return pass_state(dh0, dht, B, H, dk, dv, stream);
    const size_t need = gdr2_seg_workspace_bytes(B, T, H, dk, dv, chunk, segments, dtype, 1);
    if (!workspace || workspace_bytes < need) return GDR2_ERR_WORKSPACE;

    gdr2::Args a = {};
    a.q = q; a.k = k; a.v = v; a.g = g; a.b = b; a.w = w;
    a.h0 = h0; a.dout = dout; a.dht = dht;
    a.dq = dq; a.dk = dk_; a.dv = dv_; a.dg = dg; a.db = db; a.dw = dw; a.dh0 = dh0;
    a.o = nullptr; a.ht = nullptr;
    a.act = act; a.g_scale = g_scale; a.b_scale = b_scale;
    fill_common(a, B, T, H, dk, dv, dtype, workspace, segments);
    const bool bf = dtype == GDR2_DTYPE_BF16;
    hipError_t e = hipSuccess;
    a.events = (hipEvent_t const*)stage_events;
    if (!fwd_saved) {
        e = gdr2::launch_fwd(a, bf, true, (hipStream_t)stream);
        if (a.events) {  // the backward stages follow the two forward ones, whose end is their start
            a.events += 2;
            a.events_continue = 1;
        }
    }
    if (e == hipSuccess) e = gdr2::launch_bwd(a, bf, (hipStream_t)stream);
    return e == hipSuccess ? GDR2_OK : GDR2_ERR_HIP;
}

int step_impl(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
              float* state, void* o, int B, int T, int H, int dk, int dv, int dtype, void* stream, int act,
              float g_scale, float b_scale) {
    int st = check_shape(B, T, H, dk, dv, 64, dtype);
    if (st != GDR2_OK) return st;
    const bool none = no_tokens(B, T, H);
    if (!none && (!q || !k || !v || !g || !b || !w || !o)) return GDR2_ERR_NULL;
    if ((long long)B * H > 0 && !state) return GDR2_ERR_NULL;  // the state is not a token tensor
    if (act && !scales_ok(g_scale, b_scale)) return GDR2_ERR_VALUE;
    const void* ptrs[] = {q, k, v, g, b, w, state, o};
    for (const void* p : ptrs)
        if (p && !aligned(p)) return GDR2_ERR_ALIGN;
    if (none) return GDR2_OK;  // no tokens: the state stays as it is
    gdr2::Args a = {};
    a.q = q; a.k = k; a.v = v; a.g = g; a.b = b; a.w = w;
    a.o = o; a.state = state;
    a.act = act; a.g_scale = g_scale; a.b_scale = b_scale;
    fill_common(a, B, T, H, dk, dv, dtype, nullptr);
    a.nt_out = (size_t)B * H * dk * dv * sizeof(float) >= NT_OUT_MIN_BYTES;
    hipError_t e = gdr2::launch_step(a, dtype == GDR2_DTYPE_BF16, (hipStream_t)stream);
    return e == hipSuccess ? GDR2_OK : GDR2_ERR_HIP;
}

}  // namespace

namespace gdr2 {

int fwd_validate(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
                 const float* h0, void* o, float* ht, int B, int T, int H, int dk, int dv, int chunk, int dtype,
                 size_t* need) {
    int segments = 0;
    size_t n = 0;
    const int st = fwd_check(q, k, v, g, b, w, h0, o, ht, B, T, H, dk, dv, chunk, dtype, 0, 0, 1.f, 1.f, segments, n);
    *need = n;
    return st;
}

int fwd_with_workspace(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
                       const float* h0, void* o, float* ht, int B, int T, int H, int dk, int dv, int chunk,
                       int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    return fwd_impl(q, k, v, g, b, w, h0, o, ht, B, T, H, dk, dv, chunk, dtype, 0, workspace, workspace_bytes,
                    stream, nullptr, 0, 1.f, 1.f, 0);
}

}  // namespace gdr2

extern "C" {

int gdr2_fwd(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
             const float* h0, void* o, float* ht, int B, int T, int H, int dk, int dv, int chunk, int dtype,
             int save_for_bwd, void* workspace, size_t workspace_bytes, void* stream,
             void* const* stage_events) {
    return fwd_impl(q, k, v, g, b, w, h0, o, ht, B, T, H, dk, dv, chunk, dtype, save_for_bwd, workspace,
                    workspace_bytes, stream, stage_events, 0, 1.f, 1.f, 0);
}

int gdr2_fwd_seg(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
                 const float* h0, void* o, float* ht, int B, int T, int H, int dk, int dv, int chunk, int segments,
                 int dtype, int save_for_bwd, void* workspace, size_t workspace_bytes, void* stream,
                 void* const* stage_events) {
    return fwd_impl(q, k, v, g, b, w, h0, o, ht, B, T, H, dk, dv, chunk, dtype, save_for_bwd, workspace,
                    workspace_bytes, stream, stage_events, 0, 1.f, 1.f, segments < 1 ? -1 : segments);
}

int gdr2_fwd_logits(const void* q, const void* k, const void* v, const void* zg, const void* zb, const void* zw,
                    float g_scale, float b_scale, const float* h0, void* o, float* ht, int B, int T, int H,
                    int dk, int dv, int chunk, int dtype, int save_for_bwd, void* workspace,
                    size_t workspace_bytes, void* stream, void* const* stage_events) {
    return fwd_impl(q, k, v, zg, zb, zw, h0, o, ht, B, T, H, dk, dv, chunk, dtype, save_for_bwd, workspace,
                    workspace_bytes, stream, stage_events, 1, g_scale, b_scale, 0);
}

int gdr2_bwd(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
             const float* h0, const void* dout, const float* dht, void* dq, void* dk_, void* dv_, void* dg,
             void* db, void* dw, float* dh0, int B, int T, int H, int dk, int dv, int chunk, int dtype,
             int fwd_saved, void* workspace, size_t workspace_bytes, void* stream,
             void* const* stage_events) {
    return bwd_impl(q, k, v, g, b, w, h0, dout, dht, dq, dk_, dv_, dg, db, dw, dh0, B, T, H, dk, dv, chunk,
                    dtype, fwd_saved, workspace, workspace_bytes, stream, stage_events, 0, 1.f, 1.f, 0);
}

int gdr2_bwd_seg(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
                 const float* h0, const void* dout, const float* dht, void* dq, void* dk_, void* dv_, void* dg,
                 void* db, void* dw, float* dh0, int B, int T, int H, int dk, int dv, int chunk, int segments,
                 int dtype, int fwd_saved, void* workspace, size_t workspace_bytes, void* stream,
                 void* const* stage_events) {
    return bwd_impl(q, k, v, g, b, w, h0, dout, dht, dq, dk_, dv_, dg, db, dw, dh0, B, T, H, dk, dv, chunk,
                    dtype, fwd_saved, workspace, workspace_bytes, stream, stage_events, 0, 1.f, 1.f,
                    segments < 1 ? -1 : segments);
}

int gdr2_bwd_logits(const void* q, const void* k, const void* v, const void* zg, const void* zb,
                    const void* zw, float g_scale, float b_scale, const float* h0, const void* dout,
                    const float* dht, void* dq, void* dk_, void* dv_, void* dzg, void* dzb, void* dzw,
                    float* dh0, int B, int T, int H, int dk, int dv, int chunk, int dtype, int fwd_saved,
                    void* workspace, size_t workspace_bytes, void* stream, void* const* stage_events) {
    return bwd_impl(q, k, v, zg, zb, zw, h0, dout, dht, dq, dk_, dv_, dzg, dzb, dzw, dh0, B, T, H, dk, dv,
                    chunk, dtype, fwd_saved, workspace, workspace_bytes, stream, stage_events, 1, g_scale,
                    b_scale, 0);
}

int gdr2_step(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
              float* state, void* o, int B, int T, int H, int dk, int dv, int dtype, void* stream) {
    return step_impl(q, k, v, g, b, w, state, o, B, T, H, dk, dv, dtype, stream, 0, 1.f, 1.f);
}

int gdr2_step_logits(const void* q, const void* k, const void* v, const void* zg, const void* zb,
                     const void* zw, float g_scale, float b_scale, float* state, void* o, int B, int T,
                     int H, int dk, int dv, int dtype, void* stream) {
    return step_impl(q, k, v, zg, zb, zw, state, o, B, T, H, dk, dv, dtype, stream, 1, g_scale, b_scale);
}

const char* gdr2_strerror(int status) {
    switch (status) {
        case GDR2_OK: return "ok";
        case GDR2_ERR_NULL: return "a required pointer is NULL";
        case GDR2_ERR_SHAPE: return "invalid shape (B, T and H must be >= 0; sizes must fit)";
        case GDR2_ERR_UNSUPPORTED: return "unsupported dk/dv/chunk/dtype combination";
        case GDR2_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case GDR2_ERR_WORKSPACE: return "workspace is NULL or too small";
        case GDR2_ERR_HIP: return "HIP launch failed";
        case GDR2_ERR_VALUE:
            return "a scalar argument is out of range (g_scale > 0 finite, 0 < b_scale <= 2, segments >= 1)";
        case GDR2_ERR_SCRATCH:
            return "the call needs more workspace than the library's fixed device array "
                   "(GDR2_NOALLOC_SCRATCH_BYTES) holds";
        default: return "unknown status";
    }
}

int gdr2_version(void) { return 100; }

}  // extern "C"
