// Kernel arguments and launcher declarations (internal to libgdr2).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "gdr2_layout.hpp"

namespace gdr2 {

struct Args {
    // inputs, [B, T, H, D] row-major in the operand type
    const void *q, *k, *v, *g, *b, *w;
    const float* h0;    // [B, H, DK, DV] or null
    const void* dout;   // [B, T, H, DV]
    const float* dht;   // [B, H, DK, DV] or null
    // outputs
    void* o;            // [B, T, H, DV] or null (forward recompute inside the backward)
    float* ht;          // [B, H, DK, DV] or null
    void *dq, *dk, *dv, *dg, *db, *dw;
    float* dh0;         // [B, H, DK, DV] or null
    float* state;       // recurrent step: [B, H, DK, DV], read and overwritten
    // gates: act = 0 -> g, b, w are the gates themselves; act = 1 -> they are logits,
    // g = -g_scale softplus(g), b = b_scale sigmoid(b), w = sigmoid(w), and the backward
    // writes the gradients with respect to the logits into dg, db, dw
    int act;
    float g_scale, b_scale;
    // 1: results that a later kernel reads (the chains' per-chunk operands, the backward
    // chain's outputs, the gradients, the decode state) go out with non-temporal stores; the
    // library sets it for problems whose data is large next to the 256 MB Infinity Cache, and
    // the launchers pick the kernel instantiation that matches
    int nt_out;
    char* ws;           // workspace base
    Layout L;
    int B, T, H, NT;
    int nseg, seg_len;  // state chains: segments per sequence and chunks per segment (nseg = 1: one walk)
    long long NC;       // B * H * NT chunks
    // k_bwd_intra: the workgroups of one round are one per compute unit, so the chunk that
    // runs next on this workgroup's XCD (workgroups go to the XCDs round-robin) is
    // blockIdx + l2_ahead with l2_ahead = the compute unit count; its staged input rows are
    // pulled into L2 during this chunk's work (0: no warm-up)
    long long l2_ahead;
    hipEvent_t const* events;  // optional: per-stage timing events (see stage_event)
    int events_continue;       // 1: events[0] was recorded by the stages before (backward after a recompute)
};

// events[i] when per-stage timing was requested, else null. The launches attach them to
// their kernels (hipExtLaunchKernelGGL start / stop events), so timing adds no packets to
// the stream between the kernels.
inline hipEvent_t stage_event(const Args& a, int i) {
    return a.events && !(i == 0 && a.events_continue) ? a.events[i] : nullptr;
}

// Launchers: enqueue on `stream`, return hipSuccess or the launch error.
// The chain launchers take the events for the start of their first kernel and the end of
// their last (either may be null).
template <class OT, int DK, int DV>
hipError_t launch_fwd_chain_t(const Args& a, bool train, hipStream_t stream, hipEvent_t start, hipEvent_t stop);
template <class OT, int DK, int DV>
hipError_t launch_bwd_chain_t(const Args& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop);
hipError_t launch_fwd(const Args& a, bool bf16, bool train, hipStream_t stream);
hipError_t launch_bwd(const Args& a, bool bf16, hipStream_t stream);
hipError_t launch_step(const Args& a, bool bf16, hipStream_t stream);
// dst[0 .. n) = src[0 .. n), or zeros when src is null (n a multiple of 4, both 16-byte
// aligned): the state a call without tokens passes through.
hipError_t launch_state_pass(float* dst, const float* src, long long n, hipStream_t stream);
size_t fwd_intra_lds_bytes(int DK, int DV, int esz);

// The forward entry point's host validation (all but the workspace; *need = the workspace
// bytes of an inference forward) and the forward on a given workspace (gdr2_api.cpp).
int fwd_validate(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
                 const float* h0, void* o, float* ht, int B, int T, int H, int dk, int dv, int chunk, int dtype,
                 size_t* need);
int fwd_with_workspace(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
                       const float* h0, void* o, float* ht, int B, int T, int H, int dk, int dv, int chunk,
                       int dtype, void* workspace, size_t workspace_bytes, void* stream);
size_t bwd_intra_lds_bytes(int DK, int DV, int esz);

}  // namespace gdr2
