/*
 * gdr2.h -- C ABI of libgdr2, the MI355X (gfx950) implementation of the
 * Gated Delta Rule-2 sequence-mixing operator.
 *
 * Operator ("Gated DeltaNet-2: Decoupling Erase and Write in Linear
 * Attention", anthology record LIT-802, "Key takeaways", first bullet; paper
 * Sec. 3.1, Eqs. 8-10), for every batch row b and head h independently:
 *
 *     S_t = (I - k_t (b_t * k_t)^T) diag(exp g_t) S_{t-1} + k_t (w_t * v_t)^T
 *     o_t = S_t^T q_t                        (readout after the update)
 *
 * b_t is the channel-wise erase gate on the key axis, w_t the channel-wise
 * write gate on the value axis, g_t the channel-wise log-decay on the key axis
 * (alpha_t = exp g_t). gdr2_fwd / gdr2_bwd / gdr2_step take the gates already
 * activated; the *_logits variants take their logits and activate them inside
 * the kernels (see below). Nothing is normalised inside the operator. The
 * forward pass runs the chunkwise algorithm with the cumulative decay folded
 * into asymmetric erase factors and one shared WY/UT inverse (LIT-802
 * takeaway 2, App. A); the backward pass is the gate-aware one (App. B).
 *
 * Layouts (all contiguous, row-major, in the element type `dtype`):
 *   q, k, g, b and dq, dk, dg, db : [B][T][H][dk]
 *   v, w, o, dout and dv, dw      : [B][T][H][dv]
 *   h0, ht, dht, dh0              : [B][H][dk][dv], always fp32
 * Supported: dtype BF16 with dk, dv in {64, 128}; dtype F32 with dk = dv = 64;
 * chunk = 64; any T >= 0 (a partial last chunk is padded with zero tokens,
 * which leave the recurrence unchanged).
 *
 * Calls without tokens (B, T or H zero): the token tensors are empty, their pointers
 * may be NULL, and no workspace is needed (the size functions return 0, a NULL
 * workspace is accepted). A recurrence over no tokens ends where it starts, so
 * gdr2_fwd writes ht = h0 (zeros when h0 is NULL) and gdr2_bwd writes dh0 = dht
 * (zeros when dht is NULL), when ht / dh0 are given and B * H > 0; gdr2_step leaves
 * the state as it is (the state pointer is still required when B * H > 0). Nothing
 * else is enqueued.
 *
 * Ownership: the caller owns every buffer, including the workspace. All device
 * pointers must stay valid until the stream has passed the enqueued work. The
 * library allocates nothing, keeps no state between calls, never synchronises
 * and enqueues everything on `stream` (a hipStream_t, 0 = null stream). Calls on
 * different streams with different workspaces may run concurrently.
 *
 * Errors: every argument is checked on the host before any HIP call; a failed
 * check returns a negative status and enqueues nothing. A failed launch
 * returns GDR2_ERR_HIP. Non-finite inputs are not checked; they propagate.
 *
 * Decay: g is a log-decay (g <= 0, exp g in (0, 1]) of any finite size. The chunkwise
 * kernels scale their factors by exponentials of the decay summed over 16-token blocks;
 * where a block's decay is strong enough that the diagonal block factor would leave the
 * fp32 range, they form that block from per-element decay products instead, so every
 * finite g <= 0 gives finite results (LIT-802 takeaway 1: the channel-wise decay of
 * KDA, which bounds no decay strength).
 */
#ifndef GDR2_H
#define GDR2_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gdr2_dtype { GDR2_DTYPE_F32 = 0, GDR2_DTYPE_BF16 = 1 };

enum gdr2_status {
    GDR2_OK = 0,
    GDR2_ERR_NULL = -1,        /* a required pointer is NULL */
    GDR2_ERR_SHAPE = -2,       /* B, T or H negative, or sizes overflow */
    GDR2_ERR_UNSUPPORTED = -3, /* dk/dv/chunk/dtype combination not built */
    GDR2_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
    GDR2_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required */
    GDR2_ERR_HIP = -6,         /* a HIP launch failed */
    GDR2_ERR_VALUE = -7,       /* a scalar argument is out of range (gate scales, segments) */
    GDR2_ERR_SCRATCH = -8      /* gdr2_fwd_noalloc: the call needs more than the fixed scratch */
};

/* Bytes of workspace gdr2_fwd needs. save_for_bwd = 1 sizes it for a later
 * gdr2_bwd(..., fwd_saved = 1) on the same buffer. Returns 0 for unsupported
 * or invalid arguments, and for calls without tokens, which need none. */
size_t gdr2_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype,
                                int save_for_bwd);

/* Bytes of workspace gdr2_bwd needs (either value of fwd_saved). */
size_t gdr2_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int dtype);

/* Forward pass: writes o and, if ht != NULL, the final state.
 * h0: initial state or NULL (= 0). save_for_bwd = 1 also keeps in the
 * workspace what gdr2_bwd needs (per-chunk states and operands), so the
 * backward does not recompute the forward. */
int gdr2_fwd(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
             const float* h0, void* o, float* ht, int B, int T, int H, int dk, int dv, int chunk,
             int dtype, int save_for_bwd, void* workspace, size_t workspace_bytes, void* stream,
             void* const* stage_events);

/* Backward pass: given dout (= dL/do) and dht (= dL/dS_T, NULL = 0), writes
 * dq, dk_, dv_, dg, db, dw (same layouts and dtype as the inputs) and, if
 * dh0 != NULL, dL/dh0. fwd_saved = 1: the workspace holds what
 * gdr2_fwd(..., save_for_bwd = 1) left there for the same inputs and has not
 * been touched since; fwd_saved = 0: the forward quantities are recomputed
 * inside this call (o is not written). */
int gdr2_bwd(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
             const float* h0, const void* dout, const float* dht, void* dq, void* dk_, void* dv_,
             void* dg, void* db, void* dw, float* dh0, int B, int T, int H, int dk, int dv, int chunk,
             int dtype, int fwd_saved, void* workspace, size_t workspace_bytes, void* stream,
             void* const* stage_events);

/* Chunk-parallel scan of the state chains. gdr2_fwd / gdr2_bwd walk each sequence's
 * chunks in order, one chain per sequence and 16-column slice of the value axis, so a
 * call with few sequences and many chunks leaves most of the GPU idle. Only the state
 * is carried between chunks ("Gated DeltaNet-2", anthology record LIT-802, "Key
 * takeaways", second bullet; digg thread post 9/), and the carry is affine in it:
 * S_{c+1} = P_c S_c + H_c with P_c = diag(exp gamma_C) - Kd^T Wm and H_c = Kd^T U. These
 * variants cut every sequence into `segments` pieces of ceil(NT / segments) chunks
 * (NT = ceil(T / chunk); fewer pieces if T is short) and walk them at the same time:
 * summaries of each piece (its end state from a zero start and its transition, the
 * product of its P_c), an fp32 scan over the pieces for their true start states, then
 * the usual walk of every piece. The backward does the same in reverse with P^T.
 * Results equal the one-walk chains up to rounding order. The work grows (about 3x the
 * chain's), so it pays only when the sequences are too few to fill the GPU: gdr2_fwd,
 * gdr2_bwd and their _logits variants use it by themselves when B * H * dv / 16 <= 128,
 * with 512 / (B * H * dv / 16) segments, at most 8, of at least 16 chunks each (their
 * workspace sizes include it), and walk the chains whole otherwise; segments = 1 here
 * forces one walk. Workspace: gdr2_seg_workspace_bytes (with
 * save_for_bwd = 1 for the backward; a gdr2_bwd_seg(..., fwd_saved = 1) needs the
 * workspace of a gdr2_fwd_seg(..., save_for_bwd = 1) with the same segments). Errors
 * as gdr2_fwd / gdr2_bwd; segments < 1 returns GDR2_ERR_VALUE. */
size_t gdr2_seg_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, int segments, int dtype,
                                int save_for_bwd);

int gdr2_fwd_seg(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
                 const float* h0, void* o, float* ht, int B, int T, int H, int dk, int dv, int chunk,
                 int segments, int dtype, int save_for_bwd, void* workspace, size_t workspace_bytes,
                 void* stream, void* const* stage_events);

int gdr2_bwd_seg(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
                 const float* h0, const void* dout, const float* dht, void* dq, void* dk_, void* dv_,
                 void* dg, void* db, void* dw, float* dh0, int B, int T, int H, int dk, int dv, int chunk,
                 int segments, int dtype, int fwd_saved, void* workspace, size_t workspace_bytes,
                 void* stream, void* const* stage_events);

/* Recurrent step, for decoding: processes the T tokens of q, k, v, g, b, w one at a
 * time, starting from the state in `state` (fp32 [B][H][dk][dv], required), which is
 * read and then overwritten with the state after the last token; writes o (layouts as
 * above). Same recurrence as gdr2_fwd -- for state = h0 it returns the same o and final
 * state up to fp32 rounding order -- computed token by token with each head's state
 * held on chip: constant memory per head however long the sequence (chatpaper.ai
 * abstract of "Gated DeltaNet-2": constant-memory decoding). Supported dk/dv/dtype as
 * gdr2_fwd; no workspace; no backward. Errors as gdr2_fwd (GDR2_ERR_NULL when state
 * is NULL). */
int gdr2_step(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
              float* state, void* o, int B, int T, int H, int dk, int dv, int dtype, void* stream);

/* Gates as logits. The erase and write gates are sigmoids of their own projections
 * ("Gated DeltaNet-2", anthology record LIT-802, "Key takeaways", first bullet); these
 * entry points take the projections' outputs (logits) zg, zb, zw (layouts of g, b, w)
 * and apply, inside the kernels,
 *     b = b_scale * sigmoid(zb),   w = sigmoid(zw),   g = -g_scale * softplus(zg),
 * so that no separate elementwise pass over the gates is needed. b_scale = 1 is the
 * plain erase gate, b_scale = 2 the widened [0, 2] erase range of the paper's Table 5
 * ablation; 0 < b_scale <= 2. The log-decay parametrisation (any g_scale > 0, finite)
 * keeps the decay exp g in (0, 1); the pages leave it open and this is the reading
 * taken. The backward variant writes dL/dzg, dL/dzb, dL/dzw into dzg, dzb, dzw (the
 * other outputs as gdr2_bwd). Everything else -- layouts, dtypes, workspace (the same
 * size functions), ownership, events, errors -- is as for gdr2_fwd / gdr2_bwd /
 * gdr2_step; a scale out of range returns GDR2_ERR_VALUE and enqueues nothing.
 * A gdr2_bwd_logits(..., fwd_saved = 1) must follow gdr2_fwd_logits with the same
 * logits and scales. */
int gdr2_fwd_logits(const void* q, const void* k, const void* v, const void* zg, const void* zb,
                    const void* zw, float g_scale, float b_scale, const float* h0, void* o, float* ht,
                    int B, int T, int H, int dk, int dv, int chunk, int dtype, int save_for_bwd,
                    void* workspace, size_t workspace_bytes, void* stream, void* const* stage_events);

int gdr2_bwd_logits(const void* q, const void* k, const void* v, const void* zg, const void* zb,
                    const void* zw, float g_scale, float b_scale, const float* h0, const void* dout,
                    const float* dht, void* dq, void* dk_, void* dv_, void* dzg, void* dzb, void* dzw,
                    float* dh0, int B, int T, int H, int dk, int dv, int chunk, int dtype, int fwd_saved,
                    void* workspace, size_t workspace_bytes, void* stream, void* const* stage_events);

int gdr2_step_logits(const void* q, const void* k, const void* v, const void* zg, const void* zb,
                     const void* zw, float g_scale, float b_scale, float* state, void* o, int B, int T,
                     int H, int dk, int dv, int dtype, void* stream);

/* stage_events (gdr2_fwd and gdr2_bwd, and their _logits and _seg variants): NULL, or
 * an array of hipEvent_t for per-stage timing on `stream`: element 0 marks the start of
 * the first stage and element i the end of the i-th (a NULL element: no event at that
 * boundary). The events are attached to the
 * stages' kernel launches (start of the first kernel, end of the last), so timing puts no
 * extra commands between the kernels; a stage's interval therefore includes the launch
 * gap before its first kernel.
 * gdr2_fwd runs 2 stages (intra-chunk, state chain), so it needs 3 events; gdr2_bwd
 * runs 2 (reverse state chain, intra-chunk gradients) when fwd_saved = 1, and 4 (the
 * two forward stages first) when fwd_saved = 0, so it needs 3 or 5. With segments > 1
 * the chain stage also holds the summary and scan kernels. The events belong to the
 * caller. */

/* For callers that cannot allocate device memory -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc: the inference forward (gdr2_fwd with
 * save_for_bwd = 0) without a workspace argument. Its workspace is a fixed array of
 * GDR2_NOALLOC_SCRATCH_BYTES (64 MiB) of device memory inside the library; each GPU the
 * library runs on holds its own copy until the process ends. The call allocates nothing
 * (no hipMalloc, no hipFree, no allocating library routine); the caller still passes
 * every input and output. A call whose workspace, gdr2_fwd_workspace_bytes(B, T, H, dk,
 * dv, chunk, dtype, 0), exceeds the array returns GDR2_ERR_SCRATCH and enqueues nothing
 * (at d_k = d_v = 128 in bf16 about 72.5 KB per chunk of 64 tokens and head, so e.g.
 * B = 1, H = 16, T = 2048 fits); other errors as gdr2_fwd. All calls on one GPU share the
 * array, which keeps the last call's contents: calls that overlap on one GPU (several
 * streams, or several host threads) race on it and must be serialised by the caller.
 * Arguments, layouts and results otherwise as gdr2_fwd (bitwise the same results). */
#define GDR2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

int gdr2_fwd_noalloc(const void* q, const void* k, const void* v, const void* g, const void* b, const void* w,
                     const float* h0, void* o, float* ht, int B, int T, int H, int dk, int dv, int chunk,
                     int dtype, void* stream);

/* Static description of a status code. */
const char* gdr2_strerror(int status);

/* Library version as an integer (major * 10000 + minor * 100 + patch). */
int gdr2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR2_H */
