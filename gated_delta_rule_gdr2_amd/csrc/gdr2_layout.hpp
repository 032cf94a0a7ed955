// Workspace layout shared by the host launcher and the kernels.
//
// Every array is chunk-major: element offset = chunk_id * per_chunk + local,
// chunk_id = (b * H + h) * NT + c. Per-chunk matrices are stored once each in the
// operand type: Wm, Kd^T, Qg and M as fragment images (fimg() in gdr2_device.hpp),
// which the forward chain loads fragment by fragment into registers and the backward
// chain copies into LDS and reads transposed; T as a swizzled row-major tile (swz()).
// Accumulator-tile dumps (U, Delta, dY) hold 16x16 tiles as 64 lanes x 4 elements,
// ordered [value-column tile][token tile]. The saved states S and dS' are fragment-major
// (fmaj_off in gdr2_device.hpp). Each array starts on a 256-byte boundary.
//
// With the chains split into NSEG segments per sequence (chunk-parallel scan), three
// fp32 arrays per (sequence, segment) come last (after the training arrays in a training
// workspace, after the forward's in an inference one, so that no other offset depends on
// NSEG): the segment's transition P [DK][DK], a zero-start summary [DK][DV] (forward:
// end state; backward: start-state gradient) and the true boundary state [DK][DV]
// (forward: start state; backward: end-state gradient), all row-major.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace gdr2 {

struct Layout {
    int DK, DV, esz;  // esz: bytes per operand element (2 for bf16, 4 for fp32)
    // per-chunk element counts
    size_t wm, kd, qg, m, u, gc;     // forward: Wm [64][DK], Kd^T [DK][64], Qg [64][DK], M [64][64], U tiles, exp(gam_C)
    size_t t;                        // backward: T = (I + A)^-1 [64][64]
    size_t s, ds, delta, dy;         // chunk start state / end-state gradient [DK][DV], Delta / dY tiles
    size_t o_wm, o_kd, o_qg, o_m, o_u, o_gc, o_t, o_s, o_ds, o_delta, o_dy;  // byte offsets
    int nseg;                        // segments per sequence (1: no scan arrays)
    size_t segp, segh, segx;         // per (sequence, segment) element counts, fp32
    size_t o_segp, o_segh, o_segx;   // byte offsets
    size_t fwd_infer_bytes;          // arrays an inference forward needs
    size_t train_bytes;              // everything a forward + backward needs
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// train: the layout of a workspace that also holds what the backward needs
inline Layout make_layout(long long nchunks, int DK, int DV, int esz, long long nseq, int nseg, bool train) {
    Layout L;
    L.DK = DK;
    L.DV = DV;
    L.esz = esz;
    const size_t C = 64;
    L.wm = C * DK;
    L.kd = C * DK;
    L.qg = C * DK;
    L.m = C * C;
    L.u = C * DV;
    L.gc = DK;  // fp32
    L.t = C * C;
    L.s = (size_t)DK * DV;
    L.ds = (size_t)DK * DV;
    L.delta = C * DV;
    L.dy = C * DV;
    size_t off = 0;
    auto take = [&](size_t elems, size_t el_bytes) {
        size_t o = off;
        off += align256((size_t)nchunks * elems * el_bytes);
        return o;
    };
    L.o_wm = take(L.wm, esz);
    L.o_kd = take(L.kd, esz);
    L.o_qg = take(L.qg, esz);
    L.o_m = take(L.m, esz);
    L.o_u = take(L.u, esz);
    L.o_gc = take(L.gc, 4);
    const size_t fwd_end = off;
    L.o_t = take(L.t, esz);
    L.o_s = take(L.s, esz);
    L.o_ds = take(L.ds, esz);
    L.o_delta = take(L.delta, esz);
    L.o_dy = take(L.dy, esz);
    const size_t train_end = off;
    L.nseg = nseg;
    L.segp = (size_t)DK * DK;
    L.segh = (size_t)DK * DV;
    L.segx = (size_t)DK * DV;
    const long long nsub = nseg > 1 ? nseq * nseg : 0;  // (sequence, segment) pairs
    const size_t segbytes = align256((size_t)nsub * L.segp * 4) + 2 * align256((size_t)nsub * L.segh * 4);
    L.o_segp = train ? train_end : fwd_end;
    L.o_segh = L.o_segp + align256((size_t)nsub * L.segp * 4);
    L.o_segx = L.o_segh + align256((size_t)nsub * L.segh * 4);
    L.fwd_infer_bytes = fwd_end + segbytes;
    L.train_bytes = train_end + segbytes;
    return L;
}

}  // namespace gdr2
