// Workspace layout shared by the host launcher and the kernels.
//
// Every array is chunk-major: element offset = chunk_id * per_chunk + local.
// chunk_id = (b * H + h) * NT + c. Fragment arrays hold 16x32 operand blocks of
// 512 elements (64 lanes x 8); tile dumps hold 16x16 accumulator tiles of 256
// elements (64 lanes x 4). Each array starts on a 256-byte boundary.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace gdr2 {

struct Layout {
    int DK, DV, esz;  // esz: bytes per operand element (2 for bf16, 4 for fp32)
    // per-chunk element counts
    size_t wmA, kdA, qgB, mB, u, gc;              // forward chain operands
    size_t mtA, kdRA, qgtA, wmtA, ttA;            // backward chain operands
    size_t s, ds, delta, dy;                      // saved states and chain outputs
    // byte offsets of each array from the workspace base
    size_t o_wmA, o_kdA, o_qgB, o_mB, o_u, o_gc;
    size_t o_mtA, o_kdRA, o_qgtA, o_wmtA, o_ttA;
    size_t o_s, o_ds, o_delta, o_dy;
    size_t fwd_infer_bytes;  // arrays needed by an inference forward
    size_t train_bytes;      // everything a forward + backward needs
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline Layout make_layout(long long nchunks, int DK, int DV, int esz) {
    Layout L;
    L.DK = DK;
    L.DV = DV;
    L.esz = esz;
    const size_t C = 64;
    L.wmA = C * DK;        // A fragments of Wm          [4 mt][DK/32 kb]
    L.kdA = (size_t)DK * C;  // A fragments of Kd^T      [DK/16 mt][2 kb]
    L.qgB = C * DK;        // B fragments of Qg^T        [4 nt][DK/32 kb]
    L.mB = C * C;          // B fragments of M^T         [4 nt][2 kb]
    L.u = C * DV;          // U accumulator tiles        [DV/16][4]
    L.gc = DK;             // exp(gamma_C), fp32
    L.mtA = C * C;         // A fragments of M^T         [4 mt][2 kb]
    L.kdRA = C * DK;       // A fragments of Kd          [4 mt][DK/32 kb]
    L.qgtA = (size_t)DK * C;  // A fragments of Qg^T     [DK/16 mt][2 kb]
    L.wmtA = (size_t)DK * C;  // A fragments of Wm^T     [DK/16 mt][2 kb]
    L.ttA = C * C;         // A fragments of T^T         [4 mt][2 kb]
    L.s = (size_t)DK * DV;   // chunk start state, row-major [DK][DV]
    L.ds = (size_t)DK * DV;  // gradient w.r.t. the chunk end state, row-major
    L.delta = C * DV;      // Delta tiles                [DV/16][4]
    L.dy = C * DV;         // dY tiles                   [DV/16][4]
    size_t off = 0;
    auto take = [&](size_t elems, size_t el_bytes) {
        size_t o = off;
        off += align256((size_t)nchunks * elems * el_bytes);
        return o;
    };
    L.o_wmA = take(L.wmA, esz);
    L.o_kdA = take(L.kdA, esz);
    L.o_qgB = take(L.qgB, esz);
    L.o_mB = take(L.mB, esz);
    L.o_u = take(L.u, esz);
    L.o_gc = take(L.gc, 4);
    L.fwd_infer_bytes = off;
    L.o_mtA = take(L.mtA, esz);
    L.o_kdRA = take(L.kdRA, esz);
    L.o_qgtA = take(L.qgtA, esz);
    L.o_wmtA = take(L.wmtA, esz);
    L.o_ttA = take(L.ttA, esz);
    L.o_s = take(L.s, esz);
    L.o_ds = take(L.ds, esz);
    L.o_delta = take(L.delta, esz);
    L.o_dy = take(L.dy, esz);
    L.train_bytes = off;
    return L;
}

}  // namespace gdr2
