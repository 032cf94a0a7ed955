// Shared first phase of the two intra-chunk kernels: chunk-local cumulative
// log-decay and the decay-scaled key/query factors.
//
// Normalising the state by the cumulative decay inside a chunk folds the
// channel-wise decay into the two factors of each rank-one erase ("Gated
// DeltaNet-2", anthology record LIT-802, takeaway 2; chatpaper abstract:
// "channel-wise decay absorbed into asymmetric erase factors"). With
// gam_r = sum_{i<=r} g_i inside the chunk, the intra-chunk products need
// exp(gam_r - gam_i). To keep every exponential in range whatever the decay,
// it is split at 16-row block boundaries:
//   exp(gam_r - gam_i) = E1_r * s(R, I) * E2_i,
//   E1_r = exp(gam_r - gam_R0)   (<= 1; R0 = first row of r's block R)
//   E2_i = exp(gam_Iend - gam_i) (<= 1; Iend = last row of i's block I)
//   s(R, I) = exp(gam_R0 - gam_Iend) (<= 1 for I < R; covers < 16 tokens for I = R)
// Layout of this phase: wave w owns key-channel tiles [w*CPW, (w+1)*CPW) and
// lane (li, lq) holds channels 16a + 4lq + (0..3) of token rows 16t + li,
// t = 0..3 -- the accumulator-tile layout of a (channel x time) product, so
// the backward kernel can reuse the same registers in its final phase.
#pragma once
#include "gdr2_device.hpp"

namespace gdr2 {

// fp32 factor arrays kept in LDS, each [.][DK]:
//   eR0[R][c] = exp(gam_R0),  eCe[R][c] = exp(gam_C - gam_Rend),  s[pair(R,I)][c]
constexpr int F_ER0 = 0;
constexpr int F_ECE = NBLK;
constexpr int F_S = 2 * NBLK;
constexpr int F_ROWS = 2 * NBLK + NPAIR;

template <class OT>
constexpr int pad_ot() { return sizeof(OT) == 2 ? 8 : 4; }

// Load 4 consecutive elements of token row r (row stride rs) at column ch; rows at or
// past nvalid (>= 1) read as zero. Branch-free: the address is clamped to a valid row
// and the value selected afterwards, so independent loads can all be in flight at once.
template <class IT>
__device__ __forceinline__ void ld4_row(const IT* base, size_t rs, int r, int ch, int nvalid, float out[4]) {
    const int rr = r < nvalid ? r : nvalid - 1;
    ld4(base + (size_t)rr * rs + ch, out);
    const bool ok = r < nvalid;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = ok ? out[i] : 0.f;
}

// Computes gam (registers), the factor arrays (LDS), exp(gam_C) (global) and
// the scaled matrices XA = b*k*E1, XM = q*E1, Y = k*E2 (LDS, [CH][LDK]).
// base_* point at token row 0 of this chunk; rs = H * DK is the token stride.
template <class OT, int DK>
__device__ __forceinline__ void chunk_factors(const OT* gb, const OT* qb, const OT* kb, const OT* bb,
                                              size_t rs, int nvalid, float (&gam)[DK / 64][4][4],
                                              OT* sXA, OT* sXM, OT* sY, int LDK, float* sF,
                                              float* gc_out) {
    constexpr int CPW = DK / 64;
    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, li = l & 15, lq = l >> 4;
#pragma unroll
    for (int ac = 0; ac < CPW; ++ac) {
        const int ch0 = 16 * (wv * CPW + ac) + 4 * lq;
        float run[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = 16 * t + li;
            float gv[4];
            ld4_row(gb, rs, r, ch0, nvalid, gv);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x = row_scan16(gv[i]) + run[i];
                gam[ac][t][i] = x;
                run[i] = row_bcast(x, 15);
            }
        }
        float g0[4][4], ge[4][4];  // gam at block start / end rows, per block R
#pragma unroll
        for (int R = 0; R < 4; ++R)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                g0[R][i] = row_bcast(gam[ac][R][i], 0);
                ge[R][i] = row_bcast(gam[ac][R][i], 15);
            }
        if (li == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = ch0 + i;
#pragma unroll
                for (int R = 0; R < 4; ++R) {
                    sF[(F_ER0 + R) * DK + c] = __expf(g0[R][i]);
                    sF[(F_ECE + R) * DK + c] = __expf(ge[3][i] - ge[R][i]);
#pragma unroll
                    for (int I = 0; I <= R; ++I) sF[(F_S + pair_id(R, I)) * DK + c] = __expf(g0[R][i] - ge[I][i]);
                }
                if (gc_out) gc_out[c] = __expf(ge[3][i]);
            }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = 16 * t + li;
            float qv[4], kv[4], bv[4], xa[4], xm[4], y[4];
            ld4_row(qb, rs, r, ch0, nvalid, qv);
            ld4_row(kb, rs, r, ch0, nvalid, kv);
            ld4_row(bb, rs, r, ch0, nvalid, bv);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e1 = __expf(gam[ac][t][i] - g0[t][i]);
                const float e2 = __expf(ge[t][i] - gam[ac][t][i]);
                xa[i] = bv[i] * kv[i] * e1;
                xm[i] = qv[i] * e1;
                y[i] = kv[i] * e2;
            }
            st4(sXA + r * LDK + ch0, xa);
            st4(sXM + r * LDK + ch0, xm);
            st4(sY + r * LDK + ch0, y);
        }
    }
}

// X = w * v into LDS [CH][LDV] (value channels, same lane layout)
template <class OT, int DV>
__device__ __forceinline__ void chunk_x(const OT* vb, const OT* wb, size_t rs, int nvalid, OT* sX, int LDV) {
    constexpr int VPW = DV / 64;
    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, li = l & 15, lq = l >> 4;
#pragma unroll
    for (int jc = 0; jc < VPW; ++jc) {
        const int ch0 = 16 * (wv * VPW + jc) + 4 * lq;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = 16 * t + li;
            float vv[4], ww[4], x[4];
            ld4_row(vb, rs, r, ch0, nvalid, vv);
            ld4_row(wb, rs, r, ch0, nvalid, ww);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = vv[i] * ww[i];
            st4(sX + r * LDV + ch0, x);
        }
    }
}

}  // namespace gdr2
