// Shared pieces of the two intra-chunk kernels: chunk-local cumulative
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
// Lane layout of these phases: wave w owns key-channel tiles w, w + NW, ...
// and lane (li, lq) holds channels 16a + 4lq + (0..3) of token rows 16t + li,
// t = 0..3 -- the accumulator-tile layout of a (channel x time) product, so the
// backward kernel meets the same positions again in its final phase.
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

// Raw 4-element row pieces (Raw4, gdr2_device.hpp): loads are issued for a whole
// phase before any of them is used, so a wave has all of its HBM requests in flight.

// raw[t] = elements ch .. ch + 3 of token row 16 t + li (row clamped to nvalid - 1)
template <class OT>
__device__ __forceinline__ void ld_rows(const OT* base, size_t rs, int ch, int nvalid,
                                        typename Raw4<OT>::type (&raw)[4]) {
    const int li = lane_id() & 15;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r = 16 * t + li, rr = r < nvalid ? r : nvalid - 1;
        raw[t] = *(const typename Raw4<OT>::type*)(base + (size_t)rr * rs + ch);
    }
}
// to fp32, rows at or past nvalid read as zero
template <class OT>
__device__ __forceinline__ void cvt_rows(const typename Raw4<OT>::type (&raw)[4], int nvalid, float (&out)[4][4]) {
    const int li = lane_id() & 15;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const bool ok = 16 * t + li < nvalid;
#pragma unroll
        for (int i = 0; i < 4; ++i) out[t][i] = ok ? (float)raw[t][i] : 0.f;
    }
}

// 16-byte row pieces: raw[t] = elements ch .. ch + 16 / sizeof(OT) - 1 of token row
// 16 t + li (row clamped to nvalid - 1)
template <class OT> struct Raw16;
template <> struct Raw16<bf16> { typedef bf16x8 type; };
template <> struct Raw16<float> { typedef f32x4 type; };
template <class OT>
__device__ __forceinline__ void ld_rows16(const OT* base, size_t rs, int ch, int nvalid,
                                          typename Raw16<OT>::type (&raw)[4]) {
    const int li = lane_id() & 15;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r = 16 * t + li, rr = r < nvalid ? r : nvalid - 1;
        raw[t] = *(const typename Raw16<OT>::type*)(base + (size_t)rr * rs + ch);
    }
}
// quarter hq (elements 4 hq .. 4 hq + 3) of 16-byte row pieces, to fp32; rows at or past
// nvalid read as zero
template <class OT>
__device__ __forceinline__ void cvt_rows16(const typename Raw16<OT>::type (&raw)[4], int hq, int nvalid,
                                           float (&out)[4][4]) {
    const int li = lane_id() & 15;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const bool ok = 16 * t + li < nvalid;
#pragma unroll
        for (int i = 0; i < 4; ++i) out[t][i] = ok ? (float)raw[t][4 * hq + i] : 0.f;
    }
}

template <class OT>
__device__ __forceinline__ void lds_put4(lds_char* p, const float v[4]) {
    if constexpr (sizeof(OT) == 2) {
        bf16x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (bf16)v[i];
        lds_store<bf16x4>(p, x);
    } else {
        f32x4 x = {v[0], v[1], v[2], v[3]};
        lds_store<f32x4>(p, x);
    }
}

// Per-lane cumulative log-decay for channel tile `at` (4 channels ch0..ch0+3, rows 16t+li)
// from the log-decays gv[t][i] of those rows: gam[t][i] (inclusive running sum over the
// chunk), g0[R][i] = gam at row 16R, ge[R][i] = gam at row 16R+15.
__device__ __forceinline__ void gamma_scan(const float (&gv)[4][4], float (&gam)[4][4], float (&g0)[4][4],
                                           float (&ge)[4][4]) {
    float run[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x = row_scan16(gv[t][i]) + run[i];
            gam[t][i] = x;
            run[i] = row_bcast(x, 15);
        }
#pragma unroll
    for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            g0[R][i] = row_bcast(gam[R][i], 0);
            ge[R][i] = row_bcast(gam[R][i], 15);
        }
}
template <class OT>
__device__ __forceinline__ void chunk_gamma(const OT* gb, size_t rs, int ch0, int nvalid, float (&gam)[4][4],
                                            float (&g0)[4][4], float (&ge)[4][4]) {
    const int li = lane_id() & 15;
    float gv[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) ld4_row(gb, rs, 16 * t + li, ch0, nvalid, gv[t]);
    gamma_scan(gv, gam, g0, ge);
}

// Factor arrays for the four channels ch0..ch0+3 (written by the li == 0 lanes).
template <int DK>
__device__ __forceinline__ void write_factors(lds_char* sF, int ch0, const float (&g0)[4][4],
                                              const float (&ge)[4][4]) {
    if ((lane_id() & 15) != 0) return;
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        float e0[4], ec[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            e0[i] = __expf(g0[R][i]);
            ec[i] = __expf(ge[3][i] - ge[R][i]);
        }
        lds_put4<float>(sF + ((F_ER0 + R) * DK + ch0) * 4, e0);
        lds_put4<float>(sF + ((F_ECE + R) * DK + ch0) * 4, ec);
#pragma unroll
        for (int I = 0; I <= R; ++I) {
            float sv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sv[i] = __expf(g0[R][i] - ge[I][i]);
            lds_put4<float>(sF + ((F_S + pair_id(R, I)) * DK + ch0) * 4, sv);
        }
    }
}

// XA = b*k*E1, XM = q*E1, Y = k*E2 for channel tile rows of this lane, into swizzled LDS
// tiles [CH][DK]; optionally also Qg = q*exp(gam) and Kd = k*exp(gam_C - gam) as swizzled
// tiles in global memory.
template <class OT, int DK>
__device__ __forceinline__ void scaled_factors_from(const float (&qv)[4][4], const float (&kv)[4][4],
                                                    const float (&bv)[4][4], int ch0, const float (&gam)[4][4],
                                                    const float (&g0)[4][4], const float (&ge)[4][4],
                                                    lds_char* sXA, lds_char* sXM, lds_char* sY, OT* qg_out,
                                                    OT* kd_out) {
    const int li = lane_id() & 15;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r = 16 * t + li;
        float xa[4], xm[4], y[4], qg[4], kd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float e1 = __expf(gam[t][i] - g0[t][i]);
            const float e2 = __expf(ge[t][i] - gam[t][i]);
            xa[i] = bv[t][i] * kv[t][i] * e1;
            xm[i] = qv[t][i] * e1;
            y[i] = kv[t][i] * e2;
            qg[i] = xm[i] * __expf(g0[t][i]);
            kd[i] = y[i] * __expf(ge[3][i] - ge[t][i]);
        }
        const int o = swz<OT, DK>(r, ch0) * (int)sizeof(OT);
        lds_put4<OT>(sXA + o, xa);
        lds_put4<OT>(sXM + o, xm);
        lds_put4<OT>(sY + o, y);
        if (qg_out) st4(qg_out + swz<OT, DK>(r, ch0), qg);
        if (kd_out) st4(kd_out + swz<OT, DK>(r, ch0), kd);
    }
}
template <class OT, int DK>
__device__ __forceinline__ void scaled_factors(const OT* qb, const OT* kb, const OT* bb, size_t rs, int ch0,
                                               int nvalid, const float (&gam)[4][4], const float (&g0)[4][4],
                                               const float (&ge)[4][4], lds_char* sXA, lds_char* sXM,
                                               lds_char* sY, OT* qg_out, OT* kd_out) {
    const int li = lane_id() & 15;
    float qv[4][4], kv[4][4], bv[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        ld4_row(qb, rs, 16 * t + li, ch0, nvalid, qv[t]);
        ld4_row(kb, rs, 16 * t + li, ch0, nvalid, kv[t]);
        ld4_row(bb, rs, 16 * t + li, ch0, nvalid, bv[t]);
    }
    scaled_factors_from<OT, DK>(qv, kv, bv, ch0, gam, g0, ge, sXA, sXM, sY, qg_out, kd_out);
}

// X = w * v into a swizzled LDS tile [CH][DV] at columns ch0 .. ch0 + 3
template <class OT, int DV>
__device__ __forceinline__ void x_tile_from(const float (&vv)[4][4], const float (&ww)[4][4], int ch0,
                                            lds_char* sX) {
    const int li = lane_id() & 15;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = vv[t][i] * ww[t][i];
        lds_put4<OT>(sX + swz<OT, DV>(16 * t + li, ch0) * (int)sizeof(OT), x);
    }
}
// X = w * v into a swizzled LDS tile [CH][DV] for value-channel tile jt
template <class OT, int DV>
__device__ __forceinline__ void chunk_x_tile(const OT* vb, const OT* wb, size_t rs, int jt, int nvalid,
                                             lds_char* sX) {
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    const int ch0 = 16 * jt + 4 * lq;
    float vv[4][4], ww[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        ld4_row(vb, rs, 16 * t + li, ch0, nvalid, vv[t]);
        ld4_row(wb, rs, 16 * t + li, ch0, nvalid, ww[t]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = vv[t][i] * ww[t][i];
        lds_put4<OT>(sX + swz<OT, DV>(16 * t + li, ch0) * (int)sizeof(OT), x);
    }
}

}  // namespace gdr2
