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

// gates passed as logits: activate a lane's rows 16 t + li (4 channels each) in place;
// rows at or past nvalid stay zero (a zero log-decay keeps the chunk's cumulative decay
// at its last real token)
template <class OT, int KIND>
__device__ __forceinline__ void activate_rows(float (&x)[4][4], int nvalid, float g_scale, float b_scale) {
    const int li = lane_id() & 15;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const bool ok = 16 * t + li < nvalid;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[t][i] = ok ? gate_act<OT, KIND>(x[t][i], g_scale, b_scale) : 0.f;
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
            run[i] = row_bcast<15>(x);
        }
#pragma unroll
    for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            g0[R][i] = row_bcast<0>(gam[R][i]);
            ge[R][i] = row_bcast<15>(gam[R][i]);
        }
}
// Row-uniform exponentials of four channels ch0..ch0+3. They are the same in all 16
// lanes of a row, so each lane computes a different one: lane li holds, for channel
// ch0 + i,
//   x0[i]: li < 10          s(R, I) = exp(gam_R0 - gam_Iend), (R, I) = pair_ri(li)
//          li = 10 .. 13    exp(gam_R0), R = li - 10
//          li = 14, 15      exp(gam_C - gam_Rend), R = li - 14
//   x1[i]: li = 0           exp(gam_C - gam_2end)
//          li = 1           exp(gam_C)
//          li = 2           exp(gam_C - gam_3end) = 1
// (gam_C = gam at the chunk's last row = gam_3end.) row_bcast moves them to the
// lanes that use them.
struct RowExp {
    float x0[4], x1[4];
};
static_assert(NPAIR + NBLK + 2 == 16, "the row-uniform exponentials fill one 16-lane row");

// broadcast of lane `src` of the row; src must fold to a constant after unrolling
__device__ __forceinline__ float row_bcast_c(float x, int src) {
    switch (src) {
        case 0: return row_bcast<0>(x);
        case 1: return row_bcast<1>(x);
        case 2: return row_bcast<2>(x);
        case 3: return row_bcast<3>(x);
        case 4: return row_bcast<4>(x);
        case 5: return row_bcast<5>(x);
        case 6: return row_bcast<6>(x);
        case 7: return row_bcast<7>(x);
        case 8: return row_bcast<8>(x);
        case 9: return row_bcast<9>(x);
        case 10: return row_bcast<10>(x);
        case 11: return row_bcast<11>(x);
        case 12: return row_bcast<12>(x);
        case 13: return row_bcast<13>(x);
        case 14: return row_bcast<14>(x);
        default: return row_bcast<15>(x);
    }
}
// exp(gam_R0) and exp(gam_C - gam_Rend) of channel ch0 + i in every lane (R, i constants)
__device__ __forceinline__ float rx_er0(const RowExp& x, int R, int i) { return row_bcast_c(x.x0[i], NPAIR + R); }
__device__ __forceinline__ float rx_ece(const RowExp& x, int R, int i) {
    if (R < 2) return row_bcast_c(x.x0[i], NPAIR + NBLK + R);
    if (R == 2) return row_bcast<0>(x.x1[i]);
    return 1.f;
}

// Computes the row-uniform exponentials and writes the factor arrays of channels
// ch0..ch0+3 (eR0, eCe and s rows of sF).
template <int DK>
__device__ __forceinline__ void row_exps(lds_char* sF, int ch0, const float (&g0)[4][4], const float (&ge)[4][4],
                                         RowExp& x) {
    const int li = lane_id() & 15;
    // lane li's value is exp(A - B): ra = 0..3 -> A = gam_{ra,0}, 4 -> A = gam_C;
    // ib = 0..3 -> B = gam_{ib,end}, 4 -> B = 0
    // (all selects, no branches: pair_ri written out for li < NPAIR)
    const int pr = li >= 6 ? 3 : li >= 3 ? 2 : li >= 1 ? 1 : 0, pi = li - pr * (pr + 1) / 2;
    const int ra = li < NPAIR ? pr : li < NPAIR + NBLK ? li - NPAIR : 4;
    const int ib = li < NPAIR ? pi : li < NPAIR + NBLK ? 4 : li - NPAIR - NBLK;
    const bool a0 = ra == 0, a1 = ra == 1, a2 = ra == 2, a3 = ra == 3;
    const bool b0 = ib == 0, b1 = ib == 1, b2 = ib == 2, b3 = ib == 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float A = ge[3][i], B = 0.f;
        A = a3 ? g0[3][i] : A;
        A = a2 ? g0[2][i] : A;
        A = a1 ? g0[1][i] : A;
        A = a0 ? g0[0][i] : A;
        B = b3 ? ge[3][i] : B;
        B = b2 ? ge[2][i] : B;
        B = b1 ? ge[1][i] : B;
        B = b0 ? ge[0][i] : B;
        x.x0[i] = __expf(A - B);
        const float B1 = li == 0 ? ge[2][i] : li == 2 ? ge[3][i] : 0.f;
        x.x1[i] = __expf(ge[3][i] - B1);
    }
    const int row = li < NPAIR ? F_S + li : li < NPAIR + NBLK ? F_ER0 + (li - NPAIR) : F_ECE + (li - NPAIR - NBLK);
    lds_put4<float>(sF + (row * DK + ch0) * 4, x.x0);
    if (li == 0 || li == 2) lds_put4<float>(sF + ((F_ECE + 2 + li / 2) * DK + ch0) * 4, x.x1);
}

// XA = b*k*E1, XM = q*E1, Y = k*E2 for channel tile rows of this lane, into swizzled LDS
// tiles [CH][DK]; with OUTS also Qg = q*exp(gam) and Kd = k*exp(gam_C - gam) as swizzled
// tiles in global memory (exp(gam) = E1 * exp(gam_R0), exp(gam_C - gam) = E2 *
// exp(gam_C - gam_Rend), the row-uniform factors taken from rx).
template <class OT, int DK, bool OUTS>
__device__ __forceinline__ void scaled_factors_from(const float (&qv)[4][4], const float (&kv)[4][4],
                                                    const float (&bv)[4][4], int ch0, const float (&gam)[4][4],
                                                    const float (&g0)[4][4], const float (&ge)[4][4],
                                                    lds_char* sXA, lds_char* sXM, lds_char* sY, OT* qg_out,
                                                    OT* kd_out, const RowExp* rx) {
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
            if constexpr (OUTS) {
                qg[i] = xm[i] * rx_er0(*rx, t, i);
                kd[i] = y[i] * rx_ece(*rx, t, i);
            }
        }
        const int o = swz<OT, DK>(r, ch0) * (int)sizeof(OT);
        lds_put4<OT>(sXA + o, xa);
        lds_put4<OT>(sXM + o, xm);
        lds_put4<OT>(sY + o, y);
        if constexpr (OUTS) {
            st4(qg_out + swz<OT, DK>(r, ch0), qg);
            st4(kd_out + swz<OT, DK>(r, ch0), kd);
        }
    }
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
// Row tensors staged through LDS. A chunk's CH rows of a row-major tensor [.][RL]
// (row stride rs elements) are copied into a swizzled LDS tile [CH][RL] by
// asynchronous global->LDS DMA, 16 bytes per lane. One instruction fills 1 KB of the
// tile, i.e. whole rows (4 of 256 bytes or 8 of 128 bytes), so every request is a whole
// cache line; the lane that fills position p of row r fetches chunk p ^ f(r) of the row
// (the swizzle only permutes chunks within a row). Lanes of rows at or past nvalid
// issue no copy (their positions are written by zero_tail_rows alone, so the two never
// race). Instructions n = w, w + NW, ... belong to wave w.
template <class OT, int RL, int NW>
__device__ __forceinline__ void dma_rows(const OT* base, size_t rs, int nvalid, lds_char* tile, int wv) {
    constexpr int EPC = 16 / (int)sizeof(OT);
    constexpr int NCH = RL / EPC;  // 16-byte chunks per row
    constexpr int RPI = 64 / NCH;  // rows per instruction
    constexpr int NI = CH / RPI;   // instructions per tile
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < (NI + NW - 1) / NW; ++i) {
        const int n = wv + NW * i;
        if (NI % NW == 0 || n < NI) {
            const int row = n * RPI + l / NCH, pos = l % NCH;
            const int c = pos ^ swz_f<OT, RL>(row);
            if (row < nvalid) {
                const char* src = (const char*)(base + (size_t)row * rs + c * EPC);
                __builtin_amdgcn_global_load_lds(src, (lds_void*)(tile + n * 1024), 16, 0, 0);
            }
        }
    }
}
// Rows 0 .. nvalid - 1 of a swizzled LDS tile [CH][RL] out to a row-major tensor (row
// stride rs elements), 16 bytes per lane with consecutive lanes on consecutive chunks
// of a row, so every request is a whole cache line (all threads of the workgroup).
template <class OT, int RL, int NTHR>
__device__ __forceinline__ void store_rows_tiles(const lds_char* tile, OT* dst, size_t rs, int nvalid) {
    constexpr int EPC = 16 / (int)sizeof(OT);
    constexpr int NCH = RL / EPC;
#pragma unroll
    for (int i = 0; i < (CH * NCH + NTHR - 1) / NTHR; ++i) {
        const int u = (int)threadIdx.x + NTHR * i, row = u / NCH, pos = u % NCH;
        if ((CH * NCH % NTHR == 0 || u < CH * NCH) && row < nvalid) {
            const f32x4 x = lds_load<f32x4>(tile + u * 16);
            *(f32x4*)(dst + (size_t)row * rs + (pos ^ swz_f<OT, RL>(row)) * EPC) = x;
        }
    }
}

// zero rows nvalid .. CH - 1 of a swizzled tile [CH][RL] (all threads of the workgroup)
template <class OT, int RL, int NTHR>
__device__ __forceinline__ void zero_tail_rows(lds_char* tile, int nvalid) {
    constexpr int NCH = RL * (int)sizeof(OT) / 16;
    for (int u = nvalid * NCH + (int)threadIdx.x; u < CH * NCH; u += NTHR) lds_store<f32x4>(tile + u * 16, f32x4{});
}

}  // namespace gdr2
