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
// Every exponent is formed as a sum of exactly the log-decays it spans -- E1_r from
// the block's g summed over (R0, r], E2_i over (i, Iend], s(R, I) from the first g of
// block R and the totals of the blocks in between -- never as a difference of two
// running sums, so an exponent carries the rounding of its own terms only, however
// large the decay elsewhere in the chunk.
// For I = R the factor s(R, R) = exp(-(sum of g over (R0, Rend])) >= 1 grows with the
// decay inside the block. When it passes exp(span_max()) somewhere in the chunk
// (strong decay), the kernels compute the four diagonal 16x16 blocks from
// per-element factors exp(gam_r - gam_i) = product of exp(g_t) over t in (i, r], each
// <= 1, instead ("slow path"), which is exact for any decay.
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

// A lane's log-decays (rows 16t + li, channels ch0 + i) are kept in one of two forms,
// chosen by the operand precision (DecayRep<OT>):
//   bf16 operands: p = the block-local inclusive running sum of g (one row scan); the
//     factors are exp of differences of p (E1 = exp(p_r - p_R0), E2 = exp(p_Rend - p_r)),
//     whose rounding (a few ulp of the block's running sum) stays far below bf16's;
//   fp32 operands: the raw g; every factor is exp of a sum of exactly the log-decays it
//     spans (E1 from a prefix scan without the block's first row, E2 from a suffix scan
//     after the row), never a difference of running sums, so one very strong decay in a
//     block costs no fp32 accuracy in the factors of the others.
// From either form: f[R][i] = g at row 16R (the block's first), tot[R][i] = sum of g over
// the block, inn[R][i] = sum of g over the block without its first row (s(R, R) = exp(-inn)).
__device__ __forceinline__ float block_e1(float g) {  // exact form: exp(sum of g over (R0, r])
    return __expf(row_scan16((lane_id() & 15) == 0 ? 0.f : g));
}
__device__ __forceinline__ float block_e2(float g) { return __expf(row_suffix16(row_shl1(g))); }

template <class OT>
struct DecayRep {
    static constexpr bool EXACT = sizeof(OT) == 4;
    // the stored form from the log-decays
    static __device__ __forceinline__ void store(const float (&gv)[4][4], float (&rep)[4][4]) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) rep[t][i] = EXACT ? gv[t][i] : row_scan16(gv[t][i]);
    }
    static __device__ __forceinline__ void scan(const float (&rep)[4][4], float (&f)[4][4], float (&tot)[4][4],
                                                float (&inn)[4][4]) {
        const bool first = (lane_id() & 15) == 0;
#pragma unroll
        for (int R = 0; R < 4; ++R)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f[R][i] = row_bcast<0>(rep[R][i]);
                if constexpr (EXACT) {
                    tot[R][i] = row_sum16(rep[R][i]);
                    inn[R][i] = row_sum16(first ? 0.f : rep[R][i]);
                } else {
                    tot[R][i] = row_bcast<15>(rep[R][i]);
                    inn[R][i] = tot[R][i] - f[R][i];
                }
            }
    }
    // E1 and E2 of a lane's row in block t, one channel
    static __device__ __forceinline__ void e12(float x, float& e1, float& e2) {
        if constexpr (EXACT) {
            e1 = block_e1(x);
            e2 = block_e2(x);
        } else {
            e1 = __expf(x - row_bcast<0>(x));
            e2 = __expf(row_bcast<15>(x) - x);
        }
    }
    // exp(g) of the lane's own row
    static __device__ __forceinline__ float alpha(float x) {
        if constexpr (EXACT) return expf(x);
        else return __expf(x - row_shr1(x));
    }
    // the block's total sum of g, in every lane
    static __device__ __forceinline__ float total(float x) {
        if constexpr (EXACT) return row_sum16(x);
        else return row_bcast<15>(x);
    }
};
template <class OT>
__device__ __forceinline__ void block_factors(const float (&rep)[4][4], float (&e1)[4][4], float (&e2)[4][4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) DecayRep<OT>::e12(rep[t][i], e1[t][i], e2[t][i]);
}
// Largest s(R, R) exponent -inn_R of a lane's channels (>= 0 for a decay g <= 0).
__device__ __forceinline__ float diag_span(const float (&inn)[4][4]) {
    float m = 0.f;
#pragma unroll
    for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, -inn[R][i]);
    return m;
}
// Above this s(R, R) exponent the diagonal blocks take the slow path. bf16 operands:
// the factors stay far inside the fp32/bf16 range; fp32 operands: the fast path's
// product of three exponentials keeps about span * 1e-7 relative error, so it stops
// early enough for the 1e-5 fp32 tolerance.
template <class OT>
constexpr float span_max() { return sizeof(OT) == 2 ? 60.f : 12.f; }

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
// lanes that use them. Each exponent is a sum of the block totals tot_J and block
// first values f_R it spans (gam_R0 - gam_Iend = f_R + sum_{I<J<R} tot_J, gam_R0 =
// f_R + sum_{J<R} tot_J, gam_C - gam_Rend = sum_{J>R} tot_J; for I = R,
// gam_R0 - gam_Rend = -inn_R), so no two large running sums are subtracted.
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
// ch0..ch0+3 (eR0, eCe and s rows of sF) from the block first values f and totals tot.
template <int DK>
__device__ __forceinline__ void row_exps(lds_char* sF, int ch0, const float (&f)[4][4], const float (&tot)[4][4],
                                         const float (&inn)[4][4], RowExp& x) {
    const int li = lane_id() & 15;
    // Lane li's exponent is -inn_R for a diagonal pair, else (F_R, the first value of
    // block R, if useF) + sum of tot_J over the J in mask. Lanes: pairs (R, I) in pair_ri
    // order, then gam_R0 for R = 0..3, then gam_C - gam_Rend for R = 0, 1.
    //                      li:  0  1  2  3  4  5  6  7  8  9 10 11 12 13 14 15
    // R (row of F)         :    0  1  1  2  2  2  3  3  3  3  0  1  2  3  -  -
    // diag                 :    1  0  1  0  0  1  0  0  0  1  0  0  0  0  0  0
    // mask of tot_J        :    0  0  0  2  0  0  6  4  0  0  0  1  3  7 14 12
    const int Rof = li < 1 ? 0 : li < 3 ? 1 : li < 6 ? 2 : li < 10 ? 3 : li - 10;  // li >= 14: no F
    const bool r0 = Rof == 0, r1 = Rof == 1, r2 = Rof == 2, r3 = Rof == 3;  // (selects, no indexing)
    const bool useF = li < 14;
    const bool diag = li == 0 || li == 2 || li == 5 || li == 9;
    const int mask = li == 3 ? 2 : li == 6 ? 6 : li == 7 ? 4 : li == 11 ? 1 : li == 12 ? 3 : li == 13 ? 7
                   : li == 14 ? 14 : li == 15 ? 12 : 0;
    const bool m0 = mask & 1, m1 = mask & 2, m2 = mask & 4, m3 = mask & 8;
    const bool x1a = li == 0, x1b = li == 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float F = 0.f, In = 0.f;
        F = r3 ? f[3][i] : F;
        F = r2 ? f[2][i] : F;
        F = r1 ? f[1][i] : F;
        F = r0 ? f[0][i] : F;
        In = r3 ? inn[3][i] : In;
        In = r2 ? inn[2][i] : In;
        In = r1 ? inn[1][i] : In;
        In = r0 ? inn[0][i] : In;
        float e = useF ? F : 0.f;
        e = diag ? -In : e;
        e += m0 ? tot[0][i] : 0.f;
        e += m1 ? tot[1][i] : 0.f;
        e += m2 ? tot[2][i] : 0.f;
        e += m3 ? tot[3][i] : 0.f;
        x.x0[i] = __expf(e);
        // x1: li 0 -> gam_C - gam_2end = tot_3; li 1 -> gam_C = sum of all totals; else 0
        const float all = (tot[0][i] + tot[1][i]) + (tot[2][i] + tot[3][i]);
        float e1 = 0.f;
        e1 = x1a ? tot[3][i] : e1;
        e1 = x1b ? all : e1;
        x.x1[i] = __expf(e1);
    }
    const int row = li < NPAIR ? F_S + li : li < NPAIR + NBLK ? F_ER0 + (li - NPAIR) : F_ECE + (li - NPAIR - NBLK);
    lds_put4<float>(sF + (row * DK + ch0) * 4, x.x0);
    if (li == 0 || li == 2) lds_put4<float>(sF + ((F_ECE + 2 + li / 2) * DK + ch0) * 4, x.x1);
}

// XA = b*k*E1, XM = q*E1, Y = k*E2 (E1, E2 from the lane's log-decays in their stored form
// rep, see DecayRep) for channel tile rows of this lane, into swizzled LDS tiles [CH][DK];
// with OUTS also Qg = q*exp(gam) of the same positions into qgv (exp(gam) = E1 * exp(gam_R0),
// the row-uniform factor taken from rx).
template <class OT, int DK, bool OUTS>
__device__ __forceinline__ void scaled_factors(const float (&qv)[4][4], const float (&kv)[4][4],
                                               const float (&bv)[4][4], int ch0, const float (&e1v)[4][4],
                                               const float (&e2v)[4][4], lds_char* sXA, lds_char* sXM, lds_char* sY,
                                               float (*qgv)[4], const RowExp* rx) {
    const int li = lane_id() & 15;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r = 16 * t + li;
        float xa[4], xm[4], y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float e1 = e1v[t][i], e2 = e2v[t][i];
            xa[i] = bv[t][i] * kv[t][i] * e1;
            xm[i] = qv[t][i] * e1;
            y[i] = kv[t][i] * e2;
            if constexpr (OUTS) qgv[t][i] = xm[i] * rx_er0(*rx, t, i);
        }
        const int o = swz<OT, DK>(r, ch0) * (int)sizeof(OT);
        lds_put4<OT>(sXA + o, xa);
        lds_put4<OT>(sXM + o, xm);
        lds_put4<OT>(sY + o, y);
    }
}
// ... with E1, E2 formed here from the lane's log-decays
template <class OT, int DK, bool OUTS>
__device__ __forceinline__ void scaled_factors_from(const float (&qv)[4][4], const float (&kv)[4][4],
                                                    const float (&bv)[4][4], int ch0, const float (&rep)[4][4],
                                                    lds_char* sXA, lds_char* sXM, lds_char* sY, float (*qgv)[4],
                                                    const RowExp* rx) {
    float e1[4][4], e2[4][4];
    block_factors<OT>(rep, e1, e2);
    scaled_factors<OT, DK, OUTS>(qv, kv, bv, ch0, e1, e2, sXA, sXM, sY, qgv, rx);
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
// of a row, so every request is a whole cache line (all threads of the workgroup);
// NT: non-temporal stores (see st4_nt).
template <class OT, int RL, int NTHR, bool NT>
__device__ __forceinline__ void store_rows_tiles(const lds_char* tile, OT* dst, size_t rs, int nvalid) {
    constexpr int EPC = 16 / (int)sizeof(OT);
    constexpr int NCH = RL / EPC;
#pragma unroll
    for (int i = 0; i < (CH * NCH + NTHR - 1) / NTHR; ++i) {
        const int u = (int)threadIdx.x + NTHR * i, row = u / NCH, pos = u % NCH;
        if ((CH * NCH % NTHR == 0 || u < CH * NCH) && row < nvalid) {
            const f32x4 x = lds_load<f32x4>(tile + u * 16);
            store_out<NT>((f32x4*)(dst + (size_t)row * rs + (pos ^ swz_f<OT, RL>(row)) * EPC), x);
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
