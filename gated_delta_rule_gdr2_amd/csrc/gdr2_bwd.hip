// Backward pass of the Gated Delta Rule-2 operator on gfx950 ("gate-aware"
// backward: anthology record LIT-802, takeaway 2, paper App. B; digg thread
// post 11/ -- the per-channel gates sit inside the channel sums that
// accumulate dA and cannot be pulled out as KDA's scalar beta can).
//
// Differentiating the chunk equations (see the forward file) gives, per chunk
// with start state S, end-state gradient dS' and output gradient dO:
//   reverse chain : dDelta = M^T dO + Kd dS',  dY = T^T dDelta,
//                   dS = diag(exp gam_C) dS' + Qg^T dO - Wm^T dDelta
//   intra chunk   : dM = lower(dO Delta^T), dA = -strict_lower(dY Delta^T),
//                   dQg = dO S^T, dKb = -dY S^T, dKd = Delta dS'^T,
//                   dX = dY (dv = dY*w, dw = dY*v),
//                   plus the back-propagation of the two decay-scaled bilinear
//                   forms A = (b*k, k) and M = (q, k) with the gates inside.
// The log-decay gradient follows elementwise: gam enters only through the
// factors of q, b*k and k, so dgam = q*dq + 2*b*db - k*dk on every row, plus
// at the chunk's last row the scaling of the carried state,
// sum_r dKd*Kd + exp(gam_C) * rowsum(dS' * S); dg is its reverse running sum.
//
// Kernels:
//   k_bwd_chain : (gdr2_chain.hip) one wave per (sequence, 16-column value
//                 slice), chunks in reverse; state gradient in accumulator
//                 registers; writes dS' (row-major) and dY (tiles) per chunk.
//   k_bwd_intra : one workgroup per chunk, fully parallel; reads the saved S,
//                 Delta, dS', dY and the inputs, writes dq, dk, dv, dg, db, dw.
#include "gdr2_intra_common.hpp"
#include "gdr2_kernels.hpp"

namespace gdr2 {

template <class OT, int DK, int DV>
struct BwdLds {
    static constexpr int LDK = DK + pad_ot<OT>();
    static constexpr int LDV = DV + pad_ot<OT>();
    static constexpr int LDCO = CH + pad_ot<OT>();
    static constexpr size_t XA = 0;
    static constexpr size_t XM = XA + sizeof(OT) * CH * LDK;
    static constexpr size_t Y = XM + sizeof(OT) * CH * LDK;
    static constexpr size_t DO = Y + sizeof(OT) * CH * LDK;
    static constexpr size_t DL = DO + sizeof(OT) * CH * LDV;
    static constexpr size_t DY = DL + sizeof(OT) * CH * LDV;
    static constexpr size_t DA = DY + sizeof(OT) * CH * LDV;
    static constexpr size_t DM = DA + sizeof(OT) * CH * LDCO;
    static constexpr size_t F = DM + sizeof(OT) * CH * LDCO;
    static constexpr size_t DMD = F + sizeof(float) * F_ROWS * DK;  // diagonal of dM, fp32
    static constexpr size_t BYTES = DMD + sizeof(float) * CH;
};

// tile dump [DV/16][4][64 lanes][4] -> row-major LDS [CH][ld]
template <class OT, int DV>
__device__ __forceinline__ void undump_tiles(const OT* src, OT* dst, int ld) {
    for (int e = threadIdx.x; e < (DV / 16) * 4 * 64; e += 256) {
        const int lane = e & 63, t = (e >> 6) & 3, jj = e >> 8;
        float v[4];
        ld4(src + (size_t)e * 4, v);
        const int row = 16 * t + 4 * (lane >> 4), col = 16 * jj + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(row + i) * ld + col] = to_ot<OT>(v[i]);
    }
}

template <class OT, int DK, int DV>
__global__ __launch_bounds__(256) void k_bwd_intra(Args a) {
    using LS = BwdLds<OT, DK, DV>;
    using FT = typename Frag<OT>::type;
    constexpr int LDK = LS::LDK, LDV = LS::LDV, LDCO = LS::LDCO;
    constexpr int KV = DV / 32, CPW = DK / 64, VPW = DV / 64;
    extern __shared__ __align__(16) char smem[];
    OT* sXA = (OT*)(smem + LS::XA);
    OT* sXM = (OT*)(smem + LS::XM);
    OT* sY = (OT*)(smem + LS::Y);
    OT* sDO = (OT*)(smem + LS::DO);
    OT* sDL = (OT*)(smem + LS::DL);
    OT* sDY = (OT*)(smem + LS::DY);
    OT* sDA = (OT*)(smem + LS::DA);
    OT* sDM = (OT*)(smem + LS::DM);
    float* sF = (float*)(smem + LS::F);
    float* sDMd = (float*)(smem + LS::DMD);

    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, li = l & 15, lq = l >> 4;
    const long long cid = blockIdx.x;
    const int s = (int)(cid / a.NT), c = (int)(cid % a.NT);
    const int bidx = s / a.H, h = s % a.H;
    const int t0 = c * CH;
    const int nvalid = min(CH, a.T - t0);
    const size_t rowk0 = ((size_t)bidx * a.T + t0) * a.H + h;
    const size_t rsk = (size_t)a.H * DK, rsv = (size_t)a.H * DV;
    const Layout& L = a.L;
    char* ws = a.ws;
    const OT* qb = (const OT*)a.q + rowk0 * DK;
    const OT* kb_ = (const OT*)a.k + rowk0 * DK;
    const OT* bb = (const OT*)a.b + rowk0 * DK;

    // ---- phase 1: factors, dO, Delta, dY into LDS
    float gam[CPW][4][4];
    chunk_factors<OT, DK>((const OT*)a.g + rowk0 * DK, qb, kb_, bb, rsk, nvalid, gam, sXA, sXM, sY, LDK, sF, nullptr);
    {
        const OT* dob = (const OT*)a.dout + rowk0 * DV;
#pragma unroll
        for (int jc = 0; jc < VPW; ++jc) {
            const int ch0 = 16 * (wv * VPW + jc) + 4 * lq;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = 16 * t + li;
                float x[4];
                ld4_row(dob, rsv, r, ch0, nvalid, x);
                st4(sDO + r * LDV + ch0, x);
            }
        }
    }
    undump_tiles<OT, DV>((const OT*)(ws + L.o_delta) + cid * L.delta, sDL, LDV);
    undump_tiles<OT, DV>((const OT*)(ws + L.o_dy) + cid * L.dy, sDY, LDV);
    for (int idx = tid; idx < CH * CH; idx += 256) {  // zero the upper blocks of dA, dM
        const int r = idx / CH, cc = idx % CH;
        if ((cc >> 4) > (r >> 4)) {
            sDA[r * LDCO + cc] = to_ot<OT>(0.f);
            sDM[r * LDCO + cc] = to_ot<OT>(0.f);
        }
    }
    __syncthreads();

    // ---- phase 2: dA = -strict_lower(dY Delta^T), dM = lower(dO Delta^T)
    // The diagonal of M, q_r . k_r, does not depend on the decay; its gradient is
    // kept apart in fp32 (sDMd) so that its query-side and key-side terms cancel
    // exactly in the log-decay gradient instead of up to bf16 rounding.
    for (int p = wv; p < 2 * NPAIR; p += 4) {
        const bool isM = p >= NPAIR;
        int R, I;
        pair_ri(isM ? p - NPAIR : p, R, I);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KV; ++kb)
            mma(acc, frag_rowk<OT>(isM ? sDO : sDY, LDV, 16 * R, 32 * kb), frag_rowk<OT>(sDL, LDV, 16 * I, 32 * kb));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * R + 4 * lq + i, col = 16 * I + li;
            float v = isM ? acc[i] : -acc[i];
            if (isM && col == row) sDMd[row] = v;
            if (R == I && col >= row) v = 0.f;  // dA strictly lower; dM diagonal kept in sDMd
            (isM ? sDM : sDA)[row * LDCO + col] = to_ot<OT>(v);
        }
    }
    __syncthreads();

    // ---- phases 3+4, one key-channel tile at a time: products, then elementwise finals
    const OT* Sg = (const OT*)(ws + L.o_s) + cid * L.s;
    const OT* dSg = (const OT*)(ws + L.o_ds) + cid * L.ds;
#pragma unroll 1
    for (int ac = 0; ac < CPW; ++ac) {
        const int at = wv * CPW + ac;
        const int mcol = 16 * at + li;  // key channel held as operand row by this lane
        FT Sf[KV], dSf[KV];
        float pr = 0.f;
#pragma unroll
        for (int kb = 0; kb < KV; ++kb) {
            Sf[kb] = frag_rowk<OT>(Sg, DV, 16 * at, 32 * kb);
            dSf[kb] = frag_rowk<OT>(dSg, DV, 16 * at, 32 * kb);
#pragma unroll
            for (int e = 0; e < 8; ++e) pr += to_f(Sf[kb][e]) * to_f(dSf[kb][e]);
        }
        pr += __shfl_xor(pr, 16, 64);
        pr += __shfl_xor(pr, 32, 64);  // rowsum(dS' * S) for key channel mcol, in every lane li

        f32x4 dQg[4], dKb[4], dKd[4], xA[4], xM[4], yA[4], yM[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            dQg[t] = z; dKb[t] = z; dKd[t] = z; xA[t] = z; xM[t] = z; yA[t] = z; yM[t] = z;
#pragma unroll
            for (int kb = 0; kb < KV; ++kb) {
                mma(dQg[t], Sf[kb], frag_rowk<OT>(sDO, LDV, 16 * t, 32 * kb));
                mma(dKb[t], Sf[kb], frag_rowk<OT>(sDY, LDV, 16 * t, 32 * kb));  // (dY S^T)^T
                mma(dKd[t], dSf[kb], frag_rowk<OT>(sDL, LDV, 16 * t, 32 * kb));
            }
        }
        // bilinear back-propagation, transposed: rows = key channel, columns = token
#pragma unroll
        for (int R = 0; R < 4; ++R) {  // Xbar (erase/query side) for target block R
            for (int kb = 0; kb <= R / 2; ++kb) {
                const int I0 = 2 * kb, I1 = 2 * kb + 1;
                const float r0 = sF[(F_S + pair_id(R, I0)) * DK + mcol];
                const float r1 = I1 <= R ? sF[(F_S + pair_id(R, I1)) * DK + mcol] : 0.f;
                FT ay = frag_colk<OT, OT>(sY, LDK, 16 * at, 32 * kb, r0, r1);
                mma(xA[R], ay, frag_rowk<OT>(sDA, LDCO, 16 * R, 32 * kb));
                mma(xM[R], ay, frag_rowk<OT>(sDM, LDCO, 16 * R, 32 * kb));
            }
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {  // Ybar (key side) for source block I
            for (int kb = I / 2; kb < 2; ++kb) {
                const int R0 = 2 * kb, R1 = 2 * kb + 1;
                const float r0 = R0 >= I ? sF[(F_S + pair_id(R0, I)) * DK + mcol] : 0.f;
                const float r1 = R1 >= I ? sF[(F_S + pair_id(R1, I)) * DK + mcol] : 0.f;
                FT bA = frag_colk<OT, OT>(sDA, LDCO, 16 * I, 32 * kb);
                FT bM = frag_colk<OT, OT>(sDM, LDCO, 16 * I, 32 * kb);
                mma(yA[I], frag_colk<OT, OT>(sXA, LDK, 16 * at, 32 * kb, r0, r1), bA);
                mma(yM[I], frag_colk<OT, OT>(sXM, LDK, 16 * at, 32 * kb, r0, r1), bM);
            }
        }

        // ---- finals at (key channel 16at + 4lq + i, token 16t + li)
        const int ch0 = 16 * at + 4 * lq;
        float g0[4][4], ge[4][4];
#pragma unroll
        for (int R = 0; R < 4; ++R)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                g0[R][i] = row_bcast(gam[ac][R][i], 0);
                ge[R][i] = row_bcast(gam[ac][R][i], 15);
            }
        float kdsum[4] = {0.f, 0.f, 0.f, 0.f};
        float dgam[4][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = 16 * t + li;
            const bool ok = r < nvalid;
            float qv[4], kv[4], bv[4], dq[4], dk[4], db[4];
            ld4_row(qb, rsk, r, ch0, nvalid, qv);
            ld4_row(kb_, rsk, r, ch0, nvalid, kv);
            ld4_row(bb, rsk, r, ch0, nvalid, bv);
            const float dmd = sDMd[r];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float gm = gam[ac][t][i];
                const float e1 = __expf(gm - g0[t][i]);
                const float e2 = __expf(ge[t][i] - gm);
                const float G = __expf(gm);             // exp(gam_r)
                const float Gd = __expf(ge[3][i] - gm);  // exp(gam_C - gam_r)
                const float gq = dQg[t][i] * G + e1 * xM[t][i] + dmd * kv[i];
                const float gbk = e1 * xA[t][i] - dKb[t][i] * G;  // dKb holds +dY S^T
                const float gk = dKd[t][i] * Gd + e2 * (yA[t][i] + yM[t][i]) + dmd * qv[i];
                dq[i] = gq;
                db[i] = gbk * kv[i];
                dk[i] = gbk * bv[i] + gk;
                dgam[t][i] = qv[i] * dq[i] + 2.f * bv[i] * db[i] - kv[i] * dk[i];
                kdsum[i] += dKd[t][i] * kv[i] * Gd;
            }
            if (ok) {
                const size_t off = (size_t)r * rsk + ch0;
                st4((OT*)a.dq + rowk0 * DK + off, dq);
                st4((OT*)a.dk + rowk0 * DK + off, dk);
                st4((OT*)a.db + rowk0 * DK + off, db);
            }
        }
        // carried-state scaling at the chunk's last row, then the reverse running sum
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float rsumS = __shfl(pr, (l & 48) | (4 * lq + i), 64);  // rowsum for channel ch0 + i
            const float extra = row_sum16(kdsum[i]) + __expf(ge[3][i]) * rsumS;
            if (li == 15) dgam[3][i] += extra;
        }
        float tot[4] = {0.f, 0.f, 0.f, 0.f}, pre[4][4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = row_scan16(dgam[t][i]) + tot[i];
                pre[t][i] = x;
                tot[i] = row_bcast(x, 15);
            }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = 16 * t + li;
            if (r < nvalid) {
                float dg[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) dg[i] = tot[i] - pre[t][i] + dgam[t][i];
                st4((OT*)a.dg + rowk0 * DK + (size_t)r * rsk + ch0, dg);
            }
        }
    }

    // ---- dv = dY * w, dw = dY * v
    {
        const OT* vb = (const OT*)a.v + rowk0 * DV;
        const OT* wb = (const OT*)a.w + rowk0 * DV;
#pragma unroll
        for (int jc = 0; jc < VPW; ++jc) {
            const int ch0 = 16 * (wv * VPW + jc) + 4 * lq;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = 16 * t + li;
                float dy[4], vv[4], ww[4], dvv[4], dww[4];
                ld4(sDY + r * LDV + ch0, dy);
                ld4_row(vb, rsv, r, ch0, nvalid, vv);
                ld4_row(wb, rsv, r, ch0, nvalid, ww);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dvv[i] = dy[i] * ww[i];
                    dww[i] = dy[i] * vv[i];
                }
                if (r < nvalid) {
                    st4((OT*)a.dv + rowk0 * DV + (size_t)r * rsv + ch0, dvv);
                    st4((OT*)a.dw + rowk0 * DV + (size_t)r * rsv + ch0, dww);
                }
            }
        }
    }
}

size_t bwd_intra_lds_bytes(int DK, int DV, int esz) {
#define GDR2_LDS(OT_, DK_, DV_) \
    if (DK == DK_ && DV == DV_ && esz == (int)sizeof(OT_)) return BwdLds<OT_, DK_, DV_>::BYTES;
    GDR2_LDS(bf16, 64, 64) GDR2_LDS(bf16, 64, 128) GDR2_LDS(bf16, 128, 64) GDR2_LDS(bf16, 128, 128)
    GDR2_LDS(float, 64, 64)
#undef GDR2_LDS
    return 0;
}

template <class OT, int DK, int DV>
static hipError_t launch_bwd_t(const Args& a, hipStream_t stream) {
    const size_t lds = BwdLds<OT, DK, DV>::BYTES;
    auto intra = k_bwd_intra<OT, DK, DV>;
    hipError_t e = hipFuncSetAttribute((const void*)intra, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if ((e = mark(a, 0, stream)) != hipSuccess) return e;
    if ((e = launch_bwd_chain_t<OT, DK, DV>(a, stream)) != hipSuccess) return e;
    if ((e = mark(a, 1, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL(intra, dim3((unsigned)a.NC), dim3(256), lds, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return mark(a, 2, stream);
}

hipError_t launch_bwd(const Args& a, bool bf16_, hipStream_t stream) {
    const int DK = a.L.DK, DV = a.L.DV;
    if (bf16_) {
        if (DK == 64 && DV == 64) return launch_bwd_t<bf16, 64, 64>(a, stream);
        if (DK == 64 && DV == 128) return launch_bwd_t<bf16, 64, 128>(a, stream);
        if (DK == 128 && DV == 64) return launch_bwd_t<bf16, 128, 64>(a, stream);
        if (DK == 128 && DV == 128) return launch_bwd_t<bf16, 128, 128>(a, stream);
    } else {
        if (DK == 64 && DV == 64) return launch_bwd_t<float, 64, 64>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr2
