// Forward pass of the Gated Delta Rule-2 operator on gfx950.
//
// Operator ("Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention",
// anthology record LIT-802, takeaway 1; paper Sec. 3.1 Eqs. 8-10):
//   S_t = (I - k_t (b_t * k_t)^T) diag(exp g_t) S_{t-1} + k_t (w_t * v_t)^T,
//   o_t = S_t^T q_t (readout after the update).
// Chunkwise form (LIT-802 takeaway 2, App. A; digg thread post 9/: inside a
// chunk it is matrix products and a triangular solve, and only the state is
// carried between chunks). Per chunk of 64 tokens with start state S:
//   A = strict_lower(Kb Khat^T), M = lower(Qg Khat^T)   (decay folded into factors)
//   T = (I + A)^-1            one inverse shared by the erase and write sides
//   U = T (W*V),  Wm = T Kb,  Delta = U - Wm S
//   O = Qg S + M Delta,  S' = diag(exp gam_C) S + Kd^T Delta
// with Kb = b*k*exp(gam), Qg = q*exp(gam), Kd = k*exp(gam_C - gam).
//
// Kernels:
//   k_fwd_intra : one workgroup per chunk, fully parallel. Builds A and M on
//                 MFMA, inverts (I + A) in fp32 (16x16 diagonal blocks by
//                 substitution, off-diagonal blocks on fp32 MFMA), forms U and
//                 Wm on MFMA, and writes every per-chunk operand the two state
//                 chains need, already in MFMA fragment order.
//   k_fwd_chain : (gdr2_chain.hip) one wave per (sequence, 16-column slice of
//                 the value axis), walks the chunks in order with the state in
//                 accumulator registers.
#include "gdr2_intra_common.hpp"
#include "gdr2_kernels.hpp"

namespace gdr2 {

template <class OT, int DK, int DV>
struct FwdLds {
    static constexpr int LDK = DK + pad_ot<OT>();
    static constexpr int LDV = DV + pad_ot<OT>();
    static constexpr int LDC = CH + 4;             // fp32 [CH][CH]
    static constexpr int LDCO = CH + pad_ot<OT>();  // OT [CH][CH] and [DK][CH]
    static constexpr size_t XA = 0;
    static constexpr size_t XM = XA + sizeof(OT) * CH * LDK;
    static constexpr size_t Y = XM + sizeof(OT) * CH * LDK;
    static constexpr size_t X = Y + sizeof(OT) * CH * LDK;
    static constexpr size_t A = X + sizeof(OT) * CH * LDV;
    static constexpr size_t T = A + sizeof(float) * CH * LDC;
    static constexpr size_t M = T + sizeof(float) * CH * LDC;
    static constexpr size_t WT = M + sizeof(OT) * CH * LDCO;
    static constexpr size_t F = WT + sizeof(OT) * DK * LDCO;
    static constexpr size_t BYTES = F + sizeof(float) * F_ROWS * DK;
};

// Blocked inverse of the unit lower-triangular (I + A), A in sA (fp32), into sT.
// Diagonal 16x16 blocks by forward substitution (one wave, lane = block x column);
// then T_RI = -T_RR * sum_{K=I}^{R-1} A_RK T_KI on fp32 MFMA, one level at a time.
__device__ __forceinline__ void blocked_inverse(const float* sA, float* sT, int LDC) {
    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, li = l & 15, lq = l >> 4;
    if (wv == 0) {
        const int D = lq, j = li;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == j) ? 1.f : 0.f;
            const float* arow = sA + (16 * D + r) * LDC + 16 * D;
#pragma unroll
            for (int i = 0; i < r; ++i) acc -= arow[i] * x[i];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[(16 * D + r) * LDC + 16 * D + j] = x[r];
    }
    __syncthreads();
#pragma unroll
    for (int lev = 1; lev < NBLK; ++lev) {
        if (wv < NBLK - lev) {
            const int I = wv, R = wv + lev;
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            for (int K = I; K < R; ++K) {
                float a[4], b[4];
                ld4(sA + (16 * R + li) * LDC + 16 * K + 4 * lq, a);
#pragma unroll
                for (int e = 0; e < 4; ++e) b[e] = sT[(16 * K + 4 * lq + e) * LDC + 16 * I + li];
                mma_k16_f32(z, a, b);
            }
            float a[4], b[4] = {z[0], z[1], z[2], z[3]};
            ld4(sT + (16 * R + li) * LDC + 16 * R + 4 * lq, a);
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            mma_k16_f32(t, a, b);
#pragma unroll
            for (int i = 0; i < 4; ++i) sT[(16 * R + 4 * lq + i) * LDC + 16 * I + li] = -t[i];
        }
        __syncthreads();
    }
}

template <class OT, int DK, int DV, bool TRAIN>
__global__ __launch_bounds__(256) void k_fwd_intra(Args a) {
    using LS = FwdLds<OT, DK, DV>;
    using FT = typename Frag<OT>::type;
    constexpr int LDK = LS::LDK, LDV = LS::LDV, LDC = LS::LDC, LDCO = LS::LDCO;
    constexpr int KB = DK / 32;
    extern __shared__ __align__(16) char smem[];
    OT* sXA = (OT*)(smem + LS::XA);
    OT* sXM = (OT*)(smem + LS::XM);
    OT* sY = (OT*)(smem + LS::Y);
    OT* sX = (OT*)(smem + LS::X);
    float* sA = (float*)(smem + LS::A);
    float* sT = (float*)(smem + LS::T);
    OT* sM = (OT*)(smem + LS::M);
    OT* sWt = (OT*)(smem + LS::WT);
    float* sF = (float*)(smem + LS::F);

    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, li = l & 15, lq = l >> 4;
    const long long cid = blockIdx.x;
    const int s = (int)(cid / a.NT), c = (int)(cid % a.NT);
    const int bidx = s / a.H, h = s % a.H;
    const int t0 = c * CH;
    const int nvalid = min(CH, a.T - t0);
    const size_t rowk0 = ((size_t)bidx * a.T + t0) * a.H + h;  // token-row index of row 0
    const Layout& L = a.L;
    char* ws = a.ws;

    // ---- phase 1: cumulative decay, factors, X = w*v
    float gam[DK / 64][4][4];
    chunk_factors<OT, DK>((const OT*)a.g + rowk0 * DK, (const OT*)a.q + rowk0 * DK, (const OT*)a.k + rowk0 * DK,
                          (const OT*)a.b + rowk0 * DK, (size_t)a.H * DK, nvalid, gam, sXA, sXM, sY, LDK, sF,
                          (float*)(ws + L.o_gc) + cid * L.gc);
    chunk_x<OT, DV>((const OT*)a.v + rowk0 * DV, (const OT*)a.w + rowk0 * DV, (size_t)a.H * DV, nvalid, sX, LDV);
    // zero the upper blocks of M and T
    for (int idx = tid; idx < CH * CH; idx += 256) {
        const int r = idx / CH, cc = idx % CH;
        if ((cc >> 4) > (r >> 4)) {
            sM[r * LDCO + cc] = to_ot<OT>(0.f);
            sT[r * LDC + cc] = 0.f;
        }
    }
    __syncthreads();

    // ---- phase 2: A (strictly lower) and M (lower) per 16x16 block pair
    for (int p = wv; p < 2 * NPAIR; p += 4) {
        const bool isM = p >= NPAIR;
        const int pp = isM ? p - NPAIR : p;
        int R, I;
        pair_ri(pp, R, I);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            FT af = frag_rowk_scaled<OT, OT>(isM ? sXM : sXA, LDK, 16 * R, 32 * kb, sF + (F_S + pp) * DK);
            FT bf = frag_rowk<OT>(sY, LDK, 16 * I, 32 * kb);
            mma(acc, af, bf);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * R + 4 * lq + i, col = 16 * I + li;
            float v = acc[i];
            if (R == I && (isM ? (col > row) : (col >= row))) v = 0.f;
            if (isM)
                sM[row * LDCO + col] = to_ot<OT>(v);
            else
                sA[row * LDC + col] = v;
        }
    }
    __syncthreads();

    // ---- phase 3: T = (I + A)^-1
    blocked_inverse(sA, sT, LDC);

    // ---- phase 4: U = T X (tiles) and Wm^T = Kb^T T^T (-> A fragments of Wm)
    {
        const int tt = wv;  // time tile of U rows / Wm rows
        FT aT[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) aT[kb] = frag_rowk_f32<OT>(sT, LDC, 16 * tt, 32 * kb);
        const int nkb = tt / 2 + 1;  // T is lower triangular
        OT* u = (OT*)(ws + L.o_u) + cid * L.u;
        for (int j = 0; j < DV / 16; ++j) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int kb = 0; kb < nkb; ++kb) mma(acc, aT[kb], frag_colk<OT, OT>(sX, LDV, 16 * j, 32 * kb));
            store_tile<OT>(u + (j * 4 + tt) * 256, acc);
        }
        OT* wm = (OT*)(ws + L.o_wmA) + cid * L.wmA;
        for (int kb2 = 0; kb2 < KB; ++kb2) {
            f32x4 wt[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int at = 2 * kb2 + h2;  // key-channel tile
                const int col = 16 * at + li;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int kb = 0; kb < nkb; ++kb) {
                    FT ak = frag_colk<OT, OT>(sXA, LDK, 16 * at, 32 * kb, sF[(F_ER0 + 2 * kb) * DK + col],
                                              sF[(F_ER0 + 2 * kb + 1) * DK + col]);
                    mma(acc, ak, aT[kb]);
                }
                wt[h2] = acc;
                if (TRAIN) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) sWt[(16 * at + 4 * lq + i) * LDCO + 16 * tt + li] = to_ot<OT>(acc[i]);
                }
            }
            store_frag<OT>(wm + (tt * KB + kb2) * 512, frag_of<OT>(wt[0], wt[1]));
        }
    }
    __syncthreads();

    // ---- phase 5: operand fragments for the state chains
    {
        OT* kdA = (OT*)(ws + L.o_kdA) + cid * L.kdA;
        OT* qgB = (OT*)(ws + L.o_qgB) + cid * L.qgB;
        OT* mB = (OT*)(ws + L.o_mB) + cid * L.mB;
        constexpr int N_KDA = (DK / 16) * 2, N_QGB = 4 * KB, N_MB = 8;
        constexpr int N_FWD = N_KDA + N_QGB + N_MB;
        constexpr int N_MTA = 8, N_KDRA = 4 * KB, N_QGTA = (DK / 16) * 2, N_WMTA = (DK / 16) * 2, N_TTA = 8;
        constexpr int N_ALL = N_FWD + (TRAIN ? N_MTA + N_KDRA + N_QGTA + N_WMTA + N_TTA : 0);
        for (int f = wv; f < N_ALL; f += 4) {
            int x = f;
            if (x < N_KDA) {  // A fragments of Kd^T: rows = key channel, K = time
                const int mt = x / 2, kb = x % 2, col = 16 * mt + li;
                store_frag<OT>(kdA + x * 512, frag_colk<OT, OT>(sY, LDK, 16 * mt, 32 * kb, sF[(F_ECE + 2 * kb) * DK + col],
                                                                sF[(F_ECE + 2 * kb + 1) * DK + col]));
                continue;
            }
            x -= N_KDA;
            if (x < N_QGB) {  // B fragments of Qg^T: K = key channel, N = time
                const int nt = x / KB, kb = x % KB;
                store_frag<OT>(qgB + x * 512, frag_rowk_scaled<OT, OT>(sXM, LDK, 16 * nt, 32 * kb, sF + (F_ER0 + nt) * DK));
                continue;
            }
            x -= N_QGB;
            if (x < N_MB) {  // B fragments of M^T: K = source token i, N = target token r
                const int nt = x / 2, kb = x % 2;
                store_frag<OT>(mB + x * 512, frag_rowk<OT>(sM, LDCO, 16 * nt, 32 * kb));
                continue;
            }
            x -= N_MB;
            if (!TRAIN) continue;
            if (x < N_MTA) {  // A fragments of M^T
                const int mt = x / 2, kb = x % 2;
                store_frag<OT>((OT*)(ws + L.o_mtA) + cid * L.mtA + x * 512, frag_colk<OT, OT>(sM, LDCO, 16 * mt, 32 * kb));
                continue;
            }
            x -= N_MTA;
            if (x < N_KDRA) {  // A fragments of Kd: rows = time, K = key channel
                const int mt = x / KB, kb = x % KB;
                store_frag<OT>((OT*)(ws + L.o_kdRA) + cid * L.kdRA + x * 512,
                               frag_rowk_scaled<OT, OT>(sY, LDK, 16 * mt, 32 * kb, sF + (F_ECE + mt) * DK));
                continue;
            }
            x -= N_KDRA;
            if (x < N_QGTA) {  // A fragments of Qg^T: rows = key channel, K = time
                const int mt = x / 2, kb = x % 2, col = 16 * mt + li;
                store_frag<OT>((OT*)(ws + L.o_qgtA) + cid * L.qgtA + x * 512,
                               frag_colk<OT, OT>(sXM, LDK, 16 * mt, 32 * kb, sF[(F_ER0 + 2 * kb) * DK + col],
                                                 sF[(F_ER0 + 2 * kb + 1) * DK + col]));
                continue;
            }
            x -= N_QGTA;
            if (x < N_WMTA) {  // A fragments of Wm^T: rows = key channel, K = time
                const int mt = x / 2, kb = x % 2;
                store_frag<OT>((OT*)(ws + L.o_wmtA) + cid * L.wmtA + x * 512, frag_rowk<OT>(sWt, LDCO, 16 * mt, 32 * kb));
                continue;
            }
            x -= N_WMTA;
            {  // A fragments of T^T: rows = source token i, K = target token r
                const int mt = x / 2, kb = x % 2;
                store_frag<OT>((OT*)(ws + L.o_ttA) + cid * L.ttA + x * 512, frag_colk<OT, float>(sT, LDC, 16 * mt, 32 * kb));
            }
        }
    }
}

size_t fwd_intra_lds_bytes(int DK, int DV, int esz) {
#define GDR2_LDS(OT_, DK_, DV_) \
    if (DK == DK_ && DV == DV_ && esz == (int)sizeof(OT_)) return FwdLds<OT_, DK_, DV_>::BYTES;
    GDR2_LDS(bf16, 64, 64) GDR2_LDS(bf16, 64, 128) GDR2_LDS(bf16, 128, 64) GDR2_LDS(bf16, 128, 128)
    GDR2_LDS(float, 64, 64)
#undef GDR2_LDS
    return 0;
}

template <class OT, int DK, int DV>
static hipError_t launch_fwd_t(const Args& a, bool train, hipStream_t stream) {
    const size_t lds = FwdLds<OT, DK, DV>::BYTES;
    auto intra = train ? k_fwd_intra<OT, DK, DV, true> : k_fwd_intra<OT, DK, DV, false>;
    hipError_t e = hipFuncSetAttribute((const void*)intra, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if ((e = mark(a, 0, stream)) != hipSuccess) return e;
    hipLaunchKernelGGL(intra, dim3((unsigned)a.NC), dim3(256), lds, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = mark(a, 1, stream)) != hipSuccess) return e;
    if ((e = launch_fwd_chain_t<OT, DK, DV>(a, train, stream)) != hipSuccess) return e;
    return mark(a, 2, stream);
}

hipError_t launch_fwd(const Args& a, bool bf16_, bool train, hipStream_t stream) {
    const int DK = a.L.DK, DV = a.L.DV;
    if (bf16_) {
        if (DK == 64 && DV == 64) return launch_fwd_t<bf16, 64, 64>(a, train, stream);
        if (DK == 64 && DV == 128) return launch_fwd_t<bf16, 64, 128>(a, train, stream);
        if (DK == 128 && DV == 64) return launch_fwd_t<bf16, 128, 64>(a, train, stream);
        if (DK == 128 && DV == 128) return launch_fwd_t<bf16, 128, 128>(a, train, stream);
    } else {
        if (DK == 64 && DV == 64) return launch_fwd_t<float, 64, 64>(a, train, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr2
