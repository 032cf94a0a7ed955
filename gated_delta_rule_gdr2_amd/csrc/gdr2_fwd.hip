// Forward pass of the Gated Delta Rule-2 operator on gfx950: the intra-chunk kernel.
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
// k_fwd_intra: one workgroup (4 waves) per chunk, fully parallel. It builds A
// and M on MFMA from the block-split factors, inverts (I + A) in fp32 (16x16
// diagonal blocks by substitution from registers, off-diagonal blocks on fp32
// MFMA), forms U and Wm on MFMA, and writes the per-chunk operands of the two
// state chains (gdr2_chain.hip): Wm, Kd, Qg, M and (training) T as swizzled
// tiles, U as accumulator tiles, exp(gam_C). Phases reuse LDS (A over the
// query factors, T over the key factors once each is dead) so that two
// workgroups fit on one compute unit. With gates passed as logits (ACT) the gates are
// activated in phase 1, as they are converted to fp32; nothing else changes.
#include <type_traits>

#include "gdr2_intra_common.hpp"
#include "gdr2_kernels.hpp"

namespace gdr2 {

template <class OT, int DK, int DV>
struct FwdLds {  // all matrices are swizzled tiles (see swz())
    static constexpr int ES = sizeof(OT);
    static constexpr int KMAT = CH * DK * ES;
    static constexpr int CMAT = CH * CH * 4;  // fp32 [CH][CH]
    static constexpr int SLOT = KMAT > CMAT ? KMAT : CMAT;
    static constexpr int XA = 0;
    static constexpr int SLOTM = XA + KMAT;     // XM, later A
    static constexpr int SLOTY = SLOTM + SLOT;  // Y, later T
    static constexpr int X = SLOTY + SLOT;
    static constexpr int F = X + CH * DV * ES;
    static constexpr int FLAG = F + F_ROWS * DK * 4;  // one int per wave: strong decay seen
    static constexpr int BYTES = FLAG + 16;
    // slow-path scratch: exp(g) of one block's rows [16][DK] fp32 over F, b*k [16][DK] fp32
    // then q, k [16][DK] in the operand type over the Y/T slot (both dead then)
    static_assert(16 * DK * 4 <= F_ROWS * DK * 4, "slow-path decay rows fit in the factor area");
    static_assert(16 * DK * 4 + 2 * 16 * DK * ES <= SLOT, "slow-path rows fit in the Y/T slot");
};

// Blocked inverse of the unit lower-triangular (I + A), A in sA (fp32), into sT.
// Diagonal 16x16 blocks by forward substitution (one wave, lane = block x column,
// the block's rows read into registers first); then
// T_RI = -T_RR * sum_{K=I}^{R-1} A_RK T_KI on fp32 MFMA, one level at a time.
__device__ __forceinline__ void blocked_inverse(const lds_char* sA, lds_char* sT) {
    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, li = l & 15, lq = l >> 4;
    auto A = [&](int r, int c) { return sA + swz<float, CH>(r, c) * 4; };
    auto Tp = [&](int r, int c) { return sT + swz<float, CH>(r, c) * 4; };
    if (wv == 0) {
        const int D = lq, j = li;
        float arow[16][16];
#pragma unroll
        for (int r = 1; r < 16; ++r)
#pragma unroll
            for (int c4 = 0; c4 < r; c4 += 4) lds_get4<float>(A(16 * D + r, 16 * D + c4), &arow[r][c4]);
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) acc -= arow[r][i] * x[i];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) lds_store<float>(Tp(16 * D + r, 16 * D + j), x[r]);
    }
    sync_lds();
#pragma unroll
    for (int lev = 1; lev < NBLK; ++lev) {
        if (wv < NBLK - lev) {
            const int I = wv, R = wv + lev;
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            for (int K = I; K < R; ++K) {
                float a4[4], b4[4];
                lds_get4<float>(A(16 * R + li, 16 * K + 4 * lq), a4);
#pragma unroll
                for (int e = 0; e < 4; ++e) b4[e] = lds_load<float>(Tp(16 * K + 4 * lq + e, 16 * I + li));
                mma_k16_f32(z, a4, b4);
            }
            float a4[4], b4[4] = {z[0], z[1], z[2], z[3]};
            lds_get4<float>(Tp(16 * R + li, 16 * R + 4 * lq), a4);
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            mma_k16_f32(t, a4, b4);
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_store<float>(Tp(16 * R + 4 * lq + i, 16 * I + li), -t[i]);
        }
        sync_lds();
    }
}

// Slow path for strong decay: the four diagonal 16x16 blocks of A and M from per-element
// factors exp(gam_r - gam_i) = product of alpha_t = exp(g_t) over t in (i, r] (each <= 1,
// so nothing overflows, and no running sums are subtracted), exact for any decay,
// instead of the block-split factors whose s(R, R) overflows. Block by block, the block's
// rows are staged -- alpha in fp32 (sD), b*k in fp32 and q, k in the operand type (sS)
// -- and thread (r, i) of the block's 16 x 16 entries sums over the key channels
//   A[r][i] = sum_c (b k)_{r,c} k_{i,c} prod_{t in (i, r]} alpha_{t,c}   (i < r, else 0)
//   M[r][i] = sum_c q_{r,c} k_{i,c} prod_{t in (i, r]} alpha_{t,c}       (i <= r, else 0)
// in a fixed channel order (staggered by i so that the 16 lanes of a row group read
// different LDS banks). A goes to its fp32 LDS tile, M to the workspace.
template <class OT, int DK, bool ACT>
__device__ __forceinline__ void fwd_diag_exact(const Args& a, size_t rowk0, int nvalid, lds_char* sD, lds_char* sS,
                                               lds_char* sA, OT* m_out) {
    const int tid = threadIdx.x;
    const size_t rsk = (size_t)a.H * DK;
    const OT* gp = (const OT*)a.g + rowk0 * DK;
    const OT* qp = (const OT*)a.q + rowk0 * DK;
    const OT* kp = (const OT*)a.k + rowk0 * DK;
    const OT* bp = (const OT*)a.b + rowk0 * DK;
    lds_char* sBK = sS;                      // [16][DK] fp32
    lds_char* sQ = sS + 16 * DK * 4;         // [16][DK] OT
    lds_char* sK = sQ + 16 * DK * sizeof(OT);
    const int r = tid >> 4, i = tid & 15;
#pragma unroll 1
    for (int R = 0; R < NBLK; ++R) {
#pragma unroll 1
        for (int e = tid; e < 16 * DK; e += 256) {
            const int rr = e / DK, c = e % DK, row = 16 * R + rr;
            const bool ok = row < nvalid;  // padding rows: g = 0 (alpha = 1), q = k = b = 0
            const size_t off = (size_t)row * rsk + c;
            float gv = ok ? to_f(gp[off]) : 0.f;
            if (ACT && ok) gv = gate_act<OT, GATE_G>(gv, a.g_scale, a.b_scale);
            const float kv = ok ? to_f(kp[off]) : 0.f, qv = ok ? to_f(qp[off]) : 0.f;
            float bv = ok ? to_f(bp[off]) : 0.f;
            if (ACT && ok) bv = gate_act<OT, GATE_B>(bv, a.g_scale, a.b_scale);
            lds_store<float>(sD + e * 4, exp_op<OT>(gv));
            lds_store<float>(sBK + e * 4, bv * kv);
            lds_store<OT>(sQ + e * sizeof(OT), to_ot<OT>(qv));
            lds_store<OT>(sK + e * sizeof(OT), to_ot<OT>(kv));
        }
        sync_lds();
        float am = 0.f, mm = 0.f;
        if (i <= r) {
#pragma unroll 1
            for (int cc = 0; cc < DK; cc += 4) {
                const int c = (cc + 4 * i) & (DK - 1);
                float pr[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll 1
                for (int t = i + 1; t <= r; ++t) {
                    float al[4];
                    lds_get4<float>(sD + (t * DK + c) * 4, al);
#pragma unroll
                    for (int u = 0; u < 4; ++u) pr[u] *= al[u];
                }
                float bk[4], qr[4], ki[4];
                lds_get4<float>(sBK + (r * DK + c) * 4, bk);
                lds_get4<OT>(sQ + (r * DK + c) * sizeof(OT), qr);
                lds_get4<OT>(sK + (i * DK + c) * sizeof(OT), ki);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float ke = ki[u] * pr[u];
                    am = fmaf(bk[u], ke, am);
                    mm = fmaf(qr[u], ke, mm);
                }
            }
        }
        lds_store<float>(sA + swz<float, CH>(16 * R + r, 16 * R + i) * 4, i < r ? am : 0.f);
        m_out[fimg<OT, CH>(16 * R + r, 16 * R + i)] = to_ot<OT>(i <= r ? mm : 0.f);
        sync_lds();
    }
}

// upper 16x16 block (R, I), I > R, number u = 0..5
__device__ __forceinline__ void upper_ri(int u, int& R, int& I) {
    R = u < 3 ? 0 : (u < 5 ? 1 : 2);
    I = u < 3 ? u + 1 : (u < 5 ? u - 1 : 3);
}

template <class OT, int DK, int DV, bool TRAIN, bool ACT, bool NT>
__global__ __launch_bounds__(256, 2) void k_fwd_intra(Args a) {
    using LS = FwdLds<OT, DK, DV>;
    using FT = typename Frag<OT>::type;
    constexpr int KB = DK / 32;
    extern __shared__ __align__(16) char smem_[];
    lds_char* smem = (lds_char*)smem_;
    poison_lds(smem, LS::BYTES);
    poison_lds_done();
    lds_char* sXA = smem + LS::XA;
    lds_char* sXM = smem + LS::SLOTM;
    lds_char* sA = smem + LS::SLOTM;
    lds_char* sY = smem + LS::SLOTY;
    lds_char* sT = smem + LS::SLOTY;
    lds_char* sX = smem + LS::X;
    lds_char* sF = smem + LS::F;

    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, li = l & 15, lq = l >> 4;
    const long long cid = blockIdx.x;
    const int s = (int)(cid / a.NT), c = (int)(cid % a.NT);
    const int bidx = s / a.H, h = s % a.H;
    const int t0 = c * CH;
    const int nvalid = min(CH, a.T - t0);
    const size_t rowk0 = ((size_t)bidx * a.T + t0) * a.H + h;  // token-row index of row 0
    const size_t rsk = (size_t)a.H * DK, rsv = (size_t)a.H * DV;
    const Layout& L = a.L;
    OT* qg_out = (OT*)(a.ws + L.o_qg) + cid * L.qg;
    OT* kd_out = (OT*)(a.ws + L.o_kd) + cid * L.kd;
    OT* m_out = (OT*)(a.ws + L.o_m) + cid * L.m;
    OT* wm_out = (OT*)(a.ws + L.o_wm) + cid * L.wm;
    OT* u_out = (OT*)(a.ws + L.o_u) + cid * L.u;
    float* gc_out = (float*)(a.ws + L.o_gc) + cid * L.gc;

    // ---- phase 1: cumulative decay, factors, Qg / Kd / exp(gam_C) out, X = w*v.
    // Inputs are read 16 bytes per lane: lane (li, lq) of a wave takes rows 16 t + li and
    // W consecutive channels of a GC = 4 W channel group; wave wv owns key-channel groups
    // wv + 4 ai and value-channel groups wv + 4 ji. All loads are issued before any use;
    // the arithmetic then runs on 4-channel quarters.
    {
        constexpr int W = 16 / (int)sizeof(OT), GC = 4 * W;
        constexpr int NGK = DK / GC, NGV = DV / GC;
        constexpr int NA = (NGK + 3) / 4, NJ = (NGV + 3) / 4;
        using RT = typename Raw16<OT>::type;
        RT rg[NA][4], rq[NA][4], rk[NA][4], rb[NA][4], rv[NJ][4], rw[NJ][4];
        float span = 0.f;  // largest s(R, R) exponent of this lane's channels
#pragma unroll
        for (int ai = 0; ai < NA; ++ai) {
            if (wv + 4 * ai >= NGK) break;
            const int ch = GC * (wv + 4 * ai) + W * lq;
            ld_rows16((const OT*)a.g + rowk0 * DK, rsk, ch, nvalid, rg[ai]);
            ld_rows16((const OT*)a.q + rowk0 * DK, rsk, ch, nvalid, rq[ai]);
            ld_rows16((const OT*)a.k + rowk0 * DK, rsk, ch, nvalid, rk[ai]);
            ld_rows16((const OT*)a.b + rowk0 * DK, rsk, ch, nvalid, rb[ai]);
        }
#pragma unroll
        for (int ji = 0; ji < NJ; ++ji) {
            if (wv + 4 * ji >= NGV) break;
            const int ch = GC * (wv + 4 * ji) + W * lq;
            ld_rows16((const OT*)a.v + rowk0 * DV, rsv, ch, nvalid, rv[ji]);
            ld_rows16((const OT*)a.w + rowk0 * DV, rsv, ch, nvalid, rw[ji]);
        }
#pragma unroll
        for (int ai = 0; ai < NA; ++ai) {
            if (wv + 4 * ai >= NGK) break;
            RT qgp[4];  // Q_g of this lane's W channels, rows 16 t + li, stored once both quarters are in
#pragma unroll
            for (int hq = 0; hq < W / 4; ++hq) {
                const int ch0 = GC * (wv + 4 * ai) + W * lq + 4 * hq;
                float gv[4][4], gf[4][4], gt[4][4], gi[4][4];
                cvt_rows16<OT>(rg[ai], hq, nvalid, gv);
                if (ACT) activate_rows<OT, GATE_G>(gv, nvalid, a.g_scale, a.b_scale);
                float rep[4][4];
                DecayRep<OT>::store(gv, rep);
                DecayRep<OT>::scan(rep, gf, gt, gi);
                span = fmaxf(span, diag_span(gi));
                RowExp rx;
                row_exps<DK>(sF, ch0, gf, gt, gi, rx);
                if (li == 1) st4(gc_out + ch0, rx.x1);  // exp(gam_C)
                float qv[4][4], kv[4][4], bv[4][4];
                cvt_rows16<OT>(rq[ai], hq, nvalid, qv);
                cvt_rows16<OT>(rk[ai], hq, nvalid, kv);
                cvt_rows16<OT>(rb[ai], hq, nvalid, bv);
                if (ACT) activate_rows<OT, GATE_B>(bv, nvalid, a.g_scale, a.b_scale);
                float qg[4][4];
                scaled_factors_from<OT, DK, true>(qv, kv, bv, ch0, rep, sXA, sXM, sY, qg, &rx);
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) qgp[t][4 * hq + i] = to_ot<OT>(qg[t][i]);
            }
            // whole 16-byte pieces: with non-temporal stores, two 8-byte halves written apart
            // would each go to memory as a partial line
#pragma unroll
            for (int t = 0; t < 4; ++t)
                store_out<NT>((RT*)(qg_out + fimg<OT, DK>(16 * t + li, GC * (wv + 4 * ai) + W * lq)), qgp[t]);
        }
#pragma unroll
        for (int ji = 0; ji < NJ; ++ji) {
            if (wv + 4 * ji >= NGV) break;
#pragma unroll
            for (int hq = 0; hq < W / 4; ++hq) {
                float vv[4][4], ww[4][4];
                cvt_rows16<OT>(rv[ji], hq, nvalid, vv);
                cvt_rows16<OT>(rw[ji], hq, nvalid, ww);
                if (ACT) activate_rows<OT, GATE_W>(ww, nvalid, a.g_scale, a.b_scale);
                x_tile_from<OT, DV>(vv, ww, GC * (wv + 4 * ji) + W * lq + 4 * hq, sX);
            }
        }
        // every wave reports whether a diagonal block of its channels needs the slow path
        const bool strong = __ballot(span > span_max<OT>()) != 0;
        if (l == 0) lds_store<int>(smem + LS::FLAG + 4 * wv, strong ? 1 : 0);
    }
    sync_lds();
    const bool slow = (lds_load<int>(smem + LS::FLAG) | lds_load<int>(smem + LS::FLAG + 4) |
                       lds_load<int>(smem + LS::FLAG + 8) | lds_load<int>(smem + LS::FLAG + 12)) != 0;
    const LSwz<OT, DK> vXA{sXA}, vXM{sXM}, vY{sY};

    // ---- Kd^T = (k * exp(gam_C - gam))^T out to global as a fragment image, read from the Y
    // tile (Y = k * E2) by transposing reads, each lane's 8 tokens in one 16-token block R
    // whose factor exp(gam_C - gam_Rend) it applies; one contiguous kilobyte per fragment.
    for (int f = wv; f < (DK / 16) * (CH / 32); f += 4) {
        const int kt = f / (CH / 32), tb = f % (CH / 32);
        FT fr = lfrag_colk8<OT>(vY, 16 * kt, 32 * tb);  // lane (li, lq): Y[32 tb + 8 lq + e][16 kt + li]
        const float sc = lds_load<float>(sF + ((F_ECE + (32 * tb + 8 * lq) / 16) * DK + 16 * kt + li) * 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) fr[e] = to_ot<OT>(to_f(fr[e]) * sc);
        store_frag_img<OT, CH, NT>(kd_out, 16 * kt, 32 * tb, fr);
    }

    // ---- phase 2a: M = lower(Qg Khat^T), computed as M^T tiles, out to global
    const LSwz<OT, DV> vX{sX};
    for (int p = wv; p < NPAIR; p += 4) {
        int R, I;
        pair_ri(p, R, I);
        if (slow && R == I) continue;  // written by the slow path
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            mma(acc, lfrag_rowk<OT, OT>(vY, 16 * I, 32 * kb),
                lfrag_rowk<OT, OT>(vXM, 16 * R, 32 * kb, sF + (F_S + p) * DK * 4));
        float v[4];  // lane holds M[16R + li][16I + 4lq + i]
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (R == I && 4 * lq + i > li) ? 0.f : acc[i];
        st4_out<NT>(m_out + fimg<OT, CH>(16 * R + li, 16 * I + 4 * lq), v);
    }
    for (int u = wv; u < 6; u += 4) {
        int R, I;
        upper_ri(u, R, I);
        const float z[4] = {0.f, 0.f, 0.f, 0.f};
        st4_out<NT>(m_out + fimg<OT, CH>(16 * R + li, 16 * I + 4 * lq), z);
    }
    sync_lds();  // XM is dead from here on; its slot becomes A

    // ---- phase 2b: A = strict_lower(Kb Khat^T), fp32 into LDS
    for (int p = wv; p < NPAIR; p += 4) {
        int R, I;
        pair_ri(p, R, I);
        if (slow && R == I) continue;  // written by the slow path
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
            mma(acc, lfrag_rowk<OT, OT>(vY, 16 * I, 32 * kb),
                lfrag_rowk<OT, OT>(vXA, 16 * R, 32 * kb, sF + (F_S + p) * DK * 4));
        float v[4];  // lane holds A[16R + li][16I + 4lq + i]
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (R == I && 4 * lq + i >= li) ? 0.f : acc[i];
        lds_put4<float>(sA + swz<float, CH>(16 * R + li, 16 * I + 4 * lq) * 4, v);
    }
    sync_lds();  // Y is dead from here on; its slot becomes T

    // ---- XA -> K_b = b k exp(gam) for phase 4, once and in place (no phase reads XA before
    // then): row r takes the factor exp(gam at the first row of its 16-row block), per key
    // channel, rounded to the operand type as a rescaled fragment would be
    {
        constexpr int EPC = 16 / (int)sizeof(OT), NCK = DK / EPC;  // 16-byte chunks per row
        using RT = typename Raw16<OT>::type;
        for (int e = tid; e < CH * NCK; e += 256) {
            const int r = e / NCK, pos = e % NCK, c0 = (pos ^ swz_f<OT, DK>(r)) * EPC;
            lds_char* p = sXA + (r * DK + pos * EPC) * (int)sizeof(OT);
            RT x = lds_load<RT>(p);
            float f[EPC];
#pragma unroll
            for (int h = 0; h < EPC / 4; ++h) {
                float f4[4];
                lds_get4<float>(sF + ((F_ER0 + r / 16) * DK + c0 + 4 * h) * 4, f4);
#pragma unroll
                for (int i = 0; i < 4; ++i) f[4 * h + i] = f4[i];
            }
#pragma unroll
            for (int i = 0; i < EPC; ++i) x[i] = to_ot<OT>((float)x[i] * f[i]);
            lds_store<RT>(p, x);
        }
    }

    // ---- strong decay: the diagonal blocks of A and M, exactly (the factor rows in sF and
    // the Y slot are dead once K_b has been formed)
    if (slow) {
        sync_lds();
        fwd_diag_exact<OT, DK, ACT>(a, rowk0, nvalid, sF, sT, sA, m_out);
    }

    // ---- phase 3: T = (I + A)^-1
    for (int idx = tid; idx < 6 * 64; idx += 256) {  // zero the upper blocks of T
        int R, I;
        upper_ri(idx / 64, R, I);
        const int e = idx % 64;
        const float z[4] = {0.f, 0.f, 0.f, 0.f};
        lds_put4<float>(sT + swz<float, CH>(16 * R + e / 4, 16 * I + 4 * (e % 4)) * 4, z);
    }
    blocked_inverse(sA, sT);

    // ---- phase 4: U = T X (tiles) and Wm = T Kb (computed as Wm^T tiles -> row pieces).
    // Both K blocks are always multiplied: the upper blocks of T are stored zeros, and
    // compile-time loops keep the fragments in registers (no dynamic indexing).
    {
        const int tt = wv;  // token tile of the U / Wm rows
        const LSwz<float, CH> vT{sT};
        FT aT[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) aT[kb] = lfrag_rowk<OT, float>(vT, 16 * tt, 32 * kb);
#pragma unroll
        for (int j = 0; j < DV / 16; ++j) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) mma(acc, aT[kb], lfrag_colk<OT, OT>(vX, 16 * j, 32 * kb));
            store_tile<OT, NT>(u_out + (j * 4 + tt) * 256, acc);
        }
#pragma unroll
        for (int at = 0; at < DK / 16; ++at) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) mma(acc, lfrag_colk<OT, OT>(vXA, 16 * at, 32 * kb), aT[kb]);  // XA holds K_b
            float v[4] = {acc[0], acc[1], acc[2], acc[3]};  // Wm[16tt + li][16at + 4lq + i]
            st4_out<NT>(wm_out + fimg<OT, DK>(16 * tt + li, 16 * at + 4 * lq), v);
        }
    }
    if (TRAIN) {  // T for the backward chain
        OT* t_out = (OT*)(a.ws + L.o_t) + cid * L.t;
        for (int idx = tid; idx < CH * CH / 4; idx += 256) {
            const int r = idx / 16, c4 = 4 * (idx % 16);
            float v[4];
            lds_get4<float>(sT + swz<float, CH>(r, c4) * 4, v);
            st4_out<NT>(t_out + swz<OT, CH>(r, c4), v);
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
    auto pick = [&](auto nt) {
        constexpr bool NT = decltype(nt)::value;
        return a.act ? (train ? k_fwd_intra<OT, DK, DV, true, true, NT> : k_fwd_intra<OT, DK, DV, false, true, NT>)
                     : (train ? k_fwd_intra<OT, DK, DV, true, false, NT> : k_fwd_intra<OT, DK, DV, false, false, NT>);
    };
    auto intra = a.nt_out ? pick(std::true_type{}) : pick(std::false_type{});
    hipError_t e = hipFuncSetAttribute((const void*)intra, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // stage events: 0 at the start of the intra-chunk kernel, 1 at its end, 2 at the end of the chain
    hipExtLaunchKernelGGL(intra, dim3((unsigned)a.NC), dim3(256), lds, stream, stage_event(a, 0), stage_event(a, 1),
                          0, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_fwd_chain_t<OT, DK, DV>(a, train, stream, nullptr, stage_event(a, 2));
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
