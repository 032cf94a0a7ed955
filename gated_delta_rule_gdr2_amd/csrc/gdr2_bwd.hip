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
// The log-decay gradient: gam enters only through the factors Qg = q*exp(gam),
// Kb = b*k*exp(gam), Khat = k*exp(-gam) and Kd = k*exp(gam_C - gam), and through
// the carried state's exp(gam_C). dg_t (the gradient of g at token t = sum over
// the rows r >= t of the gradient of gam_r) is assembled from terms that never
// cancel, so it stays accurate when it is tiny (strong decay):
//   dg_t = sum_{r >= t} (Qg.dQg + Kb.dKb - Khat.dKhat)_r      (suffix sum)
//        + sum_{r < t} (Kd.dKd)_r                             (exclusive prefix sum)
//        + exp(gam_C) * rowsum(dS' * S)
// (the Kd term enters gam_r with a minus sign and gam_C with a plus sign, so only
// rows before t keep it; the diagonal of dM, q_r . k_r, does not depend on the
// decay and is left out).
//
// Kernels:
//   k_bwd_chain : (gdr2_chain.hip) one workgroup per (sequence, 16-column value
//                 slice), chunks in reverse; the state gradient's key rows split
//                 over the compute waves, held in accumulator registers; writes
//                 dS' (fragment-major) and dY (tiles) per chunk.
//   k_bwd_intra : one workgroup per chunk, fully parallel; reads the saved S,
//                 Delta, dS', dY and the inputs, writes dq, dk, dv, dg, db, dw.
//                 With gates passed as logits (ACT) it activates g and b once, in
//                 phase 1 (b, and d g / d z_g, go back into the staged tiles), w where
//                 it is read, and multiplies dg, db, dw by the activations' derivatives
//                 before they are stored (gradients with respect to the logits).
//                 NT (large workspaces): the gradients go out with non-temporal stores,
//                 and the saved S, dS', Delta and dY -- read here for the last time --
//                 come in with non-temporal loads, so that they do not displace the
//                 inputs from the Infinity Cache (measured at the headline shape: the
//                 backward itself unchanged, the next forward intra-chunk kernel over
//                 the same inputs 0.091 -> 0.085 ms).
#include "gdr2_intra_common.hpp"
#include "gdr2_kernels.hpp"

namespace gdr2 {

template <class OT, int DK, int DV>
struct BwdLds {  // all matrices are swizzled tiles (see swz())
    static constexpr int ES = sizeof(OT);
    static constexpr int KMAT = CH * DK * ES;
    static constexpr int VMAT = CH * DV * ES;
    static constexpr int SLOT = KMAT > VMAT ? KMAT : VMAT;
    static constexpr int S0 = 0;             // dO, later XA
    static constexpr int S1 = S0 + SLOT;     // Delta, later XM
    static constexpr int S2 = S1 + SLOT;     // dY, later Y
    static constexpr int DA = S2 + SLOT;     // dA [CH][CH]
    static constexpr int DM = DA + CH * CH * ES;
    static constexpr int F = DM + CH * CH * ES;
    static constexpr int DMD = F + F_ROWS * DK * 4;  // diagonal of dM, fp32
    static constexpr int CARRY = DMD + CH * 4;       // per key channel, fp32: rowsum(dS'*S) (at DK + channel)
    static constexpr int G = CARRY + 2 * DK * 4;     // g, q, k, b of the chunk [CH][DK]
    static constexpr int Q = G + KMAT;
    static constexpr int K = Q + KMAT;
    static constexpr int B = K + KMAT;
    static constexpr int FLAG = B + KMAT;  // one int per wave: strong decay seen
    static constexpr int BYTES = FLAG + 32;
};

// tile dump [DV/16][4][64 lanes][4] -> swizzled LDS tile [CH][DV], in two steps so the
// loads can be issued early: element group e = threadIdx.x + NTHR * u, u < NU
template <class OT, int DV, int NTHR>
struct Undump {
    static constexpr int NU = (DV / 16) * 4 * 64 / NTHR;
    static_assert((DV / 16) * 4 * 64 % NTHR == 0, "tile dump divides evenly over the threads");
};
template <class OT, int DV, int NTHR, bool NT>
__device__ __forceinline__ void undump_load(const OT* src, typename Raw4<OT>::type (&raw)[Undump<OT, DV, NTHR>::NU]) {
#pragma unroll
    for (int u = 0; u < Undump<OT, DV, NTHR>::NU; ++u)
        raw[u] = load_in<NT>((const typename Raw4<OT>::type*)(src + (size_t)(threadIdx.x + NTHR * u) * 4));
}
template <class OT, int DV, int NTHR>
__device__ __forceinline__ void undump_store(const typename Raw4<OT>::type (&raw)[Undump<OT, DV, NTHR>::NU],
                                             lds_char* dst) {
#pragma unroll
    for (int u = 0; u < Undump<OT, DV, NTHR>::NU; ++u) {
        const int e = threadIdx.x + NTHR * u;
        const int lane = e & 63, t = (e >> 6) & 3, jj = e >> 8;
        const int row = 16 * t + 4 * (lane >> 4), col = 16 * jj + (lane & 15);
        if constexpr (sizeof(OT) == 2) {
            // Lanes col and col ^ 1 (a DPP pair) hold rows row .. row + 3 of adjacent columns;
            // they swap halves so that each stores two rows as 4-byte column pairs.
            typedef __attribute__((address_space(3))) uint32_t U32;
            const bool odd = lane & 1;
            const bf16x4 v = raw[u];
            const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_shufflevector(v, v, 0, 1));
            const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_shufflevector(v, v, 2, 3));
            const uint32_t send = odd ? lo : hi;
            const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
            const uint32_t mine = odd ? hi : lo;  // rows row + 2, 3 (odd) or row + 0, 1 (even) of this column
            // the column-c0 and column-c0 + 1 halves; w0 / w1 = first / second row, low half = column c0
            const uint32_t lowsrc = odd ? recv : mine, highsrc = odd ? mine : recv;
            const uint32_t w0 = __builtin_amdgcn_perm(highsrc, lowsrc, 0x05040100);
            const uint32_t w1 = __builtin_amdgcn_perm(highsrc, lowsrc, 0x07060302);
            const int r0 = row + (odd ? 2 : 0), c0 = col & ~1;
            *(U32*)(dst + swz<OT, DV>(r0, c0) * 2) = w0;
            *(U32*)(dst + swz<OT, DV>(r0 + 1, c0) * 2) = w1;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_store<OT>(dst + swz<OT, DV>(row + i, col) * (int)sizeof(OT), raw[u][i]);
        }
    }
}
template <class OT, int DV, int NTHR>
__device__ __forceinline__ void undump_tiles(const OT* src, lds_char* dst) {
    for (int e = threadIdx.x; e < (DV / 16) * 4 * 64; e += NTHR) {
        const int lane = e & 63, t = (e >> 6) & 3, jj = e >> 8;
        float v[4];
        ld4(src + (size_t)e * 4, v);
        const int row = 16 * t + 4 * (lane >> 4), col = 16 * jj + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_store<OT>(dst + swz<OT, DV>(row + i, col) * (int)sizeof(OT), to_ot<OT>(v[i]));
    }
}

constexpr int BWD_NW = 8;  // waves per workgroup of the backward intra-chunk kernel

// L2 warm-up for the next round. One workgroup per compute unit and chunk means that the
// loads of a chunk (about 200 KB at d = 128) are the compute unit's only memory traffic for
// the first quarter of the chunk's time and none is in flight afterwards. During this
// chunk's phase 2, every lane reads one 4-byte word of up to NI cache lines of the rows the
// chunk at blockIdx + a.l2_ahead will stage by DMA (g, q, k, b, dO: 80 KB at d = 128) --
// the chunk the same XCD runs next -- so that they come from L2 when that workgroup starts
// (the other 128 KB it reads would not fit in L2 beside them: measured slower). The words
// are kept in registers and consumed by an empty asm statement at the end of the kernel.
template <class OT, int DK, int DV, int NTHR>
struct L2Warm {
    static constexpr int LPRK = DK * (int)sizeof(OT) / 128, LPRV = DV * (int)sizeof(OT) / 128;  // lines per row
    static constexpr int NL = 4 * CH * LPRK + CH * LPRV;
    static constexpr int NI = (NL + NTHR - 1) / NTHR;
};
template <class OT, int DK, int DV, int NTHR>
__device__ __forceinline__ void l2_warm_next(const Args& a, long long cid, uint32_t (&word)[L2Warm<OT, DK, DV, NTHR>::NI]) {
    using W = L2Warm<OT, DK, DV, NTHR>;
#pragma unroll
    for (int i = 0; i < W::NI; ++i) word[i] = 0;
    const long long cid2 = cid + a.l2_ahead;
    if (a.l2_ahead <= 0 || cid2 >= a.NC) return;
    const int s2 = (int)(cid2 / a.NT), c2 = (int)(cid2 % a.NT);
    const int nv2 = min(CH, a.T - c2 * CH);
    const size_t r0 = ((size_t)(s2 / a.H) * a.T + (size_t)c2 * CH) * a.H + s2 % a.H;  // token row of its row 0
#pragma unroll
    for (int i = 0; i < W::NI; ++i) {
        const int v = threadIdx.x + NTHR * i;  // line v: tensor, row, line in the row
        const char* p = nullptr;
        if (v < 4 * CH * W::LPRK) {
            const int t = v / (CH * W::LPRK), r = v % (CH * W::LPRK) / W::LPRK, ln = v % W::LPRK;
            const void* base = t == 0 ? a.g : t == 1 ? a.q : t == 2 ? a.k : a.b;
            if (r < nv2) p = (const char*)((const OT*)base + (r0 + (size_t)r * a.H) * DK) + ln * 128;
        } else if (v < W::NL) {
            const int u = v - 4 * CH * W::LPRK, r = u / W::LPRV, ln = u % W::LPRV;
            if (r < nv2) p = (const char*)((const OT*)a.dout + (r0 + (size_t)r * a.H) * DV) + ln * 128;
        }
        if (p) word[i] = *(const uint32_t*)p;
    }
}

template <class OT, int DK, int DV, bool ACT, bool NT>
__global__ __launch_bounds__(64 * BWD_NW) void k_bwd_intra(Args a) {
    using LS = BwdLds<OT, DK, DV>;
    using FT = typename Frag<OT>::type;
    constexpr int NW = BWD_NW, NTHR = 64 * NW;
    constexpr int KV = DV / 32;
    constexpr int CPW = (DK / 16 + NW - 1) / NW;  // key-channel tiles per wave
    extern __shared__ __align__(16) char smem_[];
    lds_char* smem = (lds_char*)smem_;
    poison_lds(smem, LS::BYTES);
    poison_lds_done();
    lds_char* sDO = smem + LS::S0;
    lds_char* sDL = smem + LS::S1;
    lds_char* sDY = smem + LS::S2;
    lds_char* sXA = smem + LS::S0;
    lds_char* sXM = smem + LS::S1;
    lds_char* sY = smem + LS::S2;
    lds_char* sDA = smem + LS::DA;
    lds_char* sDM = smem + LS::DM;
    lds_char* sF = smem + LS::F;
    lds_char* sDMd = smem + LS::DMD;

    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, li = l & 15, lq = l >> 4;
    const long long cid = blockIdx.x;
    const int s = (int)(cid / a.NT), c = (int)(cid % a.NT);
    const int bidx = s / a.H, h = s % a.H;
    const int t0 = c * CH;
    const int nvalid = min(CH, a.T - t0);
    const size_t rowk0 = ((size_t)bidx * a.T + t0) * a.H + h;
    const size_t rsk = (size_t)a.H * DK, rsv = (size_t)a.H * DV;
    const Layout& L = a.L;

    // ---- loads, all issued up front. The row tensors g, q, k, b and dO go to LDS by DMA
    // in whole rows (dma_rows); v and w come to registers as 16-byte row pieces, lane
    // t covering chunk t % NCV of row t / NCV of the chunk (pieces t, t + NTHR, ...);
    // the saved states as MFMA fragments and the Delta / dY tile dumps as 4-element
    // pieces. Wave wv owns key-channel tiles wv + NW ac.
    using RT = typename Raw4<OT>::type;
    using UD = Undump<OT, DV, NTHR>;
    lds_char* sG = smem + LS::G;
    lds_char* sQ = smem + LS::Q;
    lds_char* sK = smem + LS::K;
    lds_char* sB = smem + LS::B;
    const OT* Sg = (const OT*)(a.ws + L.o_s) + cid * L.s;
    const OT* dSg = (const OT*)(a.ws + L.o_ds) + cid * L.ds;
    dma_rows<OT, DK, NW>((const OT*)a.g + rowk0 * DK, rsk, nvalid, sG, wv);
    dma_rows<OT, DK, NW>((const OT*)a.q + rowk0 * DK, rsk, nvalid, sQ, wv);
    dma_rows<OT, DK, NW>((const OT*)a.k + rowk0 * DK, rsk, nvalid, sK, wv);
    dma_rows<OT, DK, NW>((const OT*)a.b + rowk0 * DK, rsk, nvalid, sB, wv);
    dma_rows<OT, DV, NW>((const OT*)a.dout + rowk0 * DV, rsv, nvalid, sDO, wv);
    constexpr int WV = 16 / (int)sizeof(OT), NCV = DV / WV;  // elements per piece, pieces per row
    constexpr int NPW = CH * NCV / NTHR;                     // v / w pieces per thread
    static_assert(CH * NCV % NTHR == 0, "the value rows split evenly over the threads");
    using RW = typename Raw16<OT>::type;
    RW rv[NPW], rw[NPW];
    RT rdl[UD::NU], rdy[UD::NU];
    // the saved-state fragments are fetched up front too, except for fp32 operands,
    // where they would not fit in registers next to the rest
    constexpr bool EARLY_S = sizeof(OT) == 2;
    static_assert(!EARLY_S || CPW == 1, "the load count below assumes one key-channel tile per wave");
    FT Sf[CPW][KV], dSf[CPW][KV];
    // Issue order after the DMAs: the Delta / dY dumps (needed at the end of phase 1), v and
    // w (end of phase 3a), the saved states (phase 3a). The scheduling fences keep the DMAs
    // first, so the wait below covers them alone and the later loads stay in flight
    // through phases 1 and 2. Each of these loads is one instruction (8 or 16 bytes).
    __builtin_amdgcn_sched_barrier(0);
    undump_load<OT, DV, NTHR, NT>((const OT*)(a.ws + L.o_delta) + cid * L.delta, rdl);
    undump_load<OT, DV, NTHR, NT>((const OT*)(a.ws + L.o_dy) + cid * L.dy, rdy);
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
        const int pc = tid + NTHR * i, r = pc / NCV, rr = r < nvalid ? r : nvalid - 1;
        const size_t off = (rowk0 + (size_t)rr * a.H) * DV + WV * (pc % NCV);
        rv[i] = *(const RW*)((const OT*)a.v + off);
        rw[i] = *(const RW*)((const OT*)a.w + off);
    }
    if (EARLY_S) {  // waves without a key-channel tile (d_k = 64) load tile 0 and ignore it
        const int at = wv < DK / 16 ? wv : 0;
#pragma unroll
        for (int kb = 0; kb < KV; ++kb) {
            Sf[0][kb] = frag_fmaj<OT, DV, NT>(Sg, at, kb);
            dSf[0][kb] = frag_fmaj<OT, DV, NT>(dSg, at, kb);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // wait for this wave's copies (and the barrier below for everyone's), then zero the
    // padding rows of a partial chunk (positions no DMA writes)
    wait_vm<2 * UD::NU + 2 * NPW + (EARLY_S ? 2 * KV : 0)>();
    if (nvalid < CH) {
        zero_tail_rows<OT, DK, NTHR>(sG, nvalid);
        zero_tail_rows<OT, DK, NTHR>(sQ, nvalid);
        zero_tail_rows<OT, DK, NTHR>(sK, nvalid);
        zero_tail_rows<OT, DK, NTHR>(sB, nvalid);
        zero_tail_rows<OT, DV, NTHR>(sDO, nvalid);
    }
    sync_lds();  // LDS only: the later loads stay in flight
    // this lane's 4-channel pieces (rows 16 t + li, channels ch0 .. ch0 + 3) of a staged tile
    const LSwz<OT, DK> vG{sG}, vQ{sQ}, vK{sK}, vB{sB};
    auto rows4 = [&](const LSwz<OT, DK>& v, int ch0, float (&out)[4][4]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) lds_get4<OT>(v.p + v.off(16 * t + li, ch0), out[t]);
    };

    // ---- phase 1: block sums of the log-decay (see gdr2_intra_common.hpp) and factors;
    // Delta, dY into LDS. gam keeps this lane's log-decays (activated; in their stored form,
    // see DecayRep) for the later phases.
    float gam[CPW][4][4];
    float span = 0.f;  // largest s(R, R) exponent of this lane's channels
#pragma unroll
    for (int ac = 0; ac < CPW; ++ac) {
        if (wv + NW * ac >= DK / 16) break;
        const int ch0 = 16 * (wv + NW * ac) + 4 * lq;
        float gv[4][4], gf[4][4], gt[4][4], gi[4][4];
        rows4(vG, ch0, gv);
        if (ACT) {
            // Gates given as logits, activated once here for this wave's columns: g from
            // z_g, with d g / d z = -g_scale sigmoid(z_g) written over z_g in the g tile
            // (the finals need it), and b over z_b in the b tile (phases 3b and 3c read it).
            float dz[4][4], bv[4][4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float sp, sg;
                    gate_softplus_sigmoid<OT>(gv[t][i], sp, sg);
                    gv[t][i] = 16 * t + li < nvalid ? -a.g_scale * sp : 0.f;
                    dz[t][i] = -a.g_scale * sg;
                }
            rows4(vB, ch0, bv);
            activate_rows<OT, GATE_B>(bv, nvalid, a.g_scale, a.b_scale);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                lds_put4<OT>(sG + vG.off(16 * t + li, ch0), dz[t]);
                lds_put4<OT>(sB + vB.off(16 * t + li, ch0), bv[t]);
            }
        }
        DecayRep<OT>::store(gv, gam[ac]);
        DecayRep<OT>::scan(gam[ac], gf, gt, gi);
        span = fmaxf(span, diag_span(gi));
        RowExp rx;
        row_exps<DK>(sF, ch0, gf, gt, gi, rx);
    }
    {  // every wave reports whether a diagonal block of its channels needs the slow path
        const bool strong = __ballot(span > span_max<OT>()) != 0;
        if (l == 0) lds_store<int>(smem + LS::FLAG + 4 * wv, strong ? 1 : 0);
    }
    undump_store<OT, DV, NTHR>(rdl, sDL);
    undump_store<OT, DV, NTHR>(rdy, sDY);
    {  // zero the upper blocks of dA, dM, a 16-byte chunk per store (no chunk spans two blocks)
        constexpr int EPC = 16 / (int)sizeof(OT), CPR = CH / EPC;  // elements per chunk, chunks per row
        static_assert(16 % EPC == 0 && CH * CPR % NTHR == 0, "the chunks split evenly over the threads");
#pragma unroll
        for (int u = 0; u < CH * CPR / NTHR; ++u) {
            const int idx = tid + NTHR * u, r = idx / CPR, c0 = EPC * (idx % CPR);
            if ((c0 >> 4) > (r >> 4)) {
                const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                lds_store<f32x4>(sDA + swz<OT, CH>(r, c0) * (int)sizeof(OT), z);
                lds_store<f32x4>(sDM + swz<OT, CH>(r, c0) * (int)sizeof(OT), z);
            }
        }
    }
    sync_lds();  // LDS only: the later loads stay in flight
    // Strong decay (slow path): the diagonal block pairs of the bilinear products are left
    // out of phase 3c (their factor s(R, R) is set to zero here; it may be infinite) and
    // added in the finals from per-element exponentials instead.
    bool slow = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) slow |= lds_load<int>(smem + LS::FLAG + 4 * w) != 0;
    if (slow)
        for (int e = tid; e < NBLK * DK; e += NTHR)
            lds_store<float>(sF + ((F_S + pair_id(e / DK, e / DK)) * DK + e % DK) * 4, 0.f);

    uint32_t warm[L2Warm<OT, DK, DV, NTHR>::NI];
    l2_warm_next<OT, DK, DV, NTHR>(a, cid, warm);
    __builtin_amdgcn_sched_barrier(0);

    // ---- phase 2: dA = -strict_lower(dY Delta^T), dM = lower(dO Delta^T)
    // The diagonal of M, q_r . k_r, does not depend on the decay; its gradient is
    // kept apart in fp32 (sDMd) so that its query-side and key-side terms cancel
    // exactly in the log-decay gradient instead of up to bf16 rounding.
    const LSwz<OT, DV> vDO{sDO}, vDL{sDL}, vDY{sDY};
    // Computed as transposed tiles (Delta rows as the A operand), so that each lane holds
    // four consecutive columns of one row and stores them as one 4-element piece.
    for (int p = wv; p < 2 * NPAIR; p += NW) {
        const bool isM = p >= NPAIR;
        int R, I;
        pair_ri(isM ? p - NPAIR : p, R, I);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KV; ++kb)
            mma(acc, lfrag_rowk8<OT>(vDL, 16 * I, 32 * kb), lfrag_rowk8<OT>(isM ? vDO : vDY, 16 * R, 32 * kb));
        const int row = 16 * R + li, col0 = 16 * I + 4 * lq;  // acc[i]: (row, col0 + i)
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int col = col0 + i;
            v[i] = isM ? acc[i] : -acc[i];
            if (isM && col == row) lds_store<float>(sDMd + row * 4, v[i]);
            if (R == I && col >= row) v[i] = 0.f;  // dA strictly lower; dM diagonal kept in sDMd
        }
        lds_put4<OT>((isM ? sDM : sDA) + swz<OT, CH>(row, col0) * (int)sizeof(OT), v);
    }
    sync_lds();  // LDS only: the later loads stay in flight

    // ---- phase 3a: products with the saved states, dv and dw
    // Per key-channel tile, transposed tiles (rows = key channel, columns = token):
    //   Pq = exp(gam_R0) * (dO S^T)^T, Pb = -exp(gam_R0) * (dY S^T)^T,
    //   Pk = exp(gam_C - gam_Rend) * (Delta dS'^T)^T
    // The bilinear terms are accumulated into Pq, Pb and (the key side, starting from zero)
    // Pk in phase 3c; the carried-state term of the key side stays apart in PkS.
    f32x4 Pq[CPW][4], Pb[CPW][4], Pk[CPW][4], PkS[CPW][4];
    // A per-channel sum goes from here to the finals: in registers, or through LDS (sCarry)
    // when the gates come as logits, where the registers would not hold it.
    constexpr bool CARRY_LDS = ACT;
    f32x4 rsum[CPW];  // S dS'^T over this wave's 16 key channels; its diagonal is rowsum(dS' * S)
    lds_char* sCarry = smem + LS::CARRY;
#pragma unroll
    for (int ac = 0; ac < CPW; ++ac) {
        const int at = wv + NW * ac;
        if (at >= DK / 16) break;
        if (!EARLY_S) {
#pragma unroll
            for (int kb = 0; kb < KV; ++kb) {
                Sf[ac][kb] = frag_fmaj<OT, DV, NT>(Sg, at, kb);
                dSf[ac][kb] = frag_fmaj<OT, DV, NT>(dSg, at, kb);
            }
        }
        // lane (li, lq) element i: sum over v of S[16at + 4lq + i][v] dS'[16at + li][v], so the
        // diagonal (channel 16at + 4lq + i) is element i of lane (4lq + i, lq)
        f32x4 sd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KV; ++kb) mma(sd, Sf[ac][kb], dSf[ac][kb]);
        if (!CARRY_LDS) {
            rsum[ac] = sd;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (li == 4 * lq + i) lds_store<float>(sCarry + (DK + 16 * at + li) * 4, sd[i]);
        }
        const int ch0 = 16 * at + 4 * lq;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float e0v[4], ecv[4];  // exp(gam_t0), exp(gam_C - gam_tend) of channels ch0 + i
            lds_get4<float>(sF + ((F_ER0 + t) * DK + ch0) * 4, e0v);
            lds_get4<float>(sF + ((F_ECE + t) * DK + ch0) * 4, ecv);
            f32x4 q4 = {0.f, 0.f, 0.f, 0.f}, b4 = q4, k4 = q4;
#pragma unroll
            for (int kb = 0; kb < KV; ++kb) {
                mma(q4, Sf[ac][kb], lfrag_rowk8<OT>(vDO, 16 * t, 32 * kb));
                mma(b4, Sf[ac][kb], lfrag_rowk8<OT>(vDY, 16 * t, 32 * kb));
                mma(k4, dSf[ac][kb], lfrag_rowk8<OT>(vDL, 16 * t, 32 * kb));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Pq[ac][t][i] = e0v[i] * q4[i];
                Pb[ac][t][i] = -e0v[i] * b4[i];
                PkS[ac][t][i] = ecv[i] * k4[i];
                Pk[ac][t][i] = 0.f;
            }
        }
    }
    // dv = dY * w, dw = dY * v, in the row-piece layout of v and w
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
        const int pc = tid + NTHR * i, r = pc / NCV, ch = WV * (pc % NCV);
        const RW dy = lds_load<RW>(sDY + swz<OT, DV>(r, ch) * (int)sizeof(OT));
        RW dvv, dww;
#pragma unroll
        for (int e = 0; e < WV; ++e) {
            const float w = ACT ? gate_sigmoid<OT>(to_f(rw[i][e])) : to_f(rw[i][e]);
            const float dwdz = ACT ? w * (1.f - w) : 1.f;  // gradient through the write gate's sigmoid
            dvv[e] = to_ot<OT>(to_f(dy[e]) * w);
            dww[e] = to_ot<OT>(to_f(dy[e]) * to_f(rv[i][e]) * dwdz);
        }
        if (r < nvalid) {
            store_out<NT>((RW*)((OT*)a.dv + rowk0 * DV + (size_t)r * rsv + ch), dvv);
            store_out<NT>((RW*)((OT*)a.dw + rowk0 * DV + (size_t)r * rsv + ch), dww);
        }
    }
    sync_lds();  // dO, Delta, dY are dead; their slots take the key/query factors

    // ---- phase 3b: XA = b*k*E1, XM = q*E1, Y = k*E2 into LDS; E1 and E2 are kept for the finals
    float e1f[CPW][4][4], e2f[CPW][4][4];
#pragma unroll
    for (int ac = 0; ac < CPW; ++ac) {
        if (wv + NW * ac >= DK / 16) break;
        const int ch0 = 16 * (wv + NW * ac) + 4 * lq;
        float qv[4][4], kv[4][4], bv[4][4];
        rows4(vQ, ch0, qv);
        rows4(vK, ch0, kv);
        rows4(vB, ch0, bv);  // (activated in phase 1 when the gates came as logits)
        block_factors<OT>(gam[ac], e1f[ac], e2f[ac]);
        scaled_factors<OT, DK, false>(qv, kv, bv, ch0, e1f[ac], e2f[ac], sXA, sXM, sY, nullptr, nullptr);
    }
    sync_lds();

    // ---- phase 3c: bilinear back-propagation, then the elementwise finals
    const LSwz<OT, DK> vXA{sXA}, vXM{sXM}, vY{sY};
    const LSwz<OT, CH> vDA{sDA}, vDM{sDM};
#pragma unroll
    for (int ac = 0; ac < CPW; ++ac) {
        const int at = wv + NW * ac;
        if (at >= DK / 16) break;
        // The block-pair factor s(R, I) is per key channel, which is the row of every product
        // below: each 32-deep fragment pair is split into its two 16-token blocks, multiplied
        // unscaled, and the factor applied to the fp32 result (rows 16 at + 4 lq + i of a lane).
        auto sfac4 = [&](int R, int I, float (&s4)[4]) {
            lds_get4<float>(sF + ((F_S + pair_id(R, I)) * DK + 16 * at + 4 * lq) * 4, s4);
        };
#pragma unroll
        for (int R = 0; R < 4; ++R) {  // Xbar (erase / query side) for target block R
            for (int kb = 0; kb <= R / 2; ++kb) {
                const FT ay = lfrag_colk<OT, OT>(vY, 16 * at, 32 * kb);
                const FT da = lfrag_rowk<OT, OT>(vDA, 16 * R, 32 * kb), dm = lfrag_rowk<OT, OT>(vDM, 16 * R, 32 * kb);
                f32x4 tb = {0.f, 0.f, 0.f, 0.f}, tq = tb;
                float sc[4];
                mma_half<0>(tb, ay, da);
                mma_half<0>(tq, ay, dm);
                sfac4(R, 2 * kb, sc);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    Pb[ac][R][i] = fmaf(sc[i], tb[i], Pb[ac][R][i]);
                    Pq[ac][R][i] = fmaf(sc[i], tq[i], Pq[ac][R][i]);
                }
                if (2 * kb + 1 <= R) {
                    tb = f32x4{0.f, 0.f, 0.f, 0.f};
                    tq = tb;
                    mma_half<1>(tb, ay, da);
                    mma_half<1>(tq, ay, dm);
                    sfac4(R, 2 * kb + 1, sc);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        Pb[ac][R][i] = fmaf(sc[i], tb[i], Pb[ac][R][i]);
                        Pq[ac][R][i] = fmaf(sc[i], tq[i], Pq[ac][R][i]);
                    }
                }
            }
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {  // Ybar (key side) for source block I
            for (int kb = I / 2; kb < 2; ++kb) {
                const FT xa = lfrag_colk<OT, OT>(vXA, 16 * at, 32 * kb), xm = lfrag_colk<OT, OT>(vXM, 16 * at, 32 * kb);
                const FT dat = lfrag_colk<OT, OT>(vDA, 16 * I, 32 * kb), dmt = lfrag_colk<OT, OT>(vDM, 16 * I, 32 * kb);
                float sc[4];
                if (2 * kb >= I) {  // target block R = 2 kb
                    f32x4 t = {0.f, 0.f, 0.f, 0.f};
                    mma_half<0>(t, xa, dat);
                    mma_half<0>(t, xm, dmt);
                    sfac4(2 * kb, I, sc);
#pragma unroll
                    for (int i = 0; i < 4; ++i) Pk[ac][I][i] = fmaf(sc[i], t[i], Pk[ac][I][i]);
                }
                {  // target block R = 2 kb + 1 (always >= I)
                    f32x4 t = {0.f, 0.f, 0.f, 0.f};
                    mma_half<1>(t, xa, dat);
                    mma_half<1>(t, xm, dmt);
                    sfac4(2 * kb + 1, I, sc);
#pragma unroll
                    for (int i = 0; i < 4; ++i) Pk[ac][I][i] = fmaf(sc[i], t[i], Pk[ac][I][i]);
                }
            }
        }

        // finals at (key channel 16at + 4lq + i, token 16t + li)
        const int ch0 = 16 * at + 4 * lq;
        float qv[4][4], kv[4][4], bv[4][4];
        rows4(vQ, ch0, qv);
        rows4(vK, ch0, kv);
        rows4(vB, ch0, bv);
        // First the token-side sums in place, without the diagonal of dM: Pq -> dq, Pb -> the
        // K_b gradient times exp(gam) (gbk), Pk -> the Khat part of dk, PkS -> the Kd part.
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Pq[ac][t][i] = e1f[ac][t][i] * Pq[ac][t][i];
                Pb[ac][t][i] = e1f[ac][t][i] * Pb[ac][t][i];
                Pk[ac][t][i] = e2f[ac][t][i] * Pk[ac][t][i];
                PkS[ac][t][i] = e2f[ac][t][i] * PkS[ac][t][i];
            }
        }
        if (slow) {
            // Strong decay: the diagonal blocks' terms from per-element factors. With
            // e(r, j) = exp(gam_r - gam_j) = product of alpha_t = exp(g_t) over t in (j, r]
            // (<= 1 for j < r), per channel of this lane and token r:
            //   dq  += sum_{j<r} dM[r][j] k_j e(r, j)
            //   gbk += sum_{j<r} dA[r][j] k_j e(r, j)
            //   dk  += sum_{j>r} (dA[j][r] (b k)_j + dM[j][r] q_j) e(j, r)
            // the values of token j taken from lane j of the row; the products grow one
            // factor per step, j going down from r for the first two and up from r for dk.
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = 16 * t + li;
                float al[4], pl[4] = {1.f, 1.f, 1.f, 1.f}, ph[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) al[i] = DecayRep<OT>::alpha(gam[ac][t][i]);
#pragma unroll 1
                for (int j = 15; j >= 0; --j) {  // j < r: e(r, j) = alpha_r ... alpha_{j+1}
                    const int src1 = (l & 48) | ((j + 1) & 15);
                    const int cj = 16 * t + j, src = (l & 48) | j;
                    const float aR = lds_get1<OT>(sDA + swz<OT, CH>(r, cj) * (int)sizeof(OT));
                    const float mR = lds_get1<OT>(sDM + swz<OT, CH>(r, cj) * (int)sizeof(OT));
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float a1 = __shfl(al[i], src1, 64);
                        const float kj = __shfl(kv[t][i], src, 64);
                        if (j + 1 <= li) pl[i] *= a1;
                        const float lo = j < li ? pl[i] : 0.f;
                        Pq[ac][t][i] = fmaf(mR * kj, lo, Pq[ac][t][i]);
                        Pb[ac][t][i] = fmaf(aR * kj, lo, Pb[ac][t][i]);
                    }
                }
#pragma unroll 1
                for (int j = 0; j < 16; ++j) {  // j > r: e(j, r) = alpha_{r+1} ... alpha_j
                    const int cj = 16 * t + j, src = (l & 48) | j;
                    const float aC = lds_get1<OT>(sDA + swz<OT, CH>(cj, r) * (int)sizeof(OT));
                    const float mC = lds_get1<OT>(sDM + swz<OT, CH>(cj, r) * (int)sizeof(OT));
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float aj = __shfl(al[i], src, 64);
                        const float qj = __shfl(qv[t][i], src, 64);
                        const float bkj = __shfl(bv[t][i] * kv[t][i], src, 64);
                        if (j > li) ph[i] *= aj;
                        const float hi = j > li ? ph[i] : 0.f;
                        Pk[ac][t][i] = fmaf(aC * bkj + mC * qj, hi, Pk[ac][t][i]);
                    }
                }
            }
        }
        float dgp[4][4], kk[4][4];  // per row: Qg.dQg + Kb.dKb - Khat.dKhat, and Kd.dKd
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = 16 * t + li;
            const float dmd = lds_load<float>(sDMd + r * 4);
            float dq[4], dk[4], db[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float gbk = Pb[ac][t][i];
                db[i] = gbk * kv[t][i];
                dgp[t][i] = qv[t][i] * Pq[ac][t][i] + bv[t][i] * db[i] - kv[t][i] * Pk[ac][t][i];
                kk[t][i] = kv[t][i] * PkS[ac][t][i];
                dq[i] = Pq[ac][t][i] + dmd * kv[t][i];
                dk[i] = gbk * bv[t][i] + Pk[ac][t][i] + PkS[ac][t][i] + dmd * qv[t][i];
            }
            if (ACT) {  // db through the erase gate's scaled sigmoid: b_scale s (1 - s), s = b / b_scale
                const float rb = 1.f / a.b_scale;
#pragma unroll
                for (int i = 0; i < 4; ++i) db[i] *= bv[t][i] * (1.f - bv[t][i] * rb);
            }
            // into the staged q, k, b tiles (this wave alone reads and writes these columns)
            const int o = vQ.off(r, ch0);
            lds_put4<OT>(sQ + o, dq);
            lds_put4<OT>(sK + o, dk);
            lds_put4<OT>(sB + o, db);
        }
        // dg_t = suffix sum of dgp from t + exclusive prefix sum of kk before t + the carried
        // state's term exp(gam_C) rowsum(dS' * S), per channel (blocks of 16 rows, then
        // carries across the blocks; no subtraction anywhere)
        float cst[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float rs_i = CARRY_LDS ? lds_load<float>(sCarry + (DK + ch0 + i) * 4)
                                         : __shfl(rsum[ac][i], (l & 48) | (4 * lq + i), 64);
            const float gamC = (DecayRep<OT>::total(gam[ac][0][i]) + DecayRep<OT>::total(gam[ac][1][i])) +
                               (DecayRep<OT>::total(gam[ac][2][i]) + DecayRep<OT>::total(gam[ac][3][i]));
            cst[i] = __expf(gamC) * rs_i;
        }
        float later[4] = {0.f, 0.f, 0.f, 0.f}, before[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 3; t >= 0; --t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = row_suffix16(dgp[t][i]) + later[i];
                dgp[t][i] = x;
                later[i] = row_bcast<0>(x);
            }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = row_scan16(row_shr1(kk[t][i])) + before[i];
                before[i] = row_bcast<15>(x + kk[t][i]);
                kk[t][i] = x;
            }
        float gf[4][4];  // ACT: d g / d z, left in the g tile by phase 1
        if (ACT) rows4(vG, ch0, gf);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float dg[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dg[i] = dgp[t][i] + kk[t][i] + cst[i];
                if (ACT) dg[i] *= gf[t][i];
            }
            lds_put4<OT>(sG + vG.off(16 * t + li, ch0), dg);
        }
    }
    sync_lds();

    // ---- dq, dk, db, dg out of the staged tiles in whole rows
    store_rows_tiles<OT, DK, NTHR, NT>(sQ, (OT*)a.dq + rowk0 * DK, rsk, nvalid);
    store_rows_tiles<OT, DK, NTHR, NT>(sK, (OT*)a.dk + rowk0 * DK, rsk, nvalid);
    store_rows_tiles<OT, DK, NTHR, NT>(sB, (OT*)a.db + rowk0 * DK, rsk, nvalid);
    store_rows_tiles<OT, DK, NTHR, NT>(sG, (OT*)a.dg + rowk0 * DK, rsk, nvalid);
#pragma unroll
    for (int i = 0; i < L2Warm<OT, DK, DV, NTHR>::NI; ++i) asm volatile("" ::"v"(warm[i]));  // the warm-up loads stay
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
    auto intra = a.nt_out ? (a.act ? k_bwd_intra<OT, DK, DV, true, true> : k_bwd_intra<OT, DK, DV, false, true>)
                          : (a.act ? k_bwd_intra<OT, DK, DV, true, false> : k_bwd_intra<OT, DK, DV, false, false>);
    hipError_t e = hipFuncSetAttribute((const void*)intra, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // the next round of workgroups starts (compute units x workgroups per unit) chunks later
    int dev = 0, cus = 0, per_cu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)intra, 64 * BWD_NW, lds)) != hipSuccess)
        return e;
    Args ai = a;
    ai.l2_ahead = (long long)cus * (per_cu > 0 ? per_cu : 1);
    // stage events: 0 at the start of the chain, 1 at its end, 2 at the end of the intra-chunk kernel
    if ((e = launch_bwd_chain_t<OT, DK, DV>(a, stream, stage_event(a, 0), stage_event(a, 1))) != hipSuccess) return e;
    hipExtLaunchKernelGGL(intra, dim3((unsigned)a.NC), dim3(64 * BWD_NW), lds, stream, nullptr, stage_event(a, 2),
                          0, ai);
    return hipGetLastError();
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
