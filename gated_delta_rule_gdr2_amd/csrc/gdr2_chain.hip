// The two sequential state chains of the Gated Delta Rule-2 operator on gfx950.
//
// Only the state is carried between chunks (digg thread post 9/; anthology
// record LIT-802, takeaway 2), so each (sequence, 16-column slice of the value
// axis) is an independent chain over the chunks:
//
//   forward  : Delta = U - Wm S ;  O^T = S^T Qg^T + Delta^T M^T ;
//              S' = diag(exp gam_C) S + Kd^T Delta
//   backward : dDelta = M^T dO + Kd dS' ; dY = T^T dDelta ;
//              dS = diag(exp gam_C) dS' + Qg^T dO - Wm^T dDelta
//
// One workgroup per chain: NW = d_k / 32 compute waves and NP = 2 producer waves.
//
// Compute waves split the key axis of the state. Wave w keeps rows 32w .. 32w + 31
// of the state slice in MFMA accumulator registers, in fp32, for the whole walk
// (see the K-slot convention in gdr2_device.hpp). What the products need of the
// state is its operand-type copy: at the end of every step each wave publishes its
// rows as one MFMA fragment in LDS (two alternating copies), and after the step's
// barrier every wave has the whole slice as operands. Each wave then forms all four
// token tiles of Delta (or dDelta) itself -- the contraction over the key axis is
// repeated in every wave, which costs MFMA issue slots but no exchange and no second
// barrier -- and uses them, still in registers, to update its own rows and to finish
// its own token tiles of the outputs. One barrier per chunk step.
//
// The producer waves stream the per-chunk operands (swizzled tiles written by the
// intra-chunk kernels) into LDS with asynchronous global->LDS DMA, 16 bytes per
// lane, into two buffers (two waves move about 1.5x the bytes per cycle of one):
// the operands of chunk n + 1 are fetched during step n, into the buffer that step
// n - 1 used, and waited for before the barrier that opens step n + 1. The compute
// waves issue no DMA, so their LDS reads never wait for the transfers in flight.
// Most of these operands were written long before and are no longer in L2, so the
// producers also pull the operands of the chunk PFD steps ahead into L2, with 4-byte
// DMAs (one cache line per lane) into a scratch word of LDS; the NJ workgroups of a
// sequence, which share one XCD's L2, split those lines between them.
//
// Chunk-parallel scan. The chunk transition is affine in the state, S' = P_c S + H_c
// with P_c = diag(exp gam_C) - Kd^T Wm and H_c = Kd^T U, so a sequence's chunks can be
// cut into NSEG segments that are walked at the same time: (1) a summary walk of every
// segment but the last, from a zero start (segment 0: from h0), gives its end state H,
// and a walk whose state starts as the identity and whose value input is zero gives its
// transition P (the product of its P_c); (2) a scan over the segments gives each
// segment's true start state, X_{k+1} = P_k X_k + H_k; (3) every segment is walked
// again from its true start, with all outputs. The backward mirrors it in reverse with
// P_k^T: summaries of the start-state gradient from a zero end gradient (the last
// segment: from dht), a reverse scan, and the full walks.
#include "gdr2_device.hpp"
#include "gdr2_kernels.hpp"

namespace gdr2 {

// this wave's index in the workgroup, as a wave-uniform (scalar) value
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

constexpr int NP = 2;  // producer waves per workgroup

// Producer pi's share of a copy of BYTES (a multiple of 1024) from global memory into
// LDS, 16 bytes per lane: the 1 KB pieces pi, pi + NP, ... (one DMA instruction each).
template <int BYTES>
__device__ __forceinline__ void dma16(const void* src, lds_char* dst, int pi) {
    static_assert(BYTES % 1024 == 0, "16-byte DMA copies whole 1 KB pieces");
    constexpr int P = BYTES / 1024;
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < (P + NP - 1) / NP; ++i) {
        const int k = i * NP + pi;
        if (P % NP == 0 || k < P)
            __builtin_amdgcn_global_load_lds((const char*)src + k * 1024 + l * 16, (lds_void*)(dst + k * 1024), 16,
                                             0, 0);
    }
}
// Producer pi's share of a copy of BYTES (a multiple of 256), 4 bytes per lane.
template <int BYTES>
__device__ __forceinline__ void dma4(const void* src, lds_char* dst, int pi) {
    static_assert(BYTES % 256 == 0, "4-byte DMA copies whole 256-byte pieces");
    constexpr int P = BYTES / 256;
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < (P + NP - 1) / NP; ++i) {
        const int k = i * NP + pi;
        if (P % NP == 0 || k < P)
            __builtin_amdgcn_global_load_lds((const char*)src + k * 256 + l * 4, (lds_void*)(dst + k * 256), 4, 0,
                                             0);
    }
}

// Sequence/slice mapping. Workgroups go to the 8 XCDs round-robin (XCD = id % 8);
// when the sequence count allows, all slices of one sequence share an XCD and
// hence its L2, from which they all read the same per-chunk operands.
__device__ __forceinline__ void chain_map(int gid, int NS, int NJ, int& s, int& j) {
    if (NS % 8 == 0) {
        const int x = gid % 8, rest = gid / 8;
        j = rest % NJ;
        s = (rest / NJ) * 8 + x;
    } else {
        s = gid / NJ;
        j = gid % NJ;
    }
}

// One walk of a chain over the chunks c0 .. c0 + n - 1 of a sequence (the backward walks
// them in reverse). Its state slice is the columns col .. col + 15 of the start and end
// matrices (row strides ld_start, ld_end).
struct WalkSpec {
    int c0, n;
    const float* start;  // start matrix, or null: start from zero
    int ld_start;
    bool ident;          // start from the identity instead (a transition walk)
    float* end;          // where the end state goes, or null
    int ld_end;
    int col;
    bool noU;            // no value input, U = 0 (a transition walk)
};

// Store of one wave's 32 state rows of a 16-column slice, transposed through LDS so
// each lane stores whole 16-byte row pieces.
template <class OT>
struct RowStore {
    static constexpr int LDSP = 16 + 16 / (int)sizeof(OT);             // staging pitch, rows 16-B aligned
    static constexpr int PER_LANE = 32 * 16 * (int)sizeof(OT) / 16 / 64;  // 16-byte pieces per lane
    static constexpr int BYTES = 32 * LDSP * (int)sizeof(OT);           // per wave
    static constexpr int EPP = 16 / (int)sizeof(OT);                    // elements per piece
    static constexpr int PPR = 16 / EPP;                                // pieces per row
};
// s0 / s1: accumulator tiles of rows 0..15 / 16..31; piece p = lane + 64 k covers row
// p / PPR, columns (p % PPR) * EPP .. + EPP - 1
template <class OT>
__device__ __forceinline__ void stage_rows(lds_char* stage, const f32x4& s0, const f32x4& s1,
                                           f32x4 (&pend)[RowStore<OT>::PER_LANE]) {
    typedef __attribute__((address_space(3))) OT TE;
    TE* st = (TE*)stage;
    using R = RowStore<OT>;
    const int l = lane_id(), li = l & 15, lq = l >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        st[(4 * lq + i) * R::LDSP + li] = to_ot<OT>(s0[i]);
        st[(16 + 4 * lq + i) * R::LDSP + li] = to_ot<OT>(s1[i]);
    }
#pragma unroll
    for (int k = 0; k < R::PER_LANE; ++k) {
        const int p = l + 64 * k, row = p / R::PPR, col = (p % R::PPR) * R::EPP;
        pend[k] = lds_load<f32x4>(stage + (row * R::LDSP + col) * (int)sizeof(OT));
    }
}
// ... into a [DK][DV] state in fragment-major layout (fmaj_off), where each piece is
// contiguous and a wave's pieces form whole 512-byte runs
template <class OT, int DV>
__device__ __forceinline__ void store_rows(OT* dst, int row0, int j, const f32x4 (&pend)[RowStore<OT>::PER_LANE]) {
    using R = RowStore<OT>;
    const int l = lane_id();
#pragma unroll
    for (int k = 0; k < R::PER_LANE; ++k) {
        const int p = l + 64 * k, row = p / R::PPR, col = (p % R::PPR) * R::EPP;
        *(f32x4*)(dst + fmaj_off<DV>(row0 + row, 16 * j + col)) = pend[k];
    }
}

// Exchange area in LDS: two alternating copies of the state blocks, in the operand
// type; slot w of a copy holds wave w's 32 state rows as one MFMA fragment
// (64 lanes x 8 elements).
template <class OT>
struct Xch {
    static constexpr int FRAG = 64 * 8 * (int)sizeof(OT);
    static constexpr int bytes(int nw) { return 2 * nw * FRAG; }
};
template <class OT>
__device__ __forceinline__ void put_block(lds_char* xs, int w, const f32x4& s0, const f32x4& s1) {
    using FT = typename Frag<OT>::type;
    lds_store<FT>(xs + w * Xch<OT>::FRAG + lane_id() * 8 * (int)sizeof(OT), frag_of<OT>(s0, s1));
}
template <class OT>
__device__ __forceinline__ typename Frag<OT>::type get_block(const lds_char* xs, int w) {
    using FT = typename Frag<OT>::type;
    return lds_load<FT>(xs + w * Xch<OT>::FRAG + lane_id() * 8 * (int)sizeof(OT));
}

constexpr int LDS_LIMIT = 160 * 1024;

constexpr int PFD = 4;  // L2 prefetch distance in chunk steps

// L2 prefetch of one chunk's operands: the lines of a list of regions are numbered
// 0 .. LINES - 1 in order; workgroup j of NJ, producer pi touches lines
// (( i * NP + pi) * 64 + lane) * NJ + j, i < NPF (lines past the end repeat the last).
// line(v) returns the address of line v. NPF DMA instructions, always.
template <int LINES, int NJ, class FL>
__device__ __forceinline__ void prefetch_lines(FL line, int j, int pi, lds_char* slot) {
    constexpr int NPF = (LINES + NJ * 64 * NP - 1) / (NJ * 64 * NP);
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
        int v = ((i * NP + pi) * 64 + l) * NJ + j;
        v = v < LINES ? v : LINES - 1;
        __builtin_amdgcn_global_load_lds(line(v), (lds_void*)slot, 4, 0, 0);
    }
}
template <int LINES, int NJ>
constexpr int prefetch_count() { return (LINES + NJ * 64 * NP - 1) / (NJ * 64 * NP); }

// A producer's side of a walk over NT chunks (walk index n = 0 .. NT - 1). G(n, buf)
// issues its share of the DMA of all operands of the chunk at walk index n; PF(n)
// issues the NPF prefetch DMAs for the chunk at walk index min(n, NT - 1). Two
// buffers: one barrier per step, as the compute waves have it (A_n opens step n).
// One buffer: a second barrier C_n closes every step, and the transfers do not
// overlap compute.
template <bool DBUF, int NPF, class FG, class FP>
__device__ __forceinline__ void produce(int NT, lds_char* b0, lds_char* b1, FG G, FP PF) {
    if (DBUF) {
        G(0, b0);
        wait_vm<0>();
        for (int n = 0; n < NT; n += 2) {
            sync_lds();  // A_n: chunk n is in b0; b1 is free (step n - 1 is over)
            if (n + 1 < NT) {
                G(n + 1, b1);
                PF(n + PFD);
                wait_vm<NPF>();
            }
            if (n + 1 >= NT) break;
            sync_lds();  // A_{n+1}: chunk n + 1 is in b1; b0 is free
            if (n + 2 < NT) {
                G(n + 2, b0);
                PF(n + 1 + PFD);
                wait_vm<NPF>();
            }
        }
    } else {
        G(0, b0);
        wait_vm<0>();
        (void)PF;
        for (int n = 0; n < NT; ++n) {
            sync_lds();  // A_n
            sync_lds();  // C_n
            if (n + 1 < NT) {
                G(n + 1, b0);
                wait_vm<0>();
            }
        }
    }
}

// ============================================================================ forward chain
template <class OT, int DK, int DV>
struct FwdChainBuf {
    static constexpr int ES = sizeof(OT);
    static constexpr int WM = 0;                  // Wm [64][DK] swizzled
    static constexpr int QG = WM + CH * DK * ES;  // Qg [64][DK]
    static constexpr int U = QG + CH * DK * ES;   // the 4 U tiles of this slice
    static constexpr int KD = U + 4 * 256 * ES;   // Kd [64][DK]
    static constexpr int M = KD + CH * DK * ES;   // M [64][64]
    static constexpr int GC = M + CH * CH * ES;   // exp(gam_C), DK floats
    static constexpr int BYTES = GC + DK * 4;
};

// outputs of one step held by one compute wave until the next step issues them
template <class OT, int NW>
struct FwdPend {
    static constexpr int TPW = 4 / NW;  // token tiles per wave
    f32x4 st[RowStore<OT>::PER_LANE];   // this wave's rows of the chunk start state
    f32x4 D[TPW], O[TPW];               // Delta and O^T tiles wv * TPW + u
    int c;                              // chunk, -1 = nothing pending
};

template <class OT, int DK, int DV, bool TRAIN, bool OUT, int NW>
__device__ __forceinline__ void fwd_flush(const Args& a, int s, int j, FwdPend<OT, NW>& pd) {
    if (pd.c < 0) return;
    constexpr int TPW = FwdPend<OT, NW>::TPW;
    const int l = lane_id(), li = l & 15, lq = l >> 4, wv = wave_id();
    const long long cid = (long long)s * a.NT + pd.c;
    const Layout& L = a.L;
    if (TRAIN) {
        store_rows<OT, DV>((OT*)(a.ws + L.o_s) + cid * L.s, 32 * wv, j, pd.st);
        OT* dl = (OT*)(a.ws + L.o_delta) + cid * L.delta + j * 4 * 256;
#pragma unroll
        for (int u = 0; u < TPW; ++u) store_tile<OT>(dl + (wv * TPW + u) * 256, pd.D[u]);
    }
    if (OUT) {
        const int bidx = s / a.H, h = s % a.H;
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int row = pd.c * CH + 16 * (wv * TPW + u) + li;
            if (row < a.T) {
                float ov[4] = {pd.O[u][0], pd.O[u][1], pd.O[u][2], pd.O[u][3]};
                st4((OT*)a.o + (((size_t)bidx * a.T + row) * a.H + h) * DV + 16 * j + 4 * lq, ov);
            }
        }
    }
}

// One chunk step of a compute wave. On entry the state blocks of all waves are in xr;
// on exit this wave's new block is in xw (the other copy).
template <class OT, int DK, int DV, bool TRAIN, bool OUT, int NW>
__device__ __forceinline__ void fwd_step(int c, const lds_char* buf, f32x4& S0, f32x4& S1, lds_char* stage,
                                         const lds_char* xr, lds_char* xw, FwdPend<OT, NW>& pd, bool noU) {
    using B = FwdChainBuf<OT, DK, DV>;
    using FT = typename Frag<OT>::type;
    constexpr int TPW = FwdPend<OT, NW>::TPW;
    const int l = lane_id(), lq = l >> 4, wv = wave_id();
    const LSwz<OT, DK> vWM{buf + B::WM}, vKD{buf + B::KD}, vQG{buf + B::QG};
    const LSwz<OT, CH> vM{buf + B::M};
    if (TRAIN) stage_rows<OT>(stage, S0, S1, pd.st);  // chunk start state -> pending store
    // Every LDS operand read of the step is issued before the first product (the
    // scheduling fence keeps them together), so the wave waits on LDS latency once.
    FT SB[NW], WM[4][NW], QGf[TPW][NW], Mf[TPW][2], KDf[2][2];
    float uu[4][4], g0[4], g1[4];
#pragma unroll
    for (int kb = 0; kb < NW; ++kb) SB[kb] = get_block<OT>(xr, kb);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int kb = 0; kb < NW; ++kb) WM[t][kb] = lfrag_rowk<OT, OT>(vWM, 16 * t, 32 * kb);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if (noU) {
#pragma unroll
            for (int i = 0; i < 4; ++i) uu[t][i] = 0.f;
        } else {
            lds_get4<OT>(buf + B::U + (t * 256 + l * 4) * (int)sizeof(OT), uu[t]);
        }
    }
    if (OUT) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int t = wv * TPW + u;
#pragma unroll
            for (int kb = 0; kb < NW; ++kb) QGf[u][kb] = lfrag_rowk<OT, OT>(vQG, 16 * t, 32 * kb);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) Mf[u][kb] = lfrag_rowk<OT, OT>(vM, 16 * t, 32 * kb);
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        KDf[0][kb] = lfrag_colk<OT, OT>(vKD, 32 * wv, 32 * kb);
        KDf[1][kb] = lfrag_colk<OT, OT>(vKD, 32 * wv + 16, 32 * kb);
    }
    lds_get4<float>(buf + B::GC + (32 * wv + 4 * lq) * 4, g0);
    lds_get4<float>(buf + B::GC + (32 * wv + 16 + 4 * lq) * 4, g1);
    __builtin_amdgcn_sched_barrier(0);
    // Delta = U - Wm S, all four token tiles
    f32x4 D[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) D[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NW; ++kb)
#pragma unroll
        for (int t = 0; t < 4; ++t) mma(D[t], WM[t][kb], SB[kb]);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) D[t][i] = uu[t][i] - D[t][i];
    FT DB[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) DB[kb] = frag_of<OT>(D[2 * kb], D[2 * kb + 1]);
    // O^T = S^T Qg^T + Delta^T M^T on this wave's token tiles
    if (OUT) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            f32x4 po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NW; ++kb) mma(po, SB[kb], QGf[u][kb]);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) mma(po, DB[kb], Mf[u][kb]);
            pd.O[u] = po;
        }
    }
    // S' = diag(exp gam_C) S + Kd^T Delta on this wave's rows
    {
        f32x4 a0 = {g0[0] * S0[0], g0[1] * S0[1], g0[2] * S0[2], g0[3] * S0[3]};
        f32x4 a1 = {g1[0] * S1[0], g1[1] * S1[1], g1[2] * S1[2], g1[3] * S1[3]};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            mma(a0, KDf[0][kb], DB[kb]);
            mma(a1, KDf[1][kb], DB[kb]);
        }
        S0 = a0;
        S1 = a1;
    }
    put_block<OT>(xw, wv, S0, S1);
#pragma unroll
    for (int u = 0; u < TPW; ++u) pd.D[u] = D[wv * TPW + u];
    pd.c = c;
}

template <class OT, int DK, int DV, bool TRAIN, bool OUT, int NW, bool DBUF>
__device__ __forceinline__ void fwd_walk(const Args& a, int s, int j, const WalkSpec& w, lds_char* b0, lds_char* b1,
                                         lds_char* xs, lds_char* stage_base, lds_char* pfslot) {
    using B = FwdChainBuf<OT, DK, DV>;
    const int wv = wave_id();
    const int NT = w.n;
    const long long base = (long long)s * a.NT + w.c0;
    if (wv >= NW) {  // producer
        const Layout& L = a.L;
        const int pi = wv - NW;
        auto G = [&](int n, lds_char* buf) {
            const long long cid = base + n;
            dma16<CH * DK * sizeof(OT)>(a.ws + L.o_wm + cid * L.wm * sizeof(OT), buf + B::WM, pi);
            dma16<CH * DK * sizeof(OT)>(a.ws + L.o_kd + cid * L.kd * sizeof(OT), buf + B::KD, pi);
            if (OUT) {
                dma16<CH * DK * sizeof(OT)>(a.ws + L.o_qg + cid * L.qg * sizeof(OT), buf + B::QG, pi);
                dma16<CH * CH * sizeof(OT)>(a.ws + L.o_m + cid * L.m * sizeof(OT), buf + B::M, pi);
            }
            if (!w.noU)
                dma16<4 * 256 * sizeof(OT)>(a.ws + L.o_u + (cid * L.u + (size_t)j * 4 * 256) * sizeof(OT),
                                            buf + B::U, pi);
            dma4<DK * 4>(a.ws + L.o_gc + cid * L.gc * 4, buf + B::GC, pi);
        };
        // prefetch regions: Wm, Kd, U (all slices), exp(gam_C) [, Qg, M]
        constexpr int LK = CH * DK * (int)sizeof(OT) / 128, LU = CH * DV * (int)sizeof(OT) / 128;
        constexpr int LM = CH * CH * (int)sizeof(OT) / 128, LG = DK * 4 / 128;
        constexpr int LINES = 2 * LK + LU + LG + (OUT ? LK + LM : 0);
        constexpr int NJ = DV / 16;
        auto PF = [&](int n) {
            const long long cid = base + (n < NT ? n : NT - 1);
            const char* wm = a.ws + L.o_wm + cid * L.wm * sizeof(OT);
            const char* kd = a.ws + L.o_kd + cid * L.kd * sizeof(OT);
            const char* u = a.ws + L.o_u + cid * L.u * sizeof(OT);
            const char* gc = a.ws + L.o_gc + cid * L.gc * 4;
            const char* qg = a.ws + L.o_qg + cid * L.qg * sizeof(OT);
            const char* m = a.ws + L.o_m + cid * L.m * sizeof(OT);
            auto line = [&](int v) -> const char* {
                if (v < LK) return wm + v * 128;
                v -= LK;
                if (v < LK) return kd + v * 128;
                v -= LK;
                if (v < LU) return u + v * 128;
                v -= LU;
                if (v < LG) return gc + v * 128;
                v -= LG;
                if (v < LK) return qg + v * 128;
                return m + (v - LK) * 128;
            };
            prefetch_lines<LINES, NJ>(line, j % NJ, pi, pfslot);
        };
        produce<DBUF, prefetch_count<LINES, NJ>()>(NT, b0, b1, G, PF);
        return;
    }
    // compute waves: state rows 32 wv + 4 lq + i (S0) and 32 wv + 16 + 4 lq + i (S1),
    // column w.col + li
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    lds_char* stage = stage_base + wv * RowStore<OT>::BYTES;
    const int row0 = 32 * wv + 4 * lq, col = w.col + li;
    f32x4 S0, S1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (w.ident) {
            S0[i] = row0 + i == col ? 1.f : 0.f;
            S1[i] = row0 + 16 + i == col ? 1.f : 0.f;
        } else {
            S0[i] = w.start ? w.start[(size_t)(row0 + i) * w.ld_start + col] : 0.f;
            S1[i] = w.start ? w.start[(size_t)(row0 + 16 + i) * w.ld_start + col] : 0.f;
        }
    }
    lds_char* xs0 = xs;
    lds_char* xs1 = xs + NW * Xch<OT>::FRAG;
    put_block<OT>(xs0, wv, S0, S1);
    FwdPend<OT, NW> pd;
    pd.c = -1;
    const int c0 = w.c0;
    if (DBUF) {
        for (int n = 0; n < NT; n += 2) {
            sync_lds();  // A_n
            fwd_flush<OT, DK, DV, TRAIN, OUT, NW>(a, s, j, pd);
            fwd_step<OT, DK, DV, TRAIN, OUT, NW>(c0 + n, b0, S0, S1, stage, xs0, xs1, pd, w.noU);
            if (n + 1 >= NT) break;
            sync_lds();  // A_{n+1}
            fwd_flush<OT, DK, DV, TRAIN, OUT, NW>(a, s, j, pd);
            fwd_step<OT, DK, DV, TRAIN, OUT, NW>(c0 + n + 1, b1, S0, S1, stage, xs1, xs0, pd, w.noU);
        }
    } else {
        for (int n = 0; n < NT; ++n) {
            sync_lds();  // A_n
            fwd_flush<OT, DK, DV, TRAIN, OUT, NW>(a, s, j, pd);
            fwd_step<OT, DK, DV, TRAIN, OUT, NW>(c0 + n, b0, S0, S1, stage, (n & 1) ? xs1 : xs0,
                                                 (n & 1) ? xs0 : xs1, pd, w.noU);
            sync_lds();  // C_n
        }
    }
    fwd_flush<OT, DK, DV, TRAIN, OUT, NW>(a, s, j, pd);
    if (w.end) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w.end[(size_t)(row0 + i) * w.ld_end + col] = S0[i];
            w.end[(size_t)(row0 + 16 + i) * w.ld_end + col] = S1[i];
        }
    }
}

template <class OT, int DK, int DV, bool TRAIN>
__global__ __launch_bounds__(64 * (DK / 32 + NP)) void k_fwd_chain(Args a) {
    using B = FwdChainBuf<OT, DK, DV>;
    constexpr int NW = DK / 32, NJ = DV / 16;
    constexpr int XBYTES = Xch<OT>::bytes(NW);
    constexpr int SBYTES = NW * RowStore<OT>::BYTES;
    constexpr bool DBUF = 2 * B::BYTES + XBYTES + SBYTES + 256 <= LDS_LIMIT;
    __shared__ __align__(16) char buf0[B::BYTES];
    __shared__ __align__(16) char buf1[DBUF ? B::BYTES : 16];
    __shared__ __align__(16) char xch[XBYTES];
    __shared__ __align__(16) char stage[SBYTES];
    __shared__ __align__(16) char pfslot[256];  // target of the L2 prefetch DMAs, never read
    // one walk per (sequence, segment, slice), with all outputs
    const int NSEG = a.nseg;
    int u, j;
    chain_map(blockIdx.x, a.B * a.H * NSEG, NJ, u, j);
    const int s = u / NSEG, seg = u % NSEG;
    const Layout& L = a.L;
    const size_t sq = (size_t)DK * DV;
    WalkSpec w;
    w.c0 = seg * a.seg_len;
    w.n = min(a.seg_len, a.NT - w.c0);
    w.start = seg == 0 ? (a.h0 ? a.h0 + s * sq : nullptr)
                       : (const float*)(a.ws + L.o_segx) + ((size_t)s * NSEG + seg) * L.segx;
    w.ld_start = DV;
    w.ident = false;
    w.end = (seg == NSEG - 1 && a.ht) ? a.ht + s * sq : nullptr;
    w.ld_end = DV;
    w.col = 16 * j;
    w.noU = false;
    if (a.o)
        fwd_walk<OT, DK, DV, TRAIN, true, NW, DBUF>(a, s, j, w, (lds_char*)buf0, (lds_char*)buf1, (lds_char*)xch,
                                                    (lds_char*)stage, (lds_char*)pfslot);
    else
        fwd_walk<OT, DK, DV, TRAIN, false, NW, DBUF>(a, s, j, w, (lds_char*)buf0, (lds_char*)buf1, (lds_char*)xch,
                                                     (lds_char*)stage, (lds_char*)pfslot);
}

// Summary walks of the chunk-parallel scan, one per (sequence, segment k < NSEG - 1,
// slice): value slices j < DV / 16 walk from a zero start (segment 0: from h0) and write
// the segment's end state H_k; transition slices j >= DV / 16 walk the identity's
// columns with no value input and write P_k (not needed, and not run, for segment 0).
template <class OT, int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 32 + NP)) void k_fwd_chain_sum(Args a) {
    using B = FwdChainBuf<OT, DK, DV>;
    constexpr int NW = DK / 32, NJ = DV / 16, NJP = DK / 16;
    constexpr int XBYTES = Xch<OT>::bytes(NW);
    constexpr bool DBUF = 2 * B::BYTES + XBYTES + 256 <= LDS_LIMIT;
    __shared__ __align__(16) char buf0[B::BYTES];
    __shared__ __align__(16) char buf1[DBUF ? B::BYTES : 16];
    __shared__ __align__(16) char xch[XBYTES];
    __shared__ __align__(16) char pfslot[256];  // target of the L2 prefetch DMAs, never read
    const int NSEG = a.nseg;
    int u, j;
    chain_map(blockIdx.x, a.B * a.H * (NSEG - 1), NJ + NJP, u, j);
    const int s = u / (NSEG - 1), seg = u % (NSEG - 1);
    const bool trans = j >= NJ;
    if (trans && seg == 0) return;  // the whole workgroup: segment 0 needs no transition
    const Layout& L = a.L;
    const size_t sub = (size_t)s * NSEG + seg;
    WalkSpec w;
    w.c0 = seg * a.seg_len;
    w.n = a.seg_len;  // every segment but the last is full
    w.ident = trans;
    w.start = (!trans && seg == 0 && a.h0) ? a.h0 + (size_t)s * DK * DV : nullptr;
    w.ld_start = DV;
    w.end = trans ? (float*)(a.ws + L.o_segp) + sub * L.segp : (float*)(a.ws + L.o_segh) + sub * L.segh;
    w.ld_end = trans ? DK : DV;
    w.col = 16 * (trans ? j - NJ : j);
    w.noU = trans;
    fwd_walk<OT, DK, DV, false, false, NW, DBUF>(a, s, j, w, (lds_char*)buf0, (lds_char*)buf1, (lds_char*)xch,
                                                 nullptr, (lds_char*)pfslot);
}

// ============================================================================ backward chain
template <class OT, int DK, int DV>
struct BwdChainBuf {
    static constexpr int ES = sizeof(OT);
    static constexpr int KD = 0;                  // Kd [64][DK] swizzled
    static constexpr int M = KD + CH * DK * ES;   // M [64][64]
    static constexpr int DO = M + CH * CH * ES;   // dO rows of this slice [64][16]
    static constexpr int WM = DO + 64 * 16 * ES;  // Wm [64][DK]
    static constexpr int QG = WM + CH * DK * ES;  // Qg [64][DK]
    static constexpr int T = QG + CH * DK * ES;   // T [64][64]
    static constexpr int GC = T + CH * CH * ES;   // exp(gam_C), DK floats
    static constexpr int BYTES = GC + DK * 4;
};

template <class OT, int NW>
struct BwdPend {
    static constexpr int TPW = 4 / NW;
    f32x4 st[RowStore<OT>::PER_LANE];  // this wave's rows of the end-state gradient
    f32x4 Y[TPW];                      // dY tiles wv * TPW + u
    int c;
};

template <class OT, int DK, int DV, int NW>
__device__ __forceinline__ void bwd_flush(const Args& a, int s, int j, BwdPend<OT, NW>& pd) {
    if (pd.c < 0) return;
    constexpr int TPW = BwdPend<OT, NW>::TPW;
    const int wv = wave_id();
    const long long cid = (long long)s * a.NT + pd.c;
    const Layout& L = a.L;
    store_rows<OT, DV>((OT*)(a.ws + L.o_ds) + cid * L.ds, 32 * wv, j, pd.st);
    OT* dy = (OT*)(a.ws + L.o_dy) + cid * L.dy + j * 4 * 256;
#pragma unroll
    for (int u = 0; u < TPW; ++u) store_tile<OT>(dy + (wv * TPW + u) * 256, pd.Y[u]);
}

// One chunk step of a compute wave. On entry the gradient blocks of all waves are in
// xr; on exit this wave's new block is in xw (the other copy).
// SUM: a summary walk -- only the state gradient, no per-chunk outputs.
template <class OT, int DK, int DV, int NW, bool SUM>
__device__ __forceinline__ void bwd_step(int c, const lds_char* buf, f32x4& dS0, f32x4& dS1, lds_char* stage,
                                         const lds_char* xr, lds_char* xw, BwdPend<OT, NW>& pd) {
    using B = BwdChainBuf<OT, DK, DV>;
    using FT = typename Frag<OT>::type;
    constexpr int TPW = BwdPend<OT, NW>::TPW;
    const int l = lane_id(), lq = l >> 4, wv = wave_id();
    const LSwz<OT, DK> vKD{buf + B::KD}, vQG{buf + B::QG}, vWM{buf + B::WM};
    const LSwz<OT, CH> vM{buf + B::M}, vT{buf + B::T};
    const LPad<OT> vDO{buf + B::DO, 16};
    if (!SUM) stage_rows<OT>(stage, dS0, dS1, pd.st);  // gradient w.r.t. this chunk's end state
    // Every LDS operand read of the step is issued before the first product (the
    // scheduling fence keeps them together), so the wave waits on LDS latency once.
    FT dSB[NW], KDf[4][NW], Mf[4][2], dOB[2], WMf[2][2], QGf[2][2], Tf[TPW][2];
    float g0[4], g1[4];
#pragma unroll
    for (int kb = 0; kb < NW; ++kb) dSB[kb] = get_block<OT>(xr, kb);
    // B fragments of dO: K = token, N = this slice's 16 value channels
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) dOB[kb] = lfrag_colk<OT, OT>(vDO, 0, 32 * kb);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int kb = 0; kb < NW; ++kb) KDf[t][kb] = lfrag_rowk<OT, OT>(vKD, 16 * t, 32 * kb);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) Mf[t][kb] = lfrag_colk<OT, OT>(vM, 16 * t, 32 * kb);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        WMf[0][kb] = lfrag_colk<OT, OT>(vWM, 32 * wv, 32 * kb);
        WMf[1][kb] = lfrag_colk<OT, OT>(vWM, 32 * wv + 16, 32 * kb);
        QGf[0][kb] = lfrag_colk<OT, OT>(vQG, 32 * wv, 32 * kb);
        QGf[1][kb] = lfrag_colk<OT, OT>(vQG, 32 * wv + 16, 32 * kb);
    }
    if (!SUM) {
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) Tf[u][kb] = lfrag_colk<OT, OT>(vT, 16 * (wv * TPW + u), 32 * kb);
    }
    lds_get4<float>(buf + B::GC + (32 * wv + 4 * lq) * 4, g0);
    lds_get4<float>(buf + B::GC + (32 * wv + 16 + 4 * lq) * 4, g1);
    __builtin_amdgcn_sched_barrier(0);
    // dDelta = M^T dO + Kd dS', all four token tiles
    f32x4 dD[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) dD[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NW; ++kb)
#pragma unroll
        for (int t = 0; t < 4; ++t) mma(dD[t], KDf[t][kb], dSB[kb]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < 4; ++t) mma(dD[t], Mf[t][kb], dOB[kb]);
    FT dDB[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) dDB[kb] = frag_of<OT>(dD[2 * kb], dD[2 * kb + 1]);
    // dS = diag(exp gam_C) dS' + Qg^T dO - Wm^T dDelta on this wave's rows
    {
        f32x4 p0 = {g0[0] * dS0[0], g0[1] * dS0[1], g0[2] * dS0[2], g0[3] * dS0[3]};
        f32x4 p1 = {g1[0] * dS1[0], g1[1] * dS1[1], g1[2] * dS1[2], g1[3] * dS1[3]};
        f32x4 n0 = {0.f, 0.f, 0.f, 0.f}, n1 = n0;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            mma(n0, WMf[0][kb], dDB[kb]);
            mma(n1, WMf[1][kb], dDB[kb]);
            mma(p0, QGf[0][kb], dOB[kb]);
            mma(p1, QGf[1][kb], dOB[kb]);
        }
        dS0 = p0 - n0;
        dS1 = p1 - n1;
    }
    put_block<OT>(xw, wv, dS0, dS1);
    if (SUM) return;
    // dY = T^T dDelta on this wave's token tiles (for the intra-chunk kernel)
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mma(acc, Tf[u][kb], dDB[kb]);
        pd.Y[u] = acc;
    }
    pd.c = c;
}

template <class OT, int DK, int DV, int NW, bool DBUF, bool SUM>
__device__ __forceinline__ void bwd_walk(const Args& a, int s, int j, const WalkSpec& w, lds_char* b0, lds_char* b1,
                                         lds_char* xs, lds_char* stage_base, lds_char* pfslot) {
    using B = BwdChainBuf<OT, DK, DV>;
    const int wv = wave_id();
    const int NT = w.n, last = w.c0 + w.n - 1;  // walk index n is chunk last - n
    const long long base = (long long)s * a.NT;
    if (wv >= NW) {  // producer; walk index n is chunk last - n
        const Layout& L = a.L;
        const int pi = wv - NW;
        const int l = lane_id();
        const int bidx = s / a.H, h = s % a.H;
        constexpr int EPL = 4 / sizeof(OT);           // dO elements per lane and instruction
        constexpr int RPI = 256 / (16 * sizeof(OT));  // dO rows per instruction
        auto G = [&](int n, lds_char* buf) {
            const int c = last - n;
            const long long cid = base + c;
            dma16<CH * DK * sizeof(OT)>(a.ws + L.o_kd + cid * L.kd * sizeof(OT), buf + B::KD, pi);
            dma16<CH * CH * sizeof(OT)>(a.ws + L.o_m + cid * L.m * sizeof(OT), buf + B::M, pi);
            dma16<CH * DK * sizeof(OT)>(a.ws + L.o_wm + cid * L.wm * sizeof(OT), buf + B::WM, pi);
            dma16<CH * DK * sizeof(OT)>(a.ws + L.o_qg + cid * L.qg * sizeof(OT), buf + B::QG, pi);
            if (!SUM) dma16<CH * CH * sizeof(OT)>(a.ws + L.o_t + cid * L.t * sizeof(OT), buf + B::T, pi);
            dma4<DK * 4>(a.ws + L.o_gc + cid * L.gc * 4, buf + B::GC, pi);
            // dO rows of this slice. Rows past the end of the sequence repeat its last row:
            // every product that reads dO (M^T dO, Qg^T dO) multiplies those rows by rows of
            // M and Qg that the intra-chunk kernel wrote as exact zeros.
#pragma unroll
            for (int i = 0; i < 64 / RPI / NP; ++i) {
                const int k = i * NP + pi;
                const int r = k * RPI + l / (16 / EPL);
                const int col = (l % (16 / EPL)) * EPL;
                const int row = min(c * CH + r, a.T - 1);
                const OT* src = (const OT*)a.dout + (((size_t)bidx * a.T + row) * a.H + h) * DV + 16 * j + col;
                __builtin_amdgcn_global_load_lds(src, (lds_void*)(buf + B::DO + k * 256), 4, 0, 0);
            }
        };
        static_assert((64 / RPI) % NP == 0, "the dO rows split evenly over the producers");
        // prefetch regions: Kd, Qg, Wm, M, T, exp(gam_C), dO rows (all slices)
        constexpr int LK = CH * DK * (int)sizeof(OT) / 128, LM = CH * CH * (int)sizeof(OT) / 128;
        constexpr int LG = DK * 4 / 128, LR = DV * (int)sizeof(OT) / 128;  // lines per dO row
        constexpr int LINES = 3 * LK + 2 * LM + LG + CH * LR;
        constexpr int NJ = DV / 16;
        auto PF = [&](int n) {
            const int c = last - (n < NT ? n : NT - 1);
            const long long cid = base + c;
            const char* kd = a.ws + L.o_kd + cid * L.kd * sizeof(OT);
            const char* qg = a.ws + L.o_qg + cid * L.qg * sizeof(OT);
            const char* wm = a.ws + L.o_wm + cid * L.wm * sizeof(OT);
            const char* m = a.ws + L.o_m + cid * L.m * sizeof(OT);
            const char* t = a.ws + L.o_t + cid * L.t * sizeof(OT);
            const char* gc = a.ws + L.o_gc + cid * L.gc * 4;
            auto line = [&](int v) -> const char* {
                if (v < LK) return kd + v * 128;
                v -= LK;
                if (v < LK) return qg + v * 128;
                v -= LK;
                if (v < LK) return wm + v * 128;
                v -= LK;
                if (v < LM) return m + v * 128;
                v -= LM;
                if (v < LM) return t + v * 128;
                v -= LM;
                if (v < LG) return gc + v * 128;
                v -= LG;
                const int row = min(c * CH + v / LR, a.T - 1);
                return (const char*)a.dout + ((((size_t)bidx * a.T + row) * a.H + h) * DV) * sizeof(OT) +
                       (v % LR) * 128;
            };
            prefetch_lines<LINES, NJ>(line, j, pi, pfslot);
        };
        produce<DBUF, prefetch_count<LINES, NJ>()>(NT, b0, b1, G, PF);
        return;
    }
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    lds_char* stage = stage_base + wv * RowStore<OT>::BYTES;
    const int row0 = 32 * wv + 4 * lq, col = w.col + li;
    f32x4 dS0, dS1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dS0[i] = w.start ? w.start[(size_t)(row0 + i) * w.ld_start + col] : 0.f;
        dS1[i] = w.start ? w.start[(size_t)(row0 + 16 + i) * w.ld_start + col] : 0.f;
    }
    lds_char* xs0 = xs;
    lds_char* xs1 = xs + NW * Xch<OT>::FRAG;
    put_block<OT>(xs0, wv, dS0, dS1);
    BwdPend<OT, NW> pd;
    pd.c = -1;
    if (DBUF) {
        for (int n = 0; n < NT; n += 2) {
            sync_lds();  // A_n
            bwd_flush<OT, DK, DV, NW>(a, s, j, pd);
            bwd_step<OT, DK, DV, NW, SUM>(last - n, b0, dS0, dS1, stage, xs0, xs1, pd);
            if (n + 1 >= NT) break;
            sync_lds();  // A_{n+1}
            bwd_flush<OT, DK, DV, NW>(a, s, j, pd);
            bwd_step<OT, DK, DV, NW, SUM>(last - n - 1, b1, dS0, dS1, stage, xs1, xs0, pd);
        }
    } else {
        for (int n = 0; n < NT; ++n) {
            sync_lds();  // A_n
            bwd_flush<OT, DK, DV, NW>(a, s, j, pd);
            bwd_step<OT, DK, DV, NW, SUM>(last - n, b0, dS0, dS1, stage, (n & 1) ? xs1 : xs0, (n & 1) ? xs0 : xs1,
                                          pd);
            sync_lds();  // C_n
        }
    }
    bwd_flush<OT, DK, DV, NW>(a, s, j, pd);
    if (w.end) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w.end[(size_t)(row0 + i) * w.ld_end + col] = dS0[i];
            w.end[(size_t)(row0 + 16 + i) * w.ld_end + col] = dS1[i];
        }
    }
}

template <class OT, int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 32 + NP)) void k_bwd_chain(Args a) {
    using B = BwdChainBuf<OT, DK, DV>;
    constexpr int NW = DK / 32, NJ = DV / 16;
    constexpr int XBYTES = Xch<OT>::bytes(NW);
    constexpr int SBYTES = NW * RowStore<OT>::BYTES;
    constexpr bool DBUF = 2 * B::BYTES + XBYTES + SBYTES + 256 <= LDS_LIMIT;
    __shared__ __align__(16) char buf0[B::BYTES];
    __shared__ __align__(16) char buf1[DBUF ? B::BYTES : 16];
    __shared__ __align__(16) char xch[XBYTES];
    __shared__ __align__(16) char stage[SBYTES];
    __shared__ __align__(16) char pfslot[256];  // target of the L2 prefetch DMAs, never read
    // one walk per (sequence, segment, slice), with all outputs
    const int NSEG = a.nseg;
    int u, j;
    chain_map(blockIdx.x, a.B * a.H * NSEG, NJ, u, j);
    const int s = u / NSEG, seg = u % NSEG;
    const Layout& L = a.L;
    const size_t sq = (size_t)DK * DV;
    WalkSpec w;
    w.c0 = seg * a.seg_len;
    w.n = min(a.seg_len, a.NT - w.c0);
    w.start = seg == NSEG - 1 ? (a.dht ? a.dht + s * sq : nullptr)
                              : (const float*)(a.ws + L.o_segx) + ((size_t)s * NSEG + seg) * L.segx;
    w.ld_start = DV;
    w.ident = false;
    w.end = (seg == 0 && a.dh0) ? a.dh0 + s * sq : nullptr;
    w.ld_end = DV;
    w.col = 16 * j;
    w.noU = false;
    bwd_walk<OT, DK, DV, NW, DBUF, false>(a, s, j, w, (lds_char*)buf0, (lds_char*)buf1, (lds_char*)xch,
                                          (lds_char*)stage, (lds_char*)pfslot);
}

// Summary walks of the backward scan, one per (sequence, segment k >= 1, slice): the
// gradient with respect to the segment's start state when the gradient at its end is
// zero (the last segment: dht), into the summary array.
template <class OT, int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 32 + NP)) void k_bwd_chain_sum(Args a) {
    using B = BwdChainBuf<OT, DK, DV>;
    constexpr int NW = DK / 32, NJ = DV / 16;
    constexpr int XBYTES = Xch<OT>::bytes(NW);
    constexpr bool DBUF = 2 * B::BYTES + XBYTES + 256 <= LDS_LIMIT;
    __shared__ __align__(16) char buf0[B::BYTES];
    __shared__ __align__(16) char buf1[DBUF ? B::BYTES : 16];
    __shared__ __align__(16) char xch[XBYTES];
    __shared__ __align__(16) char pfslot[256];  // target of the L2 prefetch DMAs, never read
    const int NSEG = a.nseg;
    int u, j;
    chain_map(blockIdx.x, a.B * a.H * (NSEG - 1), NJ, u, j);
    const int s = u / (NSEG - 1), seg = 1 + u % (NSEG - 1);
    const Layout& L = a.L;
    WalkSpec w;
    w.c0 = seg * a.seg_len;
    w.n = min(a.seg_len, a.NT - w.c0);
    w.start = (seg == NSEG - 1 && a.dht) ? a.dht + (size_t)s * DK * DV : nullptr;
    w.ld_start = DV;
    w.ident = false;
    w.end = (float*)(a.ws + L.o_segh) + ((size_t)s * NSEG + seg) * L.segh;
    w.ld_end = DV;
    w.col = 16 * j;
    w.noU = false;
    bwd_walk<OT, DK, DV, NW, DBUF, true>(a, s, j, w, (lds_char*)buf0, (lds_char*)buf1, (lds_char*)xch, nullptr,
                                         (lds_char*)pfslot);
}

// Scan over the segments of one (sequence, 16-column slice), in fp32. Forward: the true
// start states X_1 = H_0, X_{k+1} = P_k X_k + H_k. Backward: the true end-state
// gradients X_{NSEG-2} = H_{NSEG-1}, X_{k-1} = P_k^T X_k + H_k. P_k is staged in LDS
// (row pitch DK + 1, so the row and the column reads are both free of bank conflicts).
template <int DK, int DV, bool BWD>
__global__ __launch_bounds__(256) void k_seg_scan(Args a) {
    constexpr int NJ = DV / 16, TPR = 256 / DK, CPT = 16 / TPR;  // threads per row, columns per thread
    constexpr int PP = DK + 1;
    extern __shared__ __align__(16) char smem_[];
    float* sP = (float*)smem_;     // [DK][PP]
    float* sx = sP + DK * PP;      // [DK][16]
    const int tid = threadIdx.x;
    const int s = blockIdx.x / NJ, j = blockIdx.x % NJ;
    const int NSEG = a.nseg;
    const Layout& L = a.L;
    const float* P = (const float*)(a.ws + L.o_segp) + (size_t)s * NSEG * L.segp;
    const float* Hm = (const float*)(a.ws + L.o_segh) + (size_t)s * NSEG * L.segh;
    float* X = (float*)(a.ws + L.o_segx) + (size_t)s * NSEG * L.segx;
    const int r = tid / TPR, cl = (tid % TPR) * CPT;  // this thread's row and first column in the slice
    const size_t e0 = (size_t)r * DV + 16 * j + cl;   // its first element in a [DK][DV] matrix
    float x[CPT];
    {
        const int first = BWD ? NSEG - 1 : 0, out = BWD ? NSEG - 2 : 1;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            x[c] = Hm[(size_t)first * L.segh + e0 + c];
            X[(size_t)out * L.segx + e0 + c] = x[c];
        }
    }
    for (int step = 1; step <= NSEG - 2; ++step) {
        const int k = BWD ? NSEG - 1 - step : step;  // the segment whose transition is applied
        const int out = BWD ? k - 1 : k + 1;        // the boundary it gives
        __syncthreads();                            // the previous step is done with sP and sx
#pragma unroll
        for (int c = 0; c < CPT; ++c) sx[r * 16 + cl + c] = x[c];
        const float* Pk = P + (size_t)k * L.segp;
        for (int e = 4 * tid; e < DK * DK; e += 4 * 256) {
            const f32x4 v = *(const f32x4*)(Pk + e);
            const int pr = e / DK, pc = e % DK;
#pragma unroll
            for (int i = 0; i < 4; ++i) sP[pr * PP + pc + i] = v[i];
        }
        __syncthreads();
        float acc[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[c] = Hm[(size_t)k * L.segh + e0 + c];
        for (int i = 0; i < DK; ++i) {
            const float p = BWD ? sP[i * PP + r] : sP[r * PP + i];
#pragma unroll
            for (int c = 0; c < CPT; ++c) acc[c] += p * sx[i * 16 + cl + c];
        }
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            x[c] = acc[c];
            X[(size_t)out * L.segx + e0 + c] = acc[c];
        }
    }
}

template <int DK, int DV, bool BWD>
static hipError_t launch_seg_scan(const Args& a, hipStream_t stream) {  // never first or last of a stage
    const size_t lds = ((size_t)DK * (DK + 1) + DK * 16) * 4;
    hipError_t e = hipFuncSetAttribute((const void*)k_seg_scan<DK, DV, BWD>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_seg_scan<DK, DV, BWD>), dim3((unsigned)(a.B * a.H * (DV / 16))), dim3(256), lds, stream,
                       a);
    return hipGetLastError();
}

// ============================================================================ launchers
template <class OT, int DK, int DV>
hipError_t launch_fwd_chain_t(const Args& a, bool train, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    const unsigned S = (unsigned)(a.B * a.H), NJ = DV / 16, NJP = DK / 16;
    const dim3 block(64 * (DK / 32 + NP));
    hipError_t e;
    if (a.nseg > 1) {
        hipExtLaunchKernelGGL((k_fwd_chain_sum<OT, DK, DV>), dim3(S * (a.nseg - 1) * (NJ + NJP)), block, 0, stream,
                              start, nullptr, 0, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_seg_scan<DK, DV, false>(a, stream)) != hipSuccess) return e;
        start = nullptr;
    }
    const dim3 grid(S * a.nseg * NJ);
    if (train)
        hipExtLaunchKernelGGL((k_fwd_chain<OT, DK, DV, true>), grid, block, 0, stream, start, stop, 0, a);
    else
        hipExtLaunchKernelGGL((k_fwd_chain<OT, DK, DV, false>), grid, block, 0, stream, start, stop, 0, a);
    return hipGetLastError();
}
template <class OT, int DK, int DV>
hipError_t launch_bwd_chain_t(const Args& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    const unsigned S = (unsigned)(a.B * a.H), NJ = DV / 16;
    const dim3 block(64 * (DK / 32 + NP));
    hipError_t e;
    if (a.nseg > 1) {
        hipExtLaunchKernelGGL((k_bwd_chain_sum<OT, DK, DV>), dim3(S * (a.nseg - 1) * NJ), block, 0, stream, start,
                              nullptr, 0, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_seg_scan<DK, DV, true>(a, stream)) != hipSuccess) return e;
        start = nullptr;
    }
    hipExtLaunchKernelGGL((k_bwd_chain<OT, DK, DV>), dim3(S * a.nseg * NJ), block, 0, stream, start, stop, 0, a);
    return hipGetLastError();
}

#define GDR2_CHAIN_INST(OT_, DK_, DV_)                                                      \
    template hipError_t launch_fwd_chain_t<OT_, DK_, DV_>(const Args&, bool, hipStream_t, hipEvent_t, hipEvent_t); \
    template hipError_t launch_bwd_chain_t<OT_, DK_, DV_>(const Args&, hipStream_t, hipEvent_t, hipEvent_t);
GDR2_CHAIN_INST(bf16, 64, 64)
GDR2_CHAIN_INST(bf16, 64, 128)
GDR2_CHAIN_INST(bf16, 128, 64)
GDR2_CHAIN_INST(bf16, 128, 128)
GDR2_CHAIN_INST(float, 64, 64)
#undef GDR2_CHAIN_INST

}  // namespace gdr2
