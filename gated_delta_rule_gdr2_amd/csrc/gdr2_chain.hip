// The two sequential state chains of the Gated Delta Rule-2 operator on gfx950.
//
// Only the state is carried between chunks (digg thread post 9/; anthology
// record LIT-802, takeaway 2), so each (sequence, 16-column slice of the value
// axis) is an independent chain over the chunks: one wave per workgroup.
//
//   forward  : Delta = U - Wm S ;  O^T = S^T Qg^T + Delta^T M^T ;
//              S' = diag(exp gam_C) S + Kd^T Delta
//   backward : dDelta = M^T dO + Kd dS' ; dY = T^T dDelta ;
//              dS = diag(exp gam_C) dS' + Qg^T dO - Wm^T dDelta
//
// The state slice lives in MFMA accumulator registers for the whole walk and
// feeds the next MFMA directly (see the K-slot convention in gdr2_device.hpp).
// Per-chunk operands were written by the intra-chunk kernel as lane-major MFMA
// fragment blocks; the chain streams them into LDS with asynchronous
// global->LDS DMA (16 bytes per lane), double-buffered one chunk ahead, so the
// next chunk's ~60 KB arrive while the current chunk computes. The two buffers
// are distinct LDS objects and the loop is unrolled by two, which lets the
// compiler see that reads of one buffer never alias the DMA into the other.
// Global stores of a step are issued at the start of the following step, so
// the per-step wait for the DMA never waits on them.
#include "gdr2_device.hpp"
#include "gdr2_kernels.hpp"

namespace gdr2 {

// Copy `bytes` (a multiple of 1024) from global memory into LDS, 16 bytes per lane.
__device__ __forceinline__ void dma16(const void* src, lds_char* dst, int bytes) {
    const int l = lane_id();
    for (int k = 0; k < bytes; k += 1024)
        __builtin_amdgcn_global_load_lds((const char*)src + k + l * 16, (lds_void*)(dst + k), 16, 0, 0);
}
// Copy `bytes` (a multiple of 256) 4 bytes per lane.
__device__ __forceinline__ void dma4(const void* src, lds_char* dst, int bytes) {
    const int l = lane_id();
    for (int k = 0; k < bytes; k += 256)
        __builtin_amdgcn_global_load_lds((const char*)src + k + l * 4, (lds_void*)(dst + k), 4, 0, 0);
}
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

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

// Row-major [DK][DV] store of one 16-column slice of a state held as accumulator
// tiles: transposed through LDS so each lane stores whole 16-byte row pieces.
template <class OT, int DK>
struct StateStore {
    static constexpr int LDSP = 16 + 16 / (int)sizeof(OT);              // staging pitch, rows 16-B aligned
    static constexpr int PER_LANE = DK * 16 * (int)sizeof(OT) / 16 / 64;  // 16-byte pieces per lane
    static constexpr int BYTES = DK * LDSP * (int)sizeof(OT);
};

template <class OT, int DK>
__device__ __forceinline__ void stage_state(lds_char* stage_, const f32x4 (&S)[DK / 16]) {
    typedef __attribute__((address_space(3))) OT TE;
    TE* stage = (TE*)stage_;
    constexpr int P = StateStore<OT, DK>::LDSP;
    const int l = lane_id(), li = l & 15, lq = l >> 4;
#pragma unroll
    for (int at = 0; at < DK / 16; ++at)
#pragma unroll
        for (int i = 0; i < 4; ++i) stage[(16 * at + 4 * lq + i) * P + li] = to_ot<OT>(S[at][i]);
}
// read the staged slice back as 16-byte row pieces; piece p = lane + 64 k covers
// row p / PPR, columns (p % PPR) * EPP .. +EPP
template <class OT, int DK>
__device__ __forceinline__ void unstage_state(const lds_char* stage, f32x4 (&pend)[StateStore<OT, DK>::PER_LANE]) {
    typedef __attribute__((address_space(3))) const f32x4 T4;
    constexpr int P = StateStore<OT, DK>::LDSP;
    constexpr int EPP = 16 / sizeof(OT), PPR = 16 / EPP;
    const int l = lane_id();
#pragma unroll
    for (int k = 0; k < StateStore<OT, DK>::PER_LANE; ++k) {
        const int p = l + 64 * k, row = p / PPR, col = (p % PPR) * EPP;
        pend[k] = *(T4*)(stage + (row * P + col) * (int)sizeof(OT));
    }
}
template <class OT, int DK, int DV>
__device__ __forceinline__ void store_state(OT* dst, int j, const f32x4 (&pend)[StateStore<OT, DK>::PER_LANE]) {
    constexpr int EPP = 16 / sizeof(OT), PPR = 16 / EPP;
    const int l = lane_id();
#pragma unroll
    for (int k = 0; k < StateStore<OT, DK>::PER_LANE; ++k) {
        const int p = l + 64 * k, row = p / PPR, col = (p % PPR) * EPP;
        *(f32x4*)(dst + (size_t)row * DV + 16 * j + col) = pend[k];
    }
}

// ============================================================================ forward chain
template <class OT, int DK, int DV>
struct FwdChainBuf {
    static constexpr int ES = sizeof(OT);
    static constexpr int WM = 0;                  // Wm [64][DK] swizzled
    static constexpr int KD = WM + CH * DK * ES;  // Kd [64][DK]
    static constexpr int QG = KD + CH * DK * ES;  // Qg [64][DK]
    static constexpr int M = QG + CH * DK * ES;   // M [64][64]
    static constexpr int U = M + CH * CH * ES;    // 4 U tiles of this slice
    static constexpr int GC = U + 4 * 256 * ES;   // DK floats
    static constexpr int BYTES = GC + DK * 4;
};

template <class OT, int DK, int DV>
__device__ __forceinline__ void fwd_prefetch(const Args& a, long long cid, int j, lds_char* buf) {
    using B = FwdChainBuf<OT, DK, DV>;
    const Layout& L = a.L;
    dma16(a.ws + L.o_wm + cid * L.wm * sizeof(OT), buf + B::WM, CH * DK * sizeof(OT));
    dma16(a.ws + L.o_kd + cid * L.kd * sizeof(OT), buf + B::KD, CH * DK * sizeof(OT));
    if (a.o) {
        dma16(a.ws + L.o_qg + cid * L.qg * sizeof(OT), buf + B::QG, CH * DK * sizeof(OT));
        dma16(a.ws + L.o_m + cid * L.m * sizeof(OT), buf + B::M, CH * CH * sizeof(OT));
    }
    dma16(a.ws + L.o_u + (cid * L.u + (size_t)j * 4 * 256) * sizeof(OT), buf + B::U, 4 * 256 * sizeof(OT));
    dma4(a.ws + L.o_gc + cid * L.gc * 4, buf + B::GC, DK * 4);
}

template <class OT, int DK, int DV, bool TRAIN>
struct FwdPending {
    f32x4 st[StateStore<OT, DK>::PER_LANE];
    f32x4 D[4];
    f32x4 O[4];
    int c;  // chunk these belong to, -1 = nothing pending
};

template <class OT, int DK, int DV, bool TRAIN>
__device__ __forceinline__ void fwd_flush(const Args& a, int s, int j, FwdPending<OT, DK, DV, TRAIN>& pd) {
    if (pd.c < 0) return;
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    const long long cid = (long long)s * a.NT + pd.c;
    const Layout& L = a.L;
    if (TRAIN) {
        store_state<OT, DK, DV>((OT*)(a.ws + L.o_s) + cid * L.s, j, pd.st);
        OT* dl = (OT*)(a.ws + L.o_delta) + cid * L.delta + j * 4 * 256;
#pragma unroll
        for (int t = 0; t < 4; ++t) store_tile<OT>(dl + t * 256, pd.D[t]);
    }
    if (a.o) {
        const int bidx = s / a.H, h = s % a.H;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int row = pd.c * CH + 16 * t + li;
            if (row < a.T) {
                float ov[4] = {pd.O[t][0], pd.O[t][1], pd.O[t][2], pd.O[t][3]};
                st4((OT*)a.o + (((size_t)bidx * a.T + row) * a.H + h) * DV + 16 * j + 4 * lq, ov);
            }
        }
    }
}

template <class OT, int DK, int DV, bool TRAIN>
__device__ __forceinline__ void fwd_step(const Args& a, int c, const lds_char* buf, f32x4 (&S)[DK / 16],
                                         lds_char* stage, FwdPending<OT, DK, DV, TRAIN>& pd) {
    using B = FwdChainBuf<OT, DK, DV>;
    using FT = typename Frag<OT>::type;
    constexpr int KB = DK / 32, AT = DK / 16;
    const int l = lane_id(), lq = l >> 4;
    const LSwz<OT, DK> vWM{buf + B::WM}, vKD{buf + B::KD}, vQG{buf + B::QG};
    const LSwz<OT, CH> vM{buf + B::M};
    if (TRAIN) {  // chunk start state -> pending row-major store
        stage_state<OT, DK>(stage, S);
        unstage_state<OT, DK>(stage, pd.st);
    }
    FT SB[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) SB[kb] = frag_of<OT>(S[2 * kb], S[2 * kb + 1]);
    // Delta = U - Wm S
    f32x4 D[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) mma(acc, lfrag_rowk<OT, OT>(vWM, 16 * t, 32 * kb), SB[kb]);
        float u[4];
        lds_get4<OT>(buf + B::U + (t * 256 + l * 4) * (int)sizeof(OT), u);
        f32x4 uu = {u[0], u[1], u[2], u[3]};
        D[t] = uu - acc;
    }
    FT DB[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) DB[kb] = frag_of<OT>(D[2 * kb], D[2 * kb + 1]);
    // S' = diag(exp gam_C) S + Kd^T Delta
#pragma unroll
    for (int at = 0; at < AT; ++at) {
        float g4[4];
        lds_get4<float>(buf + B::GC + (16 * at + 4 * lq) * 4, g4);
        f32x4 acc = {g4[0] * S[at][0], g4[1] * S[at][1], g4[2] * S[at][2], g4[3] * S[at][3]};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mma(acc, lfrag_colk<OT, OT>(vKD, 16 * at, 32 * kb), DB[kb]);
        S[at] = acc;
    }
    // O^T = S^T Qg^T + Delta^T M^T (uses the chunk start state, still in SB)
    if (a.o) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) mma(acc, SB[kb], lfrag_rowk<OT, OT>(vQG, 16 * t, 32 * kb));
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) mma(acc, DB[kb], lfrag_rowk<OT, OT>(vM, 16 * t, 32 * kb));
            pd.O[t] = acc;
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) pd.D[t] = D[t];
    pd.c = c;
}

constexpr int LDS_LIMIT = 160 * 1024;

template <class OT, int DK, int DV, bool TRAIN>
__global__ __launch_bounds__(64) void k_fwd_chain(Args a) {
    using B = FwdChainBuf<OT, DK, DV>;
    constexpr int AT = DK / 16, NJ = DV / 16;
    constexpr bool DBUF = 2 * B::BYTES + StateStore<OT, DK>::BYTES <= LDS_LIMIT;
    __shared__ __align__(16) char buf0[B::BYTES];
    __shared__ __align__(16) char buf1[DBUF ? B::BYTES : 16];
    __shared__ __align__(16) char stage_[StateStore<OT, DK>::BYTES];
    lds_char* b0 = (lds_char*)buf0;
    lds_char* b1 = (lds_char*)buf1;
    lds_char* stage = (lds_char*)stage_;
    const int l = threadIdx.x, li = l & 15, lq = l >> 4;
    int s, j;
    chain_map(blockIdx.x, a.B * a.H, NJ, s, j);

    f32x4 S[AT];
#pragma unroll
    for (int at = 0; at < AT; ++at)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[at][i] = a.h0 ? a.h0[((size_t)s * DK + 16 * at + 4 * lq + i) * DV + 16 * j + li] : 0.f;
    FwdPending<OT, DK, DV, TRAIN> pd;
    pd.c = -1;
    const long long base = (long long)s * a.NT;
    if (!DBUF) {  // one buffer: fetch, wait, compute
        for (int c = 0; c < a.NT; ++c) {
            fwd_flush<OT, DK, DV, TRAIN>(a, s, j, pd);
            fwd_prefetch<OT, DK, DV>(a, base + c, j, b0);
            wait_vm0();
            fwd_step<OT, DK, DV, TRAIN>(a, c, b0, S, stage, pd);
        }
    } else {
    fwd_prefetch<OT, DK, DV>(a, base, j, b0);
    for (int c = 0; c < a.NT; c += 2) {
        wait_vm0();
        if (c + 1 < a.NT) fwd_prefetch<OT, DK, DV>(a, base + c + 1, j, b1);
        fwd_flush<OT, DK, DV, TRAIN>(a, s, j, pd);
        fwd_step<OT, DK, DV, TRAIN>(a, c, b0, S, stage, pd);
        if (c + 1 >= a.NT) break;
        wait_vm0();
        if (c + 2 < a.NT) fwd_prefetch<OT, DK, DV>(a, base + c + 2, j, b0);
        fwd_flush<OT, DK, DV, TRAIN>(a, s, j, pd);
        fwd_step<OT, DK, DV, TRAIN>(a, c + 1, b1, S, stage, pd);
    }
    }
    fwd_flush<OT, DK, DV, TRAIN>(a, s, j, pd);
    if (a.ht) {
#pragma unroll
        for (int at = 0; at < AT; ++at)
#pragma unroll
            for (int i = 0; i < 4; ++i) a.ht[((size_t)s * DK + 16 * at + 4 * lq + i) * DV + 16 * j + li] = S[at][i];
    }
}

// ============================================================================ backward chain
template <class OT, int DK, int DV>
struct BwdChainBuf {
    static constexpr int ES = sizeof(OT);
    static constexpr int M = 0;                   // M [64][64] swizzled
    static constexpr int KD = M + CH * CH * ES;   // Kd [64][DK]
    static constexpr int QG = KD + CH * DK * ES;  // Qg [64][DK]
    static constexpr int WM = QG + CH * DK * ES;  // Wm [64][DK]
    static constexpr int T = WM + CH * DK * ES;   // T [64][64]
    static constexpr int GC = T + CH * CH * ES;   // DK floats
    static constexpr int DO = GC + DK * 4;        // dO rows [64][16]
    static constexpr int BYTES = DO + 64 * 16 * ES;
};

template <class OT, int DK, int DV>
__device__ __forceinline__ void bwd_prefetch(const Args& a, long long cid, int c, int s, int j, lds_char* buf) {
    using B = BwdChainBuf<OT, DK, DV>;
    const Layout& L = a.L;
    dma16(a.ws + L.o_m + cid * L.m * sizeof(OT), buf + B::M, CH * CH * sizeof(OT));
    dma16(a.ws + L.o_kd + cid * L.kd * sizeof(OT), buf + B::KD, CH * DK * sizeof(OT));
    dma16(a.ws + L.o_qg + cid * L.qg * sizeof(OT), buf + B::QG, CH * DK * sizeof(OT));
    dma16(a.ws + L.o_wm + cid * L.wm * sizeof(OT), buf + B::WM, CH * DK * sizeof(OT));
    dma16(a.ws + L.o_t + cid * L.t * sizeof(OT), buf + B::T, CH * CH * sizeof(OT));
    dma4(a.ws + L.o_gc + cid * L.gc * 4, buf + B::GC, DK * 4);
    // dO rows of this slice: row r, 16 columns; 4 bytes per lane, 256 bytes per instruction
    const int l = lane_id();
    const int bidx = s / a.H, h = s % a.H;
    constexpr int EPL = 4 / sizeof(OT);          // elements per lane-load
    constexpr int RPI = 256 / (16 * sizeof(OT));  // rows per instruction
#pragma unroll
    for (int k = 0; k < 64 / RPI; ++k) {
        const int r = k * RPI + l / (16 / EPL);
        const int col = (l % (16 / EPL)) * EPL;
        const int row = c * CH + r;
        lds_char* dst = buf + B::DO + k * 256;
        if (row < a.T) {
            const OT* src = (const OT*)a.dout + (((size_t)bidx * a.T + row) * a.H + h) * DV + 16 * j + col;
            __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 4, 0, 0);
        } else {
            typedef __attribute__((address_space(3))) uint32_t U32;
            *(U32*)(dst + l * 4) = 0u;
        }
    }
}

template <class OT, int DK>
struct BwdPending {
    f32x4 st[StateStore<OT, DK>::PER_LANE];
    f32x4 Y[4];
    int c;
};

template <class OT, int DK, int DV>
__device__ __forceinline__ void bwd_flush(const Args& a, int s, int j, BwdPending<OT, DK>& pd) {
    if (pd.c < 0) return;
    const long long cid = (long long)s * a.NT + pd.c;
    const Layout& L = a.L;
    store_state<OT, DK, DV>((OT*)(a.ws + L.o_ds) + cid * L.ds, j, pd.st);
    OT* dy = (OT*)(a.ws + L.o_dy) + cid * L.dy + j * 4 * 256;
#pragma unroll
    for (int t = 0; t < 4; ++t) store_tile<OT>(dy + t * 256, pd.Y[t]);
}

template <class OT, int DK, int DV>
__device__ __forceinline__ void bwd_step(int c, const lds_char* buf, f32x4 (&dS)[DK / 16], lds_char* stage,
                                         BwdPending<OT, DK>& pd) {
    using B = BwdChainBuf<OT, DK, DV>;
    using FT = typename Frag<OT>::type;
    constexpr int KB = DK / 32, AT = DK / 16;
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    const LSwz<OT, DK> vKD{buf + B::KD}, vQG{buf + B::QG}, vWM{buf + B::WM};
    const LSwz<OT, CH> vM{buf + B::M}, vT{buf + B::T};
    // gradient w.r.t. this chunk's end state -> pending row-major store
    stage_state<OT, DK>(stage, dS);
    unstage_state<OT, DK>(stage, pd.st);
    // B fragments of dO: K = token, N = this slice's 16 value channels
    FT dOB[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) dOB[kb][e] = lds_load<OT>(buf + B::DO + ((32 * kb + kmap(lq, e)) * 16 + li) * (int)sizeof(OT));
    FT dSB[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) dSB[kb] = frag_of<OT>(dS[2 * kb], dS[2 * kb + 1]);
    // dDelta = M^T dO + Kd dS'
    f32x4 dD[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) mma(acc, lfrag_rowk<OT, OT>(vKD, 16 * t, 32 * kb), dSB[kb]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mma(acc, lfrag_colk<OT, OT>(vM, 16 * t, 32 * kb), dOB[kb]);
        dD[t] = acc;
    }
    FT dDB[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) dDB[kb] = frag_of<OT>(dD[2 * kb], dD[2 * kb + 1]);
    // dS = diag(exp gam_C) dS' + Qg^T dO - Wm^T dDelta
#pragma unroll
    for (int at = 0; at < AT; ++at) {
        float g4[4];
        lds_get4<float>(buf + B::GC + (16 * at + 4 * lq) * 4, g4);
        f32x4 pos = {g4[0] * dS[at][0], g4[1] * dS[at][1], g4[2] * dS[at][2], g4[3] * dS[at][3]};
        f32x4 neg = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            mma(neg, lfrag_colk<OT, OT>(vWM, 16 * at, 32 * kb), dDB[kb]);
            mma(pos, lfrag_colk<OT, OT>(vQG, 16 * at, 32 * kb), dOB[kb]);
        }
        dS[at] = pos - neg;
    }
    // dY = T^T dDelta (for the intra-chunk kernel)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mma(acc, lfrag_colk<OT, OT>(vT, 16 * t, 32 * kb), dDB[kb]);
        pd.Y[t] = acc;
    }
    pd.c = c;
}

template <class OT, int DK, int DV>
__global__ __launch_bounds__(64) void k_bwd_chain(Args a) {
    using B = BwdChainBuf<OT, DK, DV>;
    constexpr int AT = DK / 16, NJ = DV / 16;
    constexpr bool DBUF = 2 * B::BYTES + StateStore<OT, DK>::BYTES <= LDS_LIMIT;
    __shared__ __align__(16) char buf0[B::BYTES];
    __shared__ __align__(16) char buf1[DBUF ? B::BYTES : 16];
    __shared__ __align__(16) char stage_[StateStore<OT, DK>::BYTES];
    lds_char* b0 = (lds_char*)buf0;
    lds_char* b1 = (lds_char*)buf1;
    lds_char* stage = (lds_char*)stage_;
    const int l = threadIdx.x, li = l & 15, lq = l >> 4;
    int s, j;
    chain_map(blockIdx.x, a.B * a.H, NJ, s, j);

    f32x4 dS[AT];
#pragma unroll
    for (int at = 0; at < AT; ++at)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dS[at][i] = a.dht ? a.dht[((size_t)s * DK + 16 * at + 4 * lq + i) * DV + 16 * j + li] : 0.f;
    BwdPending<OT, DK> pd;
    pd.c = -1;
    const long long base = (long long)s * a.NT;
    const int last = a.NT - 1;
    if (!DBUF) {  // one buffer: fetch, wait, compute
        for (int c = last; c >= 0; --c) {
            bwd_flush<OT, DK, DV>(a, s, j, pd);
            bwd_prefetch<OT, DK, DV>(a, base + c, c, s, j, b0);
            wait_vm0();
            bwd_step<OT, DK, DV>(c, b0, dS, stage, pd);
        }
    } else {
    bwd_prefetch<OT, DK, DV>(a, base + last, last, s, j, b0);
    for (int c = last; c >= 0; c -= 2) {
        wait_vm0();
        if (c - 1 >= 0) bwd_prefetch<OT, DK, DV>(a, base + c - 1, c - 1, s, j, b1);
        bwd_flush<OT, DK, DV>(a, s, j, pd);
        bwd_step<OT, DK, DV>(c, b0, dS, stage, pd);
        if (c - 1 < 0) break;
        wait_vm0();
        if (c - 2 >= 0) bwd_prefetch<OT, DK, DV>(a, base + c - 2, c - 2, s, j, b0);
        bwd_flush<OT, DK, DV>(a, s, j, pd);
        bwd_step<OT, DK, DV>(c - 1, b1, dS, stage, pd);
    }
    }
    bwd_flush<OT, DK, DV>(a, s, j, pd);
    if (a.dh0) {
#pragma unroll
        for (int at = 0; at < AT; ++at)
#pragma unroll
            for (int i = 0; i < 4; ++i) a.dh0[((size_t)s * DK + 16 * at + 4 * lq + i) * DV + 16 * j + li] = dS[at][i];
    }
}

// ============================================================================ launchers
template <class OT, int DK, int DV>
hipError_t launch_fwd_chain_t(const Args& a, bool train, hipStream_t stream) {
    const dim3 grid((unsigned)(a.B * a.H * (DV / 16)));
    if (train)
        hipLaunchKernelGGL((k_fwd_chain<OT, DK, DV, true>), grid, dim3(64), 0, stream, a);
    else
        hipLaunchKernelGGL((k_fwd_chain<OT, DK, DV, false>), grid, dim3(64), 0, stream, a);
    return hipGetLastError();
}
template <class OT, int DK, int DV>
hipError_t launch_bwd_chain_t(const Args& a, hipStream_t stream) {
    hipLaunchKernelGGL((k_bwd_chain<OT, DK, DV>), dim3((unsigned)(a.B * a.H * (DV / 16))), dim3(64), 0, stream, a);
    return hipGetLastError();
}

#define GDR2_CHAIN_INST(OT_, DK_, DV_)                                                           \
    template hipError_t launch_fwd_chain_t<OT_, DK_, DV_>(const Args&, bool, hipStream_t);      \
    template hipError_t launch_bwd_chain_t<OT_, DK_, DV_>(const Args&, hipStream_t);
GDR2_CHAIN_INST(bf16, 64, 64)
GDR2_CHAIN_INST(bf16, 64, 128)
GDR2_CHAIN_INST(bf16, 128, 64)
GDR2_CHAIN_INST(bf16, 128, 128)
GDR2_CHAIN_INST(float, 64, 64)
#undef GDR2_CHAIN_INST

}  // namespace gdr2
