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
// Compute wave w owns token tiles w*TPW .. (TPW = 4 / NW) of the chunk and key rows
// 32w .. 32w + 31 of the state slice, which it keeps in MFMA accumulator registers, in
// fp32, for the whole walk (see the K-slot convention in gdr2_device.hpp). A step has
// two barriers. After barrier A every wave reads the whole state slice (published by all
// waves at the end of the previous step) and forms Delta (dDelta) on its own token tiles
// only, and publishes them; after barrier B it reads all of Delta and updates its own
// state rows and outputs. The exchanges go through LDS in the operand type, in the
// contiguous-K fragment order (lane (li, lq) holds K indices 8 lq .. 8 lq + 7) -- no
// wave repeats another's contraction.
//
// The per-chunk operands written by the forward intra-chunk kernel (Wm, Qg, M, Kd^T)
// are fragment images (fimg in gdr2_device.hpp): each MFMA operand fragment is one
// contiguous kilobyte. Forward: every such fragment is read by exactly one compute wave,
// so the compute waves load their own fragments straight into registers, one step ahead
// (two register sets), spreading the loads over the step; the producer waves only pull
// the operands of the chunk PFD steps ahead into L2. Backward: the operands are read
// transposed (K = token), which the LDS transposing reads provide, so the producer waves
// stream them into LDS with asynchronous global->LDS DMA, 16 bytes per lane, in two
// parts, P1 and P2. With two buffers a chunk's whole operand set lands before the barrier
// A that opens its step, the compute waves read all of it before barrier B, and the
// buffer is refilled for the chunk two steps ahead right after B, so the copies run under
// the compute of the step in between and no operand read is left between B and the next
// step. With one buffer
// (operand sets too large for two) P1 is what the compute waves read between A and B and
// P2 what they read after B, and each part is refilled for the next step as soon as it is
// free. The backward producers also pull the operands of the chunk PFD steps ahead
// into L2, with 4-byte DMAs (one cache line per lane) into a scratch word of LDS. In both
// directions the NJ workgroups of a sequence, which share one XCD's L2, split the
// prefetched lines between them.
//
// Measured at d_k = d_v = 128, 64-token chunks, 4096 tokens: a step costs about 1.5 us
// in either direction, most of it waiting on the compute unit's vector-memory pipe (a
// workgroup moves about 60 KB of operands per step; without its global loads and stores
// a step takes about 0.4 us). Wider slices per workgroup (32 or 64 value columns, each
// fragment serving several column tiles) do not help: the bytes a workgroup moves per
// step stay the same while its arithmetic grows.
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
// Every producer issues dma16_count<BYTES>() instructions (a producer short of a piece
// repeats the last one, which writes the same bytes again), so the producers' counts of
// outstanding copies are equal and known at compile time.
template <int BYTES>
constexpr int dma16_count() { return (BYTES / 1024 + NP - 1) / NP; }
template <int BYTES>
__device__ __forceinline__ void dma16(const void* src, lds_char* dst, int pi) {
    static_assert(BYTES % 1024 == 0, "16-byte DMA copies whole 1 KB pieces");
    constexpr int P = BYTES / 1024;
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < dma16_count<BYTES>(); ++i) {
        const int k = min(i * NP + pi, P - 1);
        __builtin_amdgcn_global_load_lds((const char*)src + k * 1024 + l * 16, (lds_void*)(dst + k * 1024), 16, 0, 0);
    }
}
// Producer pi's share of a copy of BYTES (a multiple of 256), 4 bytes per lane; counts as
// for dma16.
template <int BYTES>
constexpr int dma4_count() { return (BYTES / 256 + NP - 1) / NP; }
template <int BYTES>
__device__ __forceinline__ void dma4(const void* src, lds_char* dst, int pi) {
    static_assert(BYTES % 256 == 0, "4-byte DMA copies whole 256-byte pieces");
    constexpr int P = BYTES / 256;
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < dma4_count<BYTES>(); ++i) {
        const int k = min(i * NP + pi, P - 1);
        __builtin_amdgcn_global_load_lds((const char*)src + k * 256 + l * 4, (lds_void*)(dst + k * 256), 4, 0, 0);
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
// them in reverse). Its state slice is the columns col .. col + 16 NC - 1 of the start and
// end matrices (row strides ld_start, ld_end).
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
template <class OT, int DV, bool NTS = false>
__device__ __forceinline__ void store_rows(OT* dst, int row0, int j, const f32x4 (&pend)[RowStore<OT>::PER_LANE]) {
    using R = RowStore<OT>;
    const int l = lane_id();
#pragma unroll
    for (int k = 0; k < R::PER_LANE; ++k) {
        const int p = l + 64 * k, row = p / R::PPR, col = (p % R::PPR) * R::EPP;
        store_out<NTS>((f32x4*)(dst + fmaj_off<DV>(row0 + row, 16 * j + col)), pend[k]);
    }
}

// Exchange area in LDS, in the operand type: per column tile of the workgroup, NW state
// fragments (wave w's 32 key rows of the state slice) and two token fragments (the
// chunk's tokens 0..31 and 32..63 of Delta or dDelta), each an MFMA fragment in the
// contiguous-K order.
template <class OT>
struct Xch {
    static constexpr int FRAG = 64 * 8 * (int)sizeof(OT);
    static constexpr int bytes(int nw, int nc) { return (nw + 2) * nc * FRAG; }
};
// Accumulator tile h (K rows 16 h .. 16 h + 15 of a 32-deep K block, column li) into the
// fragment slot of that block: lane (li, lq) holds rows 16 h + 4 lq + i, i.e. elements
// 4 (lq % 2) + i of reader lane li + 16 (2 h + lq / 2).
template <class OT>
__device__ __forceinline__ void put_k8(lds_char* frag, int h, const f32x4& d) {
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    lds_char* p = frag + ((li + 16 * (2 * h + (lq >> 1))) * 8 + 4 * (lq & 1)) * (int)sizeof(OT);
    if constexpr (sizeof(OT) == 2) {
        bf16x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (bf16)d[i];
        lds_store<bf16x4>(p, x);
    } else {
        lds_store<f32x4>(p, d);
    }
}
template <class OT>
__device__ __forceinline__ typename Frag<OT>::type get_k8(const lds_char* frag) {
    using FT = typename Frag<OT>::type;
    return lds_load<FT>(frag + lane_id() * 8 * (int)sizeof(OT));
}

constexpr int LDS_LIMIT = 160 * 1024;

constexpr int PFD = 2;  // L2 prefetch distance in chunk steps

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

// A producer's side of a walk over NT chunks (walk index n = 0 .. NT - 1). P1(n, buf) and
// P2(n, buf) issue its share of the DMA of the two operand parts of the chunk at walk index
// n (N1 and N2 instructions); PF(n) issues the NPF prefetch DMAs for the chunk at walk
// index min(n, NT - 1). The producer takes part in both barriers of every step (A_n opens
// step n, B_n splits it); a part must have landed before the barrier that opens its reads.
template <bool DBUF, int N1, int N2, int NPF, class F1, class F2, class FP>
__device__ __forceinline__ void produce(int NT, lds_char* b0, lds_char* b1, F1 P1, F2 P2, FP PF) {
    if (DBUF) {
        // both parts of a chunk land before the barrier that opens its step, and the compute
        // waves read all of a buffer before B_n, so the buffer of chunk n is refilled with
        // chunk n + 2 right after B_n
        P1(0, b0);
        P2(0, b0);
        if (NT > 1) {
            P1(1, b1);
            P2(1, b1);
            wait_vm<N1 + N2>();  // chunk 0 complete
        } else {
            wait_vm<0>();
        }
        for (int n = 0; n < NT; ++n) {
            lds_char* cur = (n & 1) ? b1 : b0;
            sync_lds();  // A_n: all of chunk n is in cur
            PF(n + 1 + PFD);
            sync_lds();  // B_n: step n is done with cur
            if (n + 2 < NT) {
                P1(n + 2, cur);
                P2(n + 2, cur);
                wait_vm<N1 + N2>();  // chunk n + 1 (and the prefetch) complete
            } else {
                wait_vm<0>();  // chunk n + 1, if any, and the prefetches complete
            }
        }
    } else {
        (void)PF;
        P1(0, b0);
        wait_vm<0>();
        for (int n = 0; n < NT; ++n) {
            sync_lds();  // A_n: P1 of chunk n is in; step n - 1 is done with P2
            P2(n, b0);
            wait_vm<0>();
            sync_lds();  // B_n: step n is done with P1
            if (n + 1 < NT) {
                P1(n + 1, b0);
                wait_vm<0>();
            }
        }
    }
}

// ============================================================================ forward chain
// Every per-chunk operand of the forward step (rows of Wm, Qg, M, Kd^T, the U tiles, the
// decay factors) is read by exactly one compute wave, so the compute waves load their own
// fragments straight from global memory into registers, one step ahead (two register
// sets), with no LDS staging; only the state and Delta exchanges go through LDS. The
// producer waves just pull the operands of the chunk PFD steps ahead into L2.
template <class OT, int DK, int NC>
struct FwdOps {  // one compute wave's operands of one chunk step
    using FT = typename Frag<OT>::type;
    using U4 = typename std::conditional<sizeof(OT) == 2, bf16x4, f32x4>::type;
    static constexpr int NW = DK / 32, TPW = 4 / NW;
    FT WM[TPW][NW];  // Wm rows of the wave's token tiles, K = key
    FT KT[2][2];     // Kd^T rows of the wave's keys, K = token
    FT QG[TPW][NW];  // Qg rows of the wave's token tiles, K = key (forward with output)
    FT M[TPW][2];    // M rows of the wave's token tiles, K = token (forward with output)
    U4 U[TPW][NC];   // U tiles (token tile, column tile) in accumulator order
    f32x4 g0, g1;    // exp(gam_C) of the wave's key rows 32 w + 4 lq + i and + 16
};

// The loads of a step's operands, in four groups (PART 0: Wm; 1: Kd^T, exp(gam_C);
// 2: Qg; 3: M, U) that the step before issues at different points of its own work: a
// compute unit moves about a kilobyte per vector-memory instruction through its
// address unit, so a burst of all of them would hold the issuing wave for most of a step.
template <class OT, int DK, int DV, bool OUT, int NC, int PART>
__device__ __forceinline__ void fwd_load(const Args& a, long long cid, int j, bool noU, FwdOps<OT, DK, NC>& op) {
    constexpr int NW = DK / 32, TPW = 4 / NW;
    using U4 = typename FwdOps<OT, DK, NC>::U4;
    const Layout& L = a.L;
    const int l = lane_id(), lq = l >> 4, wv = wave_id();
    if (PART == 0) {
        const OT* wm = (const OT*)(a.ws + L.o_wm) + cid * L.wm;
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int kb = 0; kb < NW; ++kb) op.WM[t][kb] = gfrag_img<OT, DK>(wm, 16 * (wv * TPW + t), 32 * kb);
    }
    if (PART == 1) {
        const OT* kd = (const OT*)(a.ws + L.o_kd) + cid * L.kd;
        const float* gc = (const float*)(a.ws + L.o_gc) + cid * L.gc;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) op.KT[h][kb] = gfrag_img<OT, CH>(kd, 32 * wv + 16 * h, 32 * kb);
        op.g0 = *(const f32x4*)(gc + 32 * wv + 4 * lq);
        op.g1 = *(const f32x4*)(gc + 32 * wv + 16 + 4 * lq);
    }
    if (PART == 2 && OUT) {
        const OT* qg = (const OT*)(a.ws + L.o_qg) + cid * L.qg;
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int kb = 0; kb < NW; ++kb) op.QG[t][kb] = gfrag_img<OT, DK>(qg, 16 * (wv * TPW + t), 32 * kb);
    }
    if (PART == 3) {
        const OT* m = (const OT*)(a.ws + L.o_m) + cid * L.m;
        const OT* u = (const OT*)(a.ws + L.o_u) + cid * L.u + (size_t)j * NC * 4 * 256;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int tt = wv * TPW + t;
            if (OUT) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) op.M[t][kb] = gfrag_img<OT, CH>(m, 16 * tt, 32 * kb);
            }
#pragma unroll
            for (int ch = 0; ch < NC; ++ch) {
                if (noU) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) op.U[t][ch][i] = (OT)0.f;
                } else {
                    op.U[t][ch] = *(const U4*)(u + (ch * 4 + tt) * 256 + l * 4);
                }
            }
        }
    }
}
template <class OT, int DK, int DV, bool OUT, int NC>
__device__ __forceinline__ void fwd_load_all(const Args& a, long long cid, int j, bool noU, FwdOps<OT, DK, NC>& op) {
    fwd_load<OT, DK, DV, OUT, NC, 0>(a, cid, j, noU, op);
    fwd_load<OT, DK, DV, OUT, NC, 1>(a, cid, j, noU, op);
    fwd_load<OT, DK, DV, OUT, NC, 2>(a, cid, j, noU, op);
    fwd_load<OT, DK, DV, OUT, NC, 3>(a, cid, j, noU, op);
}

// outputs of one step held by one compute wave until the next step issues them
template <class OT, int NW, int NC>
struct FwdPend {
    static constexpr int TPW = 4 / NW;     // token tiles per wave
    f32x4 st[NC][RowStore<OT>::PER_LANE];  // this wave's rows of the chunk start state
    f32x4 D[TPW][NC], O[TPW][NC];          // Delta and O^T tiles (token tile wv * TPW + u, column tile)
    int c;                                 // chunk, -1 = nothing pending
};

// TRAIN: 0 inference; 1 training (the chunk start states S and Delta are saved for the
// backward); 2 training with S and Delta written by non-temporal stores (large workspaces:
// they are read only by the backward intra-chunk kernel, much later).
template <class OT, int DK, int DV, int TRAIN, bool OUT, int NW, int NC>
__device__ __forceinline__ void fwd_flush(const Args& a, int s, int j, FwdPend<OT, NW, NC>& pd) {
    if (pd.c < 0) return;
    constexpr int TPW = FwdPend<OT, NW, NC>::TPW;
    const int l = lane_id(), li = l & 15, lq = l >> 4, wv = wave_id();
    const long long cid = (long long)s * a.NT + pd.c;
    const Layout& L = a.L;
#pragma unroll
    for (int ch = 0; ch < NC; ++ch) {
        const int jt = NC * j + ch;  // 16-column tile of the value axis
        if (TRAIN) {
            store_rows<OT, DV, TRAIN == 2>((OT*)(a.ws + L.o_s) + cid * L.s, 32 * wv, jt, pd.st[ch]);
            OT* dl = (OT*)(a.ws + L.o_delta) + cid * L.delta + jt * 4 * 256;
#pragma unroll
            for (int u = 0; u < TPW; ++u) store_tile<OT, TRAIN == 2>(dl + (wv * TPW + u) * 256, pd.D[u][ch]);
        }
        if (OUT) {
            const int bidx = s / a.H, h = s % a.H;
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int row = pd.c * CH + 16 * (wv * TPW + u) + li;
                if (row < a.T) {
                    float ov[4] = {pd.O[u][ch][0], pd.O[u][ch][1], pd.O[u][ch][2], pd.O[u][ch][3]};
                    st4((OT*)a.o + (((size_t)bidx * a.T + row) * a.H + h) * DV + 16 * jt + 4 * lq, ov);
                }
            }
        }
    }
}

// One chunk step of a compute wave (barrier A_n has been passed: the state fragments of
// all waves are in the exchange). Contains barrier B_n. Issues the stores of the previous
// step and, spread over its own work, the loads of the next step's operands (chunk ncid)
// into nxt. Exchange slots: state fragment (key block kb, column tile ch) at kb * NC + ch,
// Delta fragment (token block tb, column tile ch) at NW * NC + tb * NC + ch.
template <class OT, int DK, int DV, int TRAIN, bool OUT, int NW, int NC>
__device__ __forceinline__ void fwd_step(const Args& a, int s, int j, int c, const FwdOps<OT, DK, NC>& op,
                                         FwdOps<OT, DK, NC>& nxt, long long ncid, bool noU, f32x4 (&S0)[NC],
                                         f32x4 (&S1)[NC], lds_char* stage, lds_char* xs, FwdPend<OT, NW, NC>& pd) {
    using FT = typename Frag<OT>::type;
    constexpr int TPW = FwdPend<OT, NW, NC>::TPW;
    constexpr int FRAG = Xch<OT>::FRAG;
    const int wv = wave_id();
    lds_char* xsS = xs;                   // state fragments
    lds_char* xsD = xs + NW * NC * FRAG;  // Delta fragments
    FT SB[NW][NC];
#pragma unroll
    for (int kb = 0; kb < NW; ++kb)
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) SB[kb][ch] = get_k8<OT>(xsS + (kb * NC + ch) * FRAG);
    fwd_flush<OT, DK, DV, TRAIN, OUT, NW, NC>(a, s, j, pd);
    if (TRAIN) {  // chunk start state -> pending store
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) stage_rows<OT>(stage, S0[ch], S1[ch], pd.st[ch]);
    }
    __builtin_amdgcn_sched_barrier(0);
    fwd_load<OT, DK, DV, OUT, NC, 0>(a, ncid, j, noU, nxt);
    __builtin_amdgcn_sched_barrier(0);
    // Delta = U - Wm S on this wave's token tiles, published for every wave (two partial
    // sums halve the dependent MFMA chain)
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = wv * TPW + u;
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) {
            f32x4 D0 = {0.f, 0.f, 0.f, 0.f}, D1 = D0;
#pragma unroll
            for (int kb = 0; kb < NW; kb += 2) {
                mma(D0, op.WM[u][kb], SB[kb][ch]);
                if (kb + 1 < NW) mma(D1, op.WM[u][kb + 1], SB[kb + 1][ch]);
            }
            f32x4 D;
#pragma unroll
            for (int i = 0; i < 4; ++i) D[i] = (float)op.U[u][ch][i] - (D0[i] + D1[i]);
            put_k8<OT>(xsD + ((t >> 1) * NC + ch) * FRAG, t & 1, D);
            pd.D[u][ch] = D;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    fwd_load<OT, DK, DV, OUT, NC, 1>(a, ncid, j, noU, nxt);
    sync_lds();  // B_n: all of Delta is in the exchange
    FT DB[2][NC];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) DB[kb][ch] = get_k8<OT>(xsD + (kb * NC + ch) * FRAG);
    // S' = diag(exp gam_C) S + Kd^T Delta on this wave's rows, published for the next step
    // (every wave read the state fragments before B_n)
#pragma unroll
    for (int ch = 0; ch < NC; ++ch) {
        f32x4 a0 = op.g0 * S0[ch], a1 = op.g1 * S1[ch];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            mma(a0, op.KT[0][kb], DB[kb][ch]);
            mma(a1, op.KT[1][kb], DB[kb][ch]);
        }
        S0[ch] = a0;
        S1[ch] = a1;
        put_k8<OT>(xsS + (wv * NC + ch) * FRAG, 0, a0);
        put_k8<OT>(xsS + (wv * NC + ch) * FRAG, 1, a1);
    }
    __builtin_amdgcn_sched_barrier(0);
    fwd_load<OT, DK, DV, OUT, NC, 2>(a, ncid, j, noU, nxt);
    __builtin_amdgcn_sched_barrier(0);
    // O^T = S^T Qg^T + Delta^T M^T on this wave's token tiles
    if (OUT) {
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
            for (int ch = 0; ch < NC; ++ch) {
                f32x4 po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NW; ++kb) mma(po, SB[kb][ch], op.QG[u][kb]);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) mma(po, DB[kb][ch], op.M[u][kb]);
                pd.O[u][ch] = po;
            }
    }
    __builtin_amdgcn_sched_barrier(0);
    fwd_load<OT, DK, DV, OUT, NC, 3>(a, ncid, j, noU, nxt);
    pd.c = c;
}

template <class OT, int DK, int DV, int TRAIN, bool OUT, int NW, int NC>
__device__ __forceinline__ void fwd_walk(const Args& a, int s, int j, const WalkSpec& w, lds_char* xs,
                                         lds_char* stage_base, lds_char* pfslot) {
    constexpr int NJ = DV / (16 * NC);  // workgroups per sequence (value slices)
    const int wv = wave_id();
    const int NT = w.n;
    const long long base = (long long)s * a.NT + w.c0;
    if (wv >= NW) {  // producer: L2 prefetch only, in step with the compute waves' barriers
        const Layout& L = a.L;
        const int pi = wv - NW;
        constexpr int ES = sizeof(OT);
        // regions: Wm, Kd^T, U (all slices), exp(gam_C) [, Qg, M]
        constexpr int LK = CH * DK * ES / 128, LU = CH * DV * ES / 128;
        constexpr int LM = CH * CH * ES / 128, LG = DK * 4 / 128;
        constexpr int LINES = 2 * LK + LU + LG + (OUT ? LK + LM : 0);
        constexpr int NPF = prefetch_count<LINES, NJ>();
        auto PF = [&](int n) {
            const long long cid = base + (n < NT ? n : NT - 1);
            const char* wm = a.ws + L.o_wm + cid * L.wm * ES;
            const char* kd = a.ws + L.o_kd + cid * L.kd * ES;
            const char* u = a.ws + L.o_u + cid * L.u * ES;
            const char* gc = a.ws + L.o_gc + cid * L.gc * 4;
            const char* qg = a.ws + L.o_qg + cid * L.qg * ES;
            const char* m = a.ws + L.o_m + cid * L.m * ES;
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
#pragma unroll 1
        for (int n = 1; n <= PFD; ++n) PF(n);
#pragma unroll 1
        for (int n = 0; n < NT; ++n) {
            sync_lds();  // A_n
            PF(n + 1 + PFD);
            wait_vm<NPF * PFD>();  // bounds the outstanding prefetches
            sync_lds();  // B_n
        }
        wait_vm<0>();
        return;
    }
    // compute waves: state rows 32 wv + 4 lq + i (S0) and 32 wv + 16 + 4 lq + i (S1),
    // column w.col + 16 ch + li
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    lds_char* stage = stage_base + wv * RowStore<OT>::BYTES;
    const int row0 = 32 * wv + 4 * lq;
    FwdOps<OT, DK, NC> op0, op1;
    fwd_load_all<OT, DK, DV, OUT, NC>(a, base, j, w.noU, op0);
    f32x4 S0[NC], S1[NC];
#pragma unroll
    for (int ch = 0; ch < NC; ++ch) {
        const int col = w.col + 16 * ch + li;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (w.ident) {
                S0[ch][i] = row0 + i == col ? 1.f : 0.f;
                S1[ch][i] = row0 + 16 + i == col ? 1.f : 0.f;
            } else {
                S0[ch][i] = w.start ? w.start[(size_t)(row0 + i) * w.ld_start + col] : 0.f;
                S1[ch][i] = w.start ? w.start[(size_t)(row0 + 16 + i) * w.ld_start + col] : 0.f;
            }
        }
        put_k8<OT>(xs + (wv * NC + ch) * Xch<OT>::FRAG, 0, S0[ch]);
        put_k8<OT>(xs + (wv * NC + ch) * Xch<OT>::FRAG, 1, S1[ch]);
    }
    FwdPend<OT, NW, NC> pd;
    pd.c = -1;
    const int c0 = w.c0;
    // two steps per iteration, alternating the register sets; each step loads the next
    // step's operands (past the last chunk they repeat it)
#pragma unroll 1
    for (int n = 0; n < NT; n += 2) {
        sync_lds();  // A_n
        fwd_step<OT, DK, DV, TRAIN, OUT, NW, NC>(a, s, j, c0 + n, op0, op1, base + min(n + 1, NT - 1), w.noU, S0,
                                                 S1, stage, xs, pd);
        if (n + 1 == NT) break;
        sync_lds();  // A_{n+1}
        fwd_step<OT, DK, DV, TRAIN, OUT, NW, NC>(a, s, j, c0 + n + 1, op1, op0, base + min(n + 2, NT - 1), w.noU,
                                                 S0, S1, stage, xs, pd);
    }
    fwd_flush<OT, DK, DV, TRAIN, OUT, NW, NC>(a, s, j, pd);
    if (w.end) {
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) {
            const int col = w.col + 16 * ch + li;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w.end[(size_t)(row0 + i) * w.ld_end + col] = S0[ch][i];
                w.end[(size_t)(row0 + 16 + i) * w.ld_end + col] = S1[ch][i];
            }
        }
    }
}

template <class OT, int DK, int DV, int NC, int TRAIN>
__global__ __launch_bounds__(64 * (DK / 32 + NP)) void k_fwd_chain(Args a) {
    constexpr int NW = DK / 32, NJ = DV / (16 * NC);
    __shared__ __align__(16) char xch[Xch<OT>::bytes(NW, NC)];
    __shared__ __align__(16) char stage[NW * RowStore<OT>::BYTES];
    __shared__ __align__(16) char pfslot[256];  // target of the L2 prefetch DMAs, never read
    poison_lds((lds_char*)xch, sizeof(xch));
    poison_lds((lds_char*)stage, sizeof(stage));
    poison_lds_done();
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
    w.col = 16 * NC * j;
    w.noU = false;
    if (a.o)
        fwd_walk<OT, DK, DV, TRAIN, true, NW, NC>(a, s, j, w, (lds_char*)xch, (lds_char*)stage, (lds_char*)pfslot);
    else
        fwd_walk<OT, DK, DV, TRAIN, false, NW, NC>(a, s, j, w, (lds_char*)xch, (lds_char*)stage, (lds_char*)pfslot);
}

// Summary walks of the chunk-parallel scan, one per (sequence, segment k < NSEG - 1,
// 16-column slice): value slices j < DV / 16 walk from a zero start (segment 0: from h0)
// and write the segment's end state H_k; transition slices j >= DV / 16 walk the
// identity's columns with no value input and write P_k (not needed, and not run, for
// segment 0).
template <class OT, int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 32 + NP)) void k_fwd_chain_sum(Args a) {
    constexpr int NW = DK / 32, NJ = DV / 16, NJP = DK / 16;
    __shared__ __align__(16) char xch[Xch<OT>::bytes(NW, 1)];
    __shared__ __align__(16) char pfslot[256];  // target of the L2 prefetch DMAs, never read
    poison_lds((lds_char*)xch, sizeof(xch));
    poison_lds_done();
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
    fwd_walk<OT, DK, DV, 0, false, NW, 1>(a, s, j, w, (lds_char*)xch, nullptr, (lds_char*)pfslot);
}

// ============================================================================ backward chain
template <class OT, int DK, int DV, int NC>
struct BwdChainBuf {  // P1: Kd^T, M, dO rows, exp(gam_C); P2: T, Qg, Wm
    static constexpr int ES = sizeof(OT);
    static constexpr int KDT = 0;                    // Kd^T [DK][64] swizzled
    static constexpr int M = KDT + DK * CH * ES;     // M [64][64]
    static constexpr int DO = M + CH * CH * ES;      // dO rows of this slice [64][16 NC]
    static constexpr int GC = DO + 64 * 16 * NC * ES;  // exp(gam_C), DK floats
    static constexpr int T = GC + DK * 4;            // T [64][64]
    static constexpr int QG = T + CH * CH * ES;      // Qg [64][DK]
    static constexpr int WM = QG + CH * DK * ES;     // Wm [64][DK]
    static constexpr int BYTES = WM + CH * DK * ES;
};

template <class OT, int NW, int NC>
struct BwdPend {
    static constexpr int TPW = 4 / NW;
    f32x4 st[NC][RowStore<OT>::PER_LANE];  // this wave's rows of the end-state gradient
    f32x4 Y[TPW][NC];                      // dY tiles (token tile wv * TPW + u, column tile)
    int c;
};

template <class OT, int DK, int DV, int NW, int NC, bool NTS>
__device__ __forceinline__ void bwd_flush(const Args& a, int s, int j, BwdPend<OT, NW, NC>& pd) {
    if (pd.c < 0) return;
    constexpr int TPW = BwdPend<OT, NW, NC>::TPW;
    const int wv = wave_id();
    const long long cid = (long long)s * a.NT + pd.c;
    const Layout& L = a.L;
#pragma unroll
    for (int ch = 0; ch < NC; ++ch) {
        const int jt = NC * j + ch;
        store_rows<OT, DV, NTS>((OT*)(a.ws + L.o_ds) + cid * L.ds, 32 * wv, jt, pd.st[ch]);
        OT* dy = (OT*)(a.ws + L.o_dy) + cid * L.dy + jt * 4 * 256;
#pragma unroll
        for (int u = 0; u < TPW; ++u) store_tile<OT, NTS>(dy + (wv * TPW + u) * 256, pd.Y[u][ch]);
    }
}

// One chunk step of a compute wave (barrier A_n has been passed: the end-state gradient
// fragments of all waves are in the exchange and the chunk's P1 operands in buf).
// Contains barrier B_n. SUM: a summary walk -- only the state gradient, no per-chunk
// outputs. Exchange slots as in the forward.
template <class OT, int DK, int DV, int NW, int NC, bool SUM, bool EARLY>
__device__ __forceinline__ void bwd_step(int c, const lds_char* buf, f32x4 (&dS0)[NC], f32x4 (&dS1)[NC],
                                         lds_char* stage, lds_char* xs, BwdPend<OT, NW, NC>& pd) {
    using B = BwdChainBuf<OT, DK, DV, NC>;
    using FT = typename Frag<OT>::type;
    constexpr int TPW = BwdPend<OT, NW, NC>::TPW;
    constexpr int FRAG = Xch<OT>::FRAG;
    const int l = lane_id(), lq = l >> 4, wv = wave_id();
    const LImg<OT, CH> vKT{buf + B::KDT}, vM{buf + B::M};
    const LSwz<OT, CH> vT{buf + B::T};
    const LImg<OT, DK> vQG{buf + B::QG}, vWM{buf + B::WM};
    const LPad<OT> vDO{buf + B::DO, 16 * NC};
    lds_char* xsS = xs;                   // state-gradient fragments
    lds_char* xsD = xs + NW * NC * FRAG;  // dDelta fragments
    if (!SUM) {  // gradient w.r.t. this chunk's end state -> pending store
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) stage_rows<OT>(stage, dS0[ch], dS1[ch], pd.st[ch]);
    }
    // P1 reads of the step, all issued before the first product
    FT dSB[NW][NC], KDf[TPW][NW], Mf[TPW][2], dOB[2][NC];
    float g0[4], g1[4];
#pragma unroll
    for (int kb = 0; kb < NW; ++kb)
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) dSB[kb][ch] = get_k8<OT>(xsS + (kb * NC + ch) * FRAG);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) dOB[kb][ch] = lfrag_colk8<OT>(vDO, 16 * ch, 32 * kb);  // K = token
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = wv * TPW + u;
#pragma unroll
        for (int kb = 0; kb < NW; ++kb) KDf[u][kb] = lfrag_colk8<OT>(vKT, 16 * t, 32 * kb);  // Kd rows, K = key
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) Mf[u][kb] = lfrag_colk8<OT>(vM, 16 * t, 32 * kb);  // M^T rows, K = token
    }
    lds_get4<float>(buf + B::GC + (32 * wv + 4 * lq) * 4, g0);
    lds_get4<float>(buf + B::GC + (32 * wv + 16 + 4 * lq) * 4, g1);
    // EARLY (double-buffered operands): the P2 operands are in the buffer already, so they are
    // read here too and no read of the buffer is left after barrier B
    FT QGf[2][2], WMf[2][2], Tf[TPW][2];
    if constexpr (EARLY) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                QGf[h][kb] = lfrag_colk8<OT>(vQG, 32 * wv + 16 * h, 32 * kb);
                WMf[h][kb] = lfrag_colk8<OT>(vWM, 32 * wv + 16 * h, 32 * kb);
            }
        if (!SUM) {
#pragma unroll
            for (int u = 0; u < TPW; ++u)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) Tf[u][kb] = lfrag_colk8<OT>(vT, 16 * (wv * TPW + u), 32 * kb);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // dDelta = M^T dO + Kd dS' on this wave's token tiles, published for every wave
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = wv * TPW + u;
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) {
            f32x4 dD = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NW; ++kb) mma(dD, KDf[u][kb], dSB[kb][ch]);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) mma(dD, Mf[u][kb], dOB[kb][ch]);
            put_k8<OT>(xsD + ((t >> 1) * NC + ch) * FRAG, t & 1, dD);
        }
    }
    // diag(exp gam_C) dS' + Qg^T dO on this wave's rows (the part of dS without dDelta)
    f32x4 P0[NC], P1[NC];
    auto state_part = [&]() {
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) {
            P0[ch] = f32x4{g0[0] * dS0[ch][0], g0[1] * dS0[ch][1], g0[2] * dS0[ch][2], g0[3] * dS0[ch][3]};
            P1[ch] = f32x4{g1[0] * dS1[ch][0], g1[1] * dS1[ch][1], g1[2] * dS1[ch][2], g1[3] * dS1[ch][3]};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                mma(P0[ch], QGf[0][kb], dOB[kb][ch]);
                mma(P1[ch], QGf[1][kb], dOB[kb][ch]);
            }
        }
    };
    sync_lds();  // B_n: all of dDelta is in the exchange (and, without EARLY, the P2 operands in buf)
    FT dDB[2][NC];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) dDB[kb][ch] = get_k8<OT>(xsD + (kb * NC + ch) * FRAG);
        if constexpr (!EARLY) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {  // Qg^T and Wm^T rows (this wave's keys), K = token
                QGf[h][kb] = lfrag_colk8<OT>(vQG, 32 * wv + 16 * h, 32 * kb);
                WMf[h][kb] = lfrag_colk8<OT>(vWM, 32 * wv + 16 * h, 32 * kb);
            }
        }
    }
    if constexpr (!EARLY) {
        if (!SUM) {
#pragma unroll
            for (int u = 0; u < TPW; ++u)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) Tf[u][kb] = lfrag_colk8<OT>(vT, 16 * (wv * TPW + u), 32 * kb);
        }
    }
    state_part();
    // dS = diag(exp gam_C) dS' + Qg^T dO - Wm^T dDelta on this wave's rows, published for the
    // next step (every wave read the state-gradient fragments before B_n)
#pragma unroll
    for (int ch = 0; ch < NC; ++ch) {
        f32x4 n0 = {0.f, 0.f, 0.f, 0.f}, n1 = n0;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            mma(n0, WMf[0][kb], dDB[kb][ch]);
            mma(n1, WMf[1][kb], dDB[kb][ch]);
        }
        dS0[ch] = P0[ch] - n0;
        dS1[ch] = P1[ch] - n1;
        put_k8<OT>(xsS + (wv * NC + ch) * FRAG, 0, dS0[ch]);
        put_k8<OT>(xsS + (wv * NC + ch) * FRAG, 1, dS1[ch]);
    }
    if (SUM) return;
    // dY = T^T dDelta on this wave's token tiles (for the intra-chunk kernel)
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) mma(acc, Tf[u][kb], dDB[kb][ch]);
            pd.Y[u][ch] = acc;
        }
    pd.c = c;
}

template <class OT, int DK, int DV, int NW, int NC, bool DBUF, bool SUM, bool NTS = false>
__device__ __forceinline__ void bwd_walk(const Args& a, int s, int j, const WalkSpec& w, lds_char* b0, lds_char* b1,
                                         lds_char* xs, lds_char* stage_base, lds_char* pfslot) {
    using B = BwdChainBuf<OT, DK, DV, NC>;
    constexpr int NJ = DV / (16 * NC);
    const int wv = wave_id();
    const int NT = w.n, last = w.c0 + w.n - 1;  // walk index n is chunk last - n
    const long long base = (long long)s * a.NT;
    if (wv >= NW) {  // producer; walk index n is chunk last - n
        const Layout& L = a.L;
        const int pi = wv - NW;
        const int l = lane_id();
        const int bidx = s / a.H, h = s % a.H;
        constexpr int ES = sizeof(OT);
        constexpr int CW = 16 * NC;           // columns of this slice
        constexpr int LPR = CW * ES / 16;     // dO: lanes per row, 16 bytes each
        constexpr int RPI = 64 / LPR;         // dO rows per instruction
        auto P1 = [&](int n, lds_char* buf) {
            const int c = last - n;
            const long long cid = base + c;
            dma16<DK * CH * ES>(a.ws + L.o_kd + cid * L.kd * ES, buf + B::KDT, pi);
            dma16<CH * CH * ES>(a.ws + L.o_m + cid * L.m * ES, buf + B::M, pi);
            dma4<DK * 4>(a.ws + L.o_gc + cid * L.gc * 4, buf + B::GC, pi);
            // dO rows of this slice. Rows past the end of the sequence repeat its last row:
            // every product that reads dO (M^T dO, Qg^T dO) multiplies those rows by rows of
            // M and Qg that the intra-chunk kernel wrote as exact zeros.
#pragma unroll
            for (int i = 0; i < 64 / RPI / NP; ++i) {
                const int k = i * NP + pi;
                const int r = k * RPI + l / LPR;
                const int col = (l % LPR) * (16 / ES);
                const int row = min(c * CH + r, a.T - 1);
                const OT* src = (const OT*)a.dout + (((size_t)bidx * a.T + row) * a.H + h) * DV + CW * j + col;
                __builtin_amdgcn_global_load_lds(src, (lds_void*)(buf + B::DO + k * 1024), 16, 0, 0);
            }
        };
        auto P2 = [&](int n, lds_char* buf) {
            const long long cid = base + (last - n);
            if (!SUM) dma16<CH * CH * ES>(a.ws + L.o_t + cid * L.t * ES, buf + B::T, pi);
            dma16<CH * DK * ES>(a.ws + L.o_qg + cid * L.qg * ES, buf + B::QG, pi);
            dma16<CH * DK * ES>(a.ws + L.o_wm + cid * L.wm * ES, buf + B::WM, pi);
        };
        static_assert(RPI >= 1 && (64 / RPI) % NP == 0, "the dO rows split evenly over the producers");
        constexpr int N1 = dma16_count<DK * CH * ES>() + dma16_count<CH * CH * ES>() + dma4_count<DK * 4>() +
                           64 / RPI / NP;
        constexpr int N2 = 2 * dma16_count<CH * DK * ES>() + (SUM ? 0 : dma16_count<CH * CH * ES>());
        // prefetch regions: Kd^T, Qg, Wm, M, T, exp(gam_C), dO rows (all slices)
        constexpr int LK = CH * DK * ES / 128, LM = CH * CH * ES / 128;
        constexpr int LG = DK * 4 / 128, LR = DV * ES / 128;  // lines per dO row
        constexpr int LINES = 3 * LK + 2 * LM + LG + CH * LR;
        auto PF = [&](int n) {
            const int c = last - (n < NT ? n : NT - 1);
            const long long cid = base + c;
            const char* kd = a.ws + L.o_kd + cid * L.kd * ES;
            const char* qg = a.ws + L.o_qg + cid * L.qg * ES;
            const char* wm = a.ws + L.o_wm + cid * L.wm * ES;
            const char* m = a.ws + L.o_m + cid * L.m * ES;
            const char* t = a.ws + L.o_t + cid * L.t * ES;
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
                return (const char*)a.dout + ((((size_t)bidx * a.T + row) * a.H + h) * DV) * ES + (v % LR) * 128;
            };
            prefetch_lines<LINES, NJ>(line, j, pi, pfslot);
        };
        produce<DBUF, N1, N2, prefetch_count<LINES, NJ>()>(NT, b0, b1, P1, P2, PF);
        return;
    }
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    lds_char* stage = stage_base + wv * RowStore<OT>::BYTES;
    const int row0 = 32 * wv + 4 * lq;
    f32x4 dS0[NC], dS1[NC];
#pragma unroll
    for (int ch = 0; ch < NC; ++ch) {
        const int col = w.col + 16 * ch + li;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dS0[ch][i] = w.start ? w.start[(size_t)(row0 + i) * w.ld_start + col] : 0.f;
            dS1[ch][i] = w.start ? w.start[(size_t)(row0 + 16 + i) * w.ld_start + col] : 0.f;
        }
        put_k8<OT>(xs + (wv * NC + ch) * Xch<OT>::FRAG, 0, dS0[ch]);
        put_k8<OT>(xs + (wv * NC + ch) * Xch<OT>::FRAG, 1, dS1[ch]);
    }
    BwdPend<OT, NW, NC> pd;
    pd.c = -1;
    for (int n = 0; n < NT; ++n) {
        sync_lds();  // A_n
        bwd_flush<OT, DK, DV, NW, NC, NTS>(a, s, j, pd);
        bwd_step<OT, DK, DV, NW, NC, SUM, DBUF>(last - n, (DBUF && (n & 1)) ? b1 : b0, dS0, dS1, stage, xs, pd);
    }
    bwd_flush<OT, DK, DV, NW, NC, NTS>(a, s, j, pd);
    if (w.end) {
#pragma unroll
        for (int ch = 0; ch < NC; ++ch) {
            const int col = w.col + 16 * ch + li;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w.end[(size_t)(row0 + i) * w.ld_end + col] = dS0[ch][i];
                w.end[(size_t)(row0 + 16 + i) * w.ld_end + col] = dS1[ch][i];
            }
        }
    }
}

template <class OT, int DK, int DV, int NC, bool STAGE>
struct BwdChainLds {
    static constexpr int NW = DK / 32;
    static constexpr int XBYTES = Xch<OT>::bytes(NW, NC);
    static constexpr int SBYTES = STAGE ? NW * RowStore<OT>::BYTES : 16;
    static constexpr bool DBUF = 2 * BwdChainBuf<OT, DK, DV, NC>::BYTES + XBYTES + SBYTES + 256 <= LDS_LIMIT;
};

template <class OT, int DK, int DV, int NC, bool NTS>
__global__ __launch_bounds__(64 * (DK / 32 + NP)) void k_bwd_chain(Args a) {
    using B = BwdChainBuf<OT, DK, DV, NC>;
    using LZ = BwdChainLds<OT, DK, DV, NC, true>;
    constexpr int NW = DK / 32, NJ = DV / (16 * NC);
    constexpr bool DBUF = LZ::DBUF;
    __shared__ __align__(16) char buf0[B::BYTES];
    __shared__ __align__(16) char buf1[DBUF ? B::BYTES : 16];
    __shared__ __align__(16) char xch[LZ::XBYTES];
    __shared__ __align__(16) char stage[LZ::SBYTES];
    __shared__ __align__(16) char pfslot[256];  // target of the L2 prefetch DMAs, never read
    poison_lds((lds_char*)buf0, sizeof(buf0));
    poison_lds((lds_char*)buf1, sizeof(buf1));
    poison_lds((lds_char*)xch, sizeof(xch));
    poison_lds((lds_char*)stage, sizeof(stage));
    poison_lds_done();
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
    w.col = 16 * NC * j;
    w.noU = false;
    bwd_walk<OT, DK, DV, NW, NC, DBUF, false, NTS>(a, s, j, w, (lds_char*)buf0, (lds_char*)buf1, (lds_char*)xch,
                                              (lds_char*)stage, (lds_char*)pfslot);
}

// Summary walks of the backward scan, one per (sequence, segment k >= 1, 16-column slice):
// the gradient with respect to the segment's start state when the gradient at its end is
// zero (the last segment: dht), into the summary array.
template <class OT, int DK, int DV>
__global__ __launch_bounds__(64 * (DK / 32 + NP)) void k_bwd_chain_sum(Args a) {
    using B = BwdChainBuf<OT, DK, DV, 1>;
    using LZ = BwdChainLds<OT, DK, DV, 1, false>;
    constexpr int NW = DK / 32, NJ = DV / 16;
    constexpr bool DBUF = LZ::DBUF;
    __shared__ __align__(16) char buf0[B::BYTES];
    __shared__ __align__(16) char buf1[DBUF ? B::BYTES : 16];
    __shared__ __align__(16) char xch[LZ::XBYTES];
    __shared__ __align__(16) char pfslot[256];  // target of the L2 prefetch DMAs, never read
    poison_lds((lds_char*)buf0, sizeof(buf0));
    poison_lds((lds_char*)buf1, sizeof(buf1));
    poison_lds((lds_char*)xch, sizeof(xch));
    poison_lds_done();
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
    bwd_walk<OT, DK, DV, NW, 1, DBUF, true>(a, s, j, w, (lds_char*)buf0, (lds_char*)buf1, (lds_char*)xch, nullptr,
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
    poison_lds((lds_char*)smem_, (DK * PP + DK * 16) * 4);
    poison_lds_done();
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
// Value columns per main-chain workgroup: 16 (NC = 1) or 32 (NC = 2). A step's cost is set by
// the operands its workgroup moves through its compute unit's memory path (about 60 KB per step
// whatever the slice width). With at most one 16-column walk per compute unit the narrow slices
// finish first (their steps carry less arithmetic); with two or more, walks queue on the compute
// units and 32-column slices, which move the shared operands once for two column tiles, halve
// the traffic and the number of walks.
inline hipError_t chain_nc(long long walks16, int& nc) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    nc = (e == hipSuccess && walks16 >= 2LL * cus) ? 2 : 1;
    return e;
}

template <class OT, int DK, int DV>
hipError_t launch_fwd_chain_t(const Args& a, bool train, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    const unsigned S = (unsigned)(a.B * a.H), NJ1 = DV / 16, NJP = DK / 16;
    const dim3 block(64 * (DK / 32 + NP));
    hipError_t e;
    if (a.nseg > 1) {
        hipExtLaunchKernelGGL((k_fwd_chain_sum<OT, DK, DV>), dim3(S * (a.nseg - 1) * (NJ1 + NJP)), block, 0, stream,
                              start, nullptr, 0, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_seg_scan<DK, DV, false>(a, stream)) != hipSuccess) return e;
        start = nullptr;
    }
    int nc = 1;
    if ((e = chain_nc((long long)S * a.nseg * NJ1, nc)) != hipSuccess) return e;
    const dim3 grid(S * a.nseg * (NJ1 / nc));
    // the non-temporal choice is a template parameter: behind a run-time branch the
    // compiler merges the two kinds of store and drops the hint
    const int mode = train ? (a.nt_out ? 2 : 1) : 0;
    if (nc == 2) {
        if (mode == 2)
            hipExtLaunchKernelGGL((k_fwd_chain<OT, DK, DV, 2, 2>), grid, block, 0, stream, start, stop, 0, a);
        else if (mode == 1)
            hipExtLaunchKernelGGL((k_fwd_chain<OT, DK, DV, 2, 1>), grid, block, 0, stream, start, stop, 0, a);
        else
            hipExtLaunchKernelGGL((k_fwd_chain<OT, DK, DV, 2, 0>), grid, block, 0, stream, start, stop, 0, a);
    } else {
        if (mode == 2)
            hipExtLaunchKernelGGL((k_fwd_chain<OT, DK, DV, 1, 2>), grid, block, 0, stream, start, stop, 0, a);
        else if (mode == 1)
            hipExtLaunchKernelGGL((k_fwd_chain<OT, DK, DV, 1, 1>), grid, block, 0, stream, start, stop, 0, a);
        else
            hipExtLaunchKernelGGL((k_fwd_chain<OT, DK, DV, 1, 0>), grid, block, 0, stream, start, stop, 0, a);
    }
    return hipGetLastError();
}
template <class OT, int DK, int DV>
hipError_t launch_bwd_chain_t(const Args& a, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    const unsigned S = (unsigned)(a.B * a.H), NJ1 = DV / 16;
    const dim3 block(64 * (DK / 32 + NP));
    hipError_t e;
    if (a.nseg > 1) {
        hipExtLaunchKernelGGL((k_bwd_chain_sum<OT, DK, DV>), dim3(S * (a.nseg - 1) * NJ1), block, 0, stream, start,
                              nullptr, 0, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_seg_scan<DK, DV, true>(a, stream)) != hipSuccess) return e;
        start = nullptr;
    }
    int nc = 1;
    if ((e = chain_nc((long long)S * a.nseg * NJ1, nc)) != hipSuccess) return e;
    const dim3 grid(S * a.nseg * (NJ1 / nc));
    if (nc == 2) {
        if (a.nt_out)
            hipExtLaunchKernelGGL((k_bwd_chain<OT, DK, DV, 2, true>), grid, block, 0, stream, start, stop, 0, a);
        else
            hipExtLaunchKernelGGL((k_bwd_chain<OT, DK, DV, 2, false>), grid, block, 0, stream, start, stop, 0, a);
    } else {
        if (a.nt_out)
            hipExtLaunchKernelGGL((k_bwd_chain<OT, DK, DV, 1, true>), grid, block, 0, stream, start, stop, 0, a);
        else
            hipExtLaunchKernelGGL((k_bwd_chain<OT, DK, DV, 1, false>), grid, block, 0, stream, start, stop, 0, a);
    }
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
