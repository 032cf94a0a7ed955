// Device-side building blocks for the Gated Delta Rule-2 kernels (gfx950 / CDNA4).
//
// MFMA conventions used by every kernel in this library
// -----------------------------------------------------
// All products are built from 16x16 output tiles with 32-deep K blocks:
//   bf16 operands : one v_mfma_f32_16x16x32_bf16 per K block,
//   fp32 operands : eight v_mfma_f32_16x16x4_f32 per K block.
// A wave holds an operand "fragment" of 8 elements per lane. Lane l = li + 16*lq
// (li = l % 16, lq = l / 16) holds, for an A operand, row li and the 8 K indices
//     kmap(lq, e) = 16*(e/4) + 4*lq + (e%4),   e = 0..7,
// and for a B operand column li with the same 8 K indices. The hardware sums
// over (lane group, element) pairs, so any K numbering is exact as long as A and
// B agree; this one is chosen because it matches the accumulator layout:
// an accumulator tile D (16x16, 4 fp32 per lane) holds D[4*lq + i][li], i = 0..3.
// Hence two vertically stacked accumulator tiles (rows 0..15 and 16..31 of a
// 32-row block) ARE, element for element, the B fragment of that 32-row block,
// and also the A fragment of its transpose. Sequential chains therefore keep
// their state in accumulator registers and feed it straight back into the next
// MFMA without any LDS round trip.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr2 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int CH = 64;    // chunk length (tokens)
constexpr int BLK = 16;   // sub-block for the exponent split and the blocked inverse
constexpr int NBLK = CH / BLK;
constexpr int NPAIR = NBLK * (NBLK + 1) / 2;  // lower-triangular 16x16 block pairs

template <class OT> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };
// four consecutive elements in the operand type (half a fragment, or one lane's share
// of an accumulator tile)
template <class OT> struct Raw4;
template <> struct Raw4<bf16> { typedef bf16x4 type; };
template <> struct Raw4<float> { typedef f32x4 type; };

__device__ __forceinline__ int kmap(int lq, int e) { return 16 * (e >> 2) + 4 * lq + (e & 3); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier after this wave's LDS operations have completed. Unlike
// __syncthreads it does not wait for the wave's global loads (or DMAs) in flight, so
// loads issued earlier keep running through it; LDS written by DMA must be waited for
// (wait_vm) before it.
__device__ __forceinline__ void sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


// pair index -> (R, I), I <= R, in the order (0,0),(1,0),(1,1),(2,0),...
__device__ __forceinline__ void pair_ri(int p, int& R, int& I) {
    R = (p >= 6) ? 3 : (p >= 3) ? 2 : (p >= 1) ? 1 : 0;
    I = p - R * (R + 1) / 2;
}
__device__ __host__ __forceinline__ int pair_id(int R, int I) { return R * (R + 1) / 2 + I; }

// ----------------------------------------------------------------------------- MMA
__device__ __forceinline__ void mma(f32x4& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
}
// fp32 product with a 16-deep K (the first half of the K-slot map: k = 4*lq + e)
__device__ __forceinline__ void mma_k16_f32(f32x4& acc, const float a[4], const float b[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
}
// Product over one half of the K slots of two 32-deep fragments: half H holds the K
// indices 16 H + 4*lq + e (e < 4), one 16-row block of the K axis.
template <int H>
__device__ __forceinline__ void mma_half(f32x4& acc, const bf16x8& a, const bf16x8& b) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 ah = __builtin_shufflevector(a, a, 4 * H, 4 * H + 1, 4 * H + 2, 4 * H + 3);
    const bf16x4 bh = __builtin_shufflevector(b, b, 4 * H, 4 * H + 1, 4 * H + 2, 4 * H + 3);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, ah), __builtin_bit_cast(s16x4, bh), acc,
                                                    0, 0, 0);
}
template <int H>
__device__ __forceinline__ void mma_half(f32x4& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * H + e], b[4 * H + e], acc, 0, 0, 0);
}

// ----------------------------------------------------------------------------- conversions
template <class OT> __device__ __forceinline__ OT to_ot(float x);
template <> __device__ __forceinline__ bf16 to_ot<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float to_ot<float>(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }

// fragment from two accumulator tiles (rows 0..15 -> e 0..3, rows 16..31 -> e 4..7)
template <class OT>
__device__ __forceinline__ typename Frag<OT>::type frag_of(const f32x4& d0, const f32x4& d1) {
    typename Frag<OT>::type f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = to_ot<OT>(d0[i]);
        f[4 + i] = to_ot<OT>(d1[i]);
    }
    return f;
}

// ----------------------------------------------------------------------------- 4-element vectors
// load / store 4 consecutive elements (8 B for bf16, 16 B for fp32); p must be aligned
// Gate activations, for gates passed as logits. The erase gate b and the write gate w
// are sigmoids of their own projections (Gated DeltaNet-2 record LIT-802, "Key
// takeaways", first bullet), b scaled by b_scale > 0 (2: the [0, 2] erase range of the
// Table 5 ablation); the log-decay is g = -g_scale * softplus(z), which keeps
// exp g in (0, 1). The fp32 operand path takes the accurate library exp / log1p, the bf16
// path the hardware approximations (their error is far below bf16 rounding).
template <class OT>
__device__ __forceinline__ float gate_sigmoid(float z) {
    if constexpr (sizeof(OT) == 4) return 1.f / (1.f + expf(-z));
    else return __builtin_amdgcn_rcpf(1.f + __expf(-z));
}
template <class OT>
__device__ __forceinline__ float gate_softplus(float z) {
    if constexpr (sizeof(OT) == 4) return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
    else return fmaxf(z, 0.f) + __logf(1.f + __expf(-fabsf(z)));
}
// softplus(z) and sigmoid(z) from one exponential: with e = exp(-|z|),
// softplus = max(z, 0) + log(1 + e) and sigmoid = 1 / (1 + e) (z >= 0) or e / (1 + e)
template <class OT>
__device__ __forceinline__ void gate_softplus_sigmoid(float z, float& sp, float& sg) {
    const float e = sizeof(OT) == 4 ? expf(-fabsf(z)) : __expf(-fabsf(z));
    sp = fmaxf(z, 0.f) + (sizeof(OT) == 4 ? log1pf(e) : __logf(1.f + e));
    const float r = sizeof(OT) == 4 ? 1.f / (1.f + e) : __builtin_amdgcn_rcpf(1.f + e);
    sg = z >= 0.f ? r : e * r;
}
// exp in the operand path's precision: the accurate library exp for fp32 operands, the
// hardware approximation for bf16 (its error is far below bf16 rounding)
template <class OT>
__device__ __forceinline__ float exp_op(float x) {
    if constexpr (sizeof(OT) == 4) return expf(x);
    else return __expf(x);
}
enum GateKind { GATE_G, GATE_B, GATE_W };
template <class OT, int KIND>
__device__ __forceinline__ float gate_act(float z, float g_scale, float b_scale) {
    if constexpr (KIND == GATE_G) return -g_scale * gate_softplus<OT>(z);
    else if constexpr (KIND == GATE_B) return b_scale * gate_sigmoid<OT>(z);
    else return gate_sigmoid<OT>(z);
}

__device__ __forceinline__ void ld4(const bf16* p, float out[4]) {
    bf16x4 v = *(const bf16x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = (float)v[i];
}
__device__ __forceinline__ void ld4(const float* p, float out[4]) {
    f32x4 v = *(const f32x4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = v[i];
}
__device__ __forceinline__ void st4(bf16* p, const float in[4]) {
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (bf16)in[i];
    *(bf16x4*)p = v;
}
__device__ __forceinline__ void st4(float* p, const float in[4]) {
    f32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = in[i];
    *(f32x4*)p = v;
}

// Non-temporal variants, for results that another kernel reads later (the per-chunk
// operands the forward intra-chunk kernel leaves for the chains, the backward chain's
// outputs, the gradients), used when the problem's data is large next to the Infinity
// Cache (Args::nt_out). Measured on MI355X: at the 4096-token training shape (176 MB of
// per-chunk operands) the hint speeds up the kernels that come after -- the forward chain
// that reads the operands takes about 10 % less time, the whole step about 5 % -- while at
// 2048 tokens x 16 heads forward-only (37 MB, which the cache holds) plain stores are 11 %
// faster. The forward chain's own outputs are faster with plain stores at every size.
__device__ __forceinline__ void st4_nt(bf16* p, const float in[4]) {
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (bf16)in[i];
    __builtin_nontemporal_store(v, (bf16x4*)p);
}
__device__ __forceinline__ void st4_nt(float* p, const float in[4]) {
    f32x4 v = {in[0], in[1], in[2], in[3]};
    __builtin_nontemporal_store(v, (f32x4*)p);
}
// NT is a compile-time choice (the kernels are instantiated both ways): with a run-time
// branch the compiler merges the two stores into one and drops the non-temporal hint.
template <bool NT, class OT>
__device__ __forceinline__ void st4_out(OT* p, const float in[4]) {
    if constexpr (NT)
        st4_nt(p, in);
    else
        st4(p, in);
}
template <bool NT, class T>
__device__ __forceinline__ void store_out(T* p, const T& v) {
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}
// Load with the non-temporal hint as a compile-time choice, for data that nothing reads
// after this load (it then does not displace other data from the caches).
template <bool NT, class T>
__device__ __forceinline__ T load_in(const T* p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

// ----------------------------------------------------------------------------- fragment loads
// "rowk": lane (li, lq) reads X[row0 + li][k0 + kmap(lq, e)] -- contiguous along K
// (two runs of four). X is row-major with leading dimension ld (elements).
template <class OT>
__device__ __forceinline__ typename Frag<OT>::type frag_rowk(const OT* X, int ld, int row0, int k0) {
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    const OT* p = X + (size_t)(row0 + li) * ld + k0 + 4 * lq;
    if constexpr (sizeof(OT) == 2) {
        bf16x4 x0 = *(const bf16x4*)p, x1 = *(const bf16x4*)(p + 16);
        return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
        f32x4 x0 = *(const f32x4*)p, x1 = *(const f32x4*)(p + 16);
        return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}
// Fragment-major layout of a matrix with DV columns (rows a multiple of 16): its rowk8
// fragments (below) one after another. Fragment (at, kb) -- rows 16 at .. + 15, columns
// 32 kb .. + 31 -- is a block of 64 lanes x 8 elements, lane 16 lq + li holding row
// 16 at + li, columns 32 kb + 8 lq .. + 7, so a wave reads a fragment as one contiguous
// block (one 16-byte load per lane for bf16).
template <int DV>
__device__ __forceinline__ size_t fmaj_off(int r, int c) {
    return ((size_t)((r >> 4) * (DV / 32) + (c >> 5)) * 64 + ((c >> 3) & 3) * 16 + (r & 15)) * 8 + (c & 7);
}
// (NT: a non-temporal load, for data read for the last time)
template <class OT, int DV, bool NT = false>
__device__ __forceinline__ typename Frag<OT>::type frag_fmaj(const OT* X, int at, int kb) {
    const OT* p = X + ((size_t)(at * (DV / 32) + kb) * 64 + lane_id()) * 8;
    if constexpr (sizeof(OT) == 2) {
        return load_in<NT>((const bf16x8*)p);
    } else {
        f32x4 x0 = load_in<NT>((const f32x4*)p), x1 = load_in<NT>((const f32x4*)(p + 4));
        return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}
// "rowk8": the contiguous K-slot map k = k0 + 8*lq + e. Usable for a product only when
// both operands are read from memory with it (never with an accumulator-derived
// operand): lane (li, lq) reads X[row0 + li][k0 + 8*lq .. + 7], one 16-byte piece for
// bf16.
template <class OT>
__device__ __forceinline__ typename Frag<OT>::type frag_rowk8(const OT* X, int ld, int row0, int k0) {
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    const OT* p = X + (size_t)(row0 + li) * ld + k0 + 8 * lq;
    if constexpr (sizeof(OT) == 2) {
        return *(const bf16x8*)p;
    } else {
        f32x4 x0 = *(const f32x4*)p, x1 = *(const f32x4*)(p + 4);
        return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}
// rowk from an fp32 matrix, converted to the operand type
template <class OT>
__device__ __forceinline__ typename Frag<OT>::type frag_rowk_f32(const float* X, int ld, int row0, int k0) {
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    const float* p = X + (size_t)(row0 + li) * ld + k0 + 4 * lq;
    typename Frag<OT>::type f;
    float a[4], b[4];
    ld4(p, a);
    ld4(p + 16, b);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = to_ot<OT>(a[i]);
        f[4 + i] = to_ot<OT>(b[i]);
    }
    return f;
}
// rowk with a per-K-index scale (scale[k0 + kmap] multiplies element e)
template <class OT, class XT>
__device__ __forceinline__ typename Frag<OT>::type frag_rowk_scaled(const XT* X, int ld, int row0, int k0,
                                                                    const float* scale) {
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    const XT* p = X + (size_t)(row0 + li) * ld + k0 + 4 * lq;
    const float* s = scale + k0 + 4 * lq;
    typename Frag<OT>::type f;
    float a[4], b[4], sa[4], sb[4];
    ld4(p, a);
    ld4(p + 16, b);
    ld4(s, sa);
    ld4(s + 16, sb);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = to_ot<OT>(a[i] * sa[i]);
        f[4 + i] = to_ot<OT>(b[i] * sb[i]);
    }
    return f;
}
// "colk": lane (li, lq) reads X[k0 + kmap(lq, e)][col0 + li] -- strided along K.
// rs0 / rs1 scale the elements of the first / second 16-row half of the K block.
template <class OT, class XT>
__device__ __forceinline__ typename Frag<OT>::type frag_colk(const XT* X, int ld, int col0, int k0,
                                                             float rs0 = 1.f, float rs1 = 1.f) {
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    const XT* p = X + (size_t)(k0 + 4 * lq) * ld + col0 + li;
    typename Frag<OT>::type f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = to_ot<OT>(to_f(p[(size_t)i * ld]) * rs0);
        f[4 + i] = to_ot<OT>(to_f(p[(size_t)(16 + i) * ld]) * rs1);
    }
    return f;
}

// ----------------------------------------------------------------------------- LDS address space
typedef __attribute__((address_space(3))) char lds_char;

// Debug builds with -DGDR2_POISON_LDS: a kernel first fills its LDS with all-ones bytes (a
// NaN in bf16 and in fp32), so that a read of LDS that no write has reached turns the
// results into NaN. poison_lds fills one region; poison_lds_done ends the fill with a
// barrier of the whole workgroup. Without the flag both are empty.
__device__ __forceinline__ void poison_lds(lds_char* p, int bytes) {
#ifdef GDR2_POISON_LDS
    typedef __attribute__((address_space(3))) unsigned U32;
    U32* q = (U32*)p;
    for (int i = threadIdx.x; i < bytes / 4; i += blockDim.x) q[i] = 0xFFFFFFFFu;
#else
    (void)p;
    (void)bytes;
#endif
}
__device__ __forceinline__ void poison_lds_done() {
#ifdef GDR2_POISON_LDS
    __syncthreads();
#endif
}
typedef __attribute__((address_space(3))) void lds_void;

template <class T>
__device__ __forceinline__ T lds_load(const lds_char* p) {
    typedef __attribute__((address_space(3))) const T TA;
    return *(const TA*)p;
}
template <class T>
__device__ __forceinline__ void lds_store(lds_char* p, const T& v) {
    typedef __attribute__((address_space(3))) T TA;
    *(TA*)p = v;
}

// Swizzled row-major tiles. A matrix with RL elements per row is stored row by
// row, but the 16-byte chunks of row r are permuted: chunk c sits at position
// c ^ f(r). f is chosen so that the LDS reads of the MFMA fragments are free of
// bank conflicts although rows are not padded. The gfx950 LDS, as measured with
// timing probes of fixed lane patterns: 64 banks of 4 bytes (address / 4 mod 64);
// a 16-byte read is served in four passes of 16 lanes, lanes 0-3, 12-15, 20-23,
// 24-27 in one pass, 4-7, 8-11, 16-19, 28-31 in the next (the same for lanes
// 32-63); 8-byte reads, plain or transposing, in two passes of 32 lanes (0-31,
// 32-63). A pass is conflict-free when its lanes' addresses cover distinct banks
// (lanes reading the same word share it). The patterns used:
//   row reads         : rows R0 + li (li = lane % 16), chunk c + lane / 16, 16 bytes;
//   transposing reads : rows k0 + 4 (lane / 16) + li / 4 (or k0 + 8 (lane / 16) +
//                       li / 4, twice, 4 rows apart), chunks 2j, 2j + 1, 8 bytes;
//   row pieces        : rows R0 + li, 4 elements of one chunk, 8 or 16 bytes.
// f is linear over the bits of r (so the cost depends only on r mod 16):
//   16 chunks per row (256-byte rows, one bank period): f(r) = 2 (r mod 8) XOR 13 b3;
//   8 chunks per row (128-byte rows): f(r) = 2 (r / 2 mod 4) XOR 5 b3;
// b3 = bit 3 of r. Under the pass structure above both are conflict-free for every
// one of these patterns, in bf16 and in fp32 (the "plain bijection on 16 rows"
// swizzle 2 (r mod 8) + b3 costs the row reads a 2-way conflict in every pass).
// A tile is copied into LDS verbatim by DMA and read back with these views.
template <class OT, int RL>
__device__ __forceinline__ int swz_f(int r) {  // chunk permutation of row r
    constexpr int NCH = RL * (int)sizeof(OT) / 16;  // chunks per row
    static_assert(NCH == 8 || NCH == 16, "swizzled tiles have 8 or 16 chunks per row");
    const int b3 = (r >> 3) & 1;
    return NCH == 16 ? (((r & 7) << 1) ^ (13 * b3)) : ((((r >> 1) & 3) << 1) ^ (5 * b3));
}
template <class OT, int RL>
__device__ __forceinline__ int swz(int r, int c) {
    constexpr int EPC = 16 / (int)sizeof(OT);  // elements per 16-byte chunk
    return r * RL + (((c / EPC) ^ swz_f<OT, RL>(r)) * EPC) + (c % EPC);
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16). Within each 16-lane group the
// hardware returns result[k][e] = src[4e + k/4][k%4], where src[s] are the four
// 16-bit values lane s addressed. Hence, if lane (li, lq) addresses row
// k0 + 4*lq + li/4, columns c0 + 4*(li%4) .. +3 of a row-major bf16 matrix, it
// receives X[k0 + 4*lq + e][c0 + li], e = 0..3: one half of a fragment whose K
// index runs down the rows.
__device__ __forceinline__ bf16x4 lds_read_tr16(const lds_char* p) {
    typedef __attribute__((address_space(3))) bf16x4 T4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((T4*)p);
}

// ----------------------------------------------------------------------------- LDS fragment reads
// Views of a matrix held in LDS: element (r, c) lives at byte offset off(r, c).
template <class XT>
struct LPad {  // padded row-major, leading dimension ld (elements)
    const lds_char* p;
    int ld;
    __device__ __forceinline__ int off(int r, int c) const { return (r * ld + c) * (int)sizeof(XT); }
};
template <class XT, int RL>
struct LSwz {  // swizzled tile with RL elements per row
    const lds_char* p;
    __device__ __forceinline__ int off(int r, int c) const { return swz<XT, RL>(r, c) * (int)sizeof(XT); }
};

template <class XT>
__device__ __forceinline__ void lds_get4(const lds_char* p, float out[4]) {
    if constexpr (sizeof(XT) == 2) {
        bf16x4 v = lds_load<bf16x4>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = (float)v[i];
    } else {
        f32x4 v = lds_load<f32x4>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = v[i];
    }
}
template <class XT>
__device__ __forceinline__ float lds_get1(const lds_char* p) {
    if constexpr (sizeof(XT) == 2)
        return (float)lds_load<bf16>(p);
    else
        return lds_load<float>(p);
}

// rowk: lane (li, lq) gets X[row0 + li][k0 + kmap(lq, e)]. When the stored type is the
// operand type and no scale is applied the fragment is assembled from the two raw
// loads without any conversion.
template <class OT, class XT, class V>
__device__ __forceinline__ typename Frag<OT>::type lfrag_rowk(const V& m, int row0, int k0,
                                                              const lds_char* kscale = nullptr) {
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    const int r = row0 + li;
    const lds_char* p0 = m.p + m.off(r, k0 + 4 * lq);
    const lds_char* p1 = m.p + m.off(r, k0 + 16 + 4 * lq);
    if constexpr (sizeof(XT) == sizeof(OT)) {
        if (!kscale) {
            if constexpr (sizeof(OT) == 2) {
                bf16x4 x0 = lds_load<bf16x4>(p0), x1 = lds_load<bf16x4>(p1);
                return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
                f32x4 x0 = lds_load<f32x4>(p0), x1 = lds_load<f32x4>(p1);
                return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
    }
    float a[4], b[4];
    lds_get4<XT>(p0, a);
    lds_get4<XT>(p1, b);
    if (kscale) {
        float sa[4], sb[4];
        lds_get4<float>(kscale + (k0 + 4 * lq) * 4, sa);
        lds_get4<float>(kscale + (k0 + 16 + 4 * lq) * 4, sb);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[i] *= sa[i];
            b[i] *= sb[i];
        }
    }
    typename Frag<OT>::type f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = to_ot<OT>(a[i]);
        f[4 + i] = to_ot<OT>(b[i]);
    }
    return f;
}
// rowk8 (contiguous K-slot map, see frag_rowk8) from a matrix in LDS of the operand type
template <class OT, class V>
__device__ __forceinline__ typename Frag<OT>::type lfrag_rowk8(const V& m, int row0, int k0) {
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    const lds_char* p0 = m.p + m.off(row0 + li, k0 + 8 * lq);
    if constexpr (sizeof(OT) == 2) {
        return lds_load<bf16x8>(p0);
    } else {
        const lds_char* p1 = m.p + m.off(row0 + li, k0 + 8 * lq + 4);
        f32x4 x0 = lds_load<f32x4>(p0), x1 = lds_load<f32x4>(p1);
        return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}
// colk: lane (li, lq) gets X[k0 + kmap(lq, e)][col0 + li], optionally scaled by rs0 (e < 4)
// and rs1 (e >= 4). bf16: two transposing reads; fp32: eight scalar reads.
template <class OT, class XT, class V>
__device__ __forceinline__ typename Frag<OT>::type lfrag_colk(const V& m, int col0, int k0) {
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    if constexpr (sizeof(XT) == 2 && sizeof(OT) == 2) {
        const int r = k0 + 4 * lq + (li >> 2), c = col0 + 4 * (li & 3);
        bf16x4 v0 = lds_read_tr16(m.p + m.off(r, c));
        bf16x4 v1 = lds_read_tr16(m.p + m.off(r + 16, c));
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
        typename Frag<OT>::type f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[e] = to_ot<OT>(lds_get1<XT>(m.p + m.off(k0 + 4 * lq + e, col0 + li)));
            f[4 + e] = to_ot<OT>(lds_get1<XT>(m.p + m.off(k0 + 16 + 4 * lq + e, col0 + li)));
        }
        return f;
    }
}
template <class OT, class XT, class V>
__device__ __forceinline__ typename Frag<OT>::type lfrag_colk(const V& m, int col0, int k0, float rs0, float rs1) {
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    typename Frag<OT>::type f;
    if constexpr (sizeof(XT) == 2) {
        const int r = k0 + 4 * lq + (li >> 2), c = col0 + 4 * (li & 3);
        bf16x4 v0 = lds_read_tr16(m.p + m.off(r, c));
        bf16x4 v1 = lds_read_tr16(m.p + m.off(r + 16, c));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[e] = to_ot<OT>((float)v0[e] * rs0);
            f[4 + e] = to_ot<OT>((float)v1[e] * rs1);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[e] = to_ot<OT>(lds_get1<XT>(m.p + m.off(k0 + 4 * lq + e, col0 + li)) * rs0);
            f[4 + e] = to_ot<OT>(lds_get1<XT>(m.p + m.off(k0 + 16 + 4 * lq + e, col0 + li)) * rs1);
        }
    }
    return f;
}

// colk8: the contiguous K-slot map (k = k0 + 8*lq + e, as rowk8) over a matrix whose K
// index runs down the rows: lane (li, lq) gets X[k0 + 8*lq + e][col0 + li], e = 0..7.
// bf16: two transposing reads (rows k0 + 8 lq .. + 3 and + 4 .. + 7); fp32: eight scalar reads.
template <class OT, class V>
__device__ __forceinline__ typename Frag<OT>::type lfrag_colk8(const V& m, int col0, int k0) {
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    if constexpr (sizeof(OT) == 2) {
        const int r = k0 + 8 * lq + (li >> 2), c = col0 + 4 * (li & 3);
        bf16x4 v0 = lds_read_tr16(m.p + m.off(r, c));
        bf16x4 v1 = lds_read_tr16(m.p + m.off(r + 4, c));
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
        typename Frag<OT>::type f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = lds_load<float>(m.p + m.off(k0 + 8 * lq + e, col0 + li));
        return f;
    }
}

// ----------------------------------------------------------------------------- global fragments
// A fragment block (one 16x32 operand) is stored lane-major: 64 lanes x 8 elements.
template <class OT>
__device__ __forceinline__ void store_frag(OT* base, const typename Frag<OT>::type& f) {
    *(typename Frag<OT>::type*)(base + lane_id() * 8) = f;
}
template <class OT>
__device__ __forceinline__ typename Frag<OT>::type load_frag(const OT* base) {
    return *(const typename Frag<OT>::type*)(base + lane_id() * 8);
}
// Fragment image of a matrix X [R][K] (K contiguous, R and K multiples of 16 and 32):
// X stored as its row-K MFMA operand fragments, fragment (r / 16, c / 32) after
// fragment, each as P pieces of 64 x 16 bytes (P = 1 for bf16, 2 for fp32). Lane
// (li, lq) of a fragment holds X[16 rb + li][32 kb + 8 lq + e], e = 0..7, in 16-byte
// slot 16 lq + (li ^ 4 (lq & 1)) of each piece. A fragment is hence one contiguous
// 1 KB load per piece from global memory, and in LDS the transposing reads (16 lanes
// on 4 consecutive rows x 2 adjacent column groups of 4) touch 8 slots in two 64-byte
// runs 256 + 64 bytes apart, which share no bank; 4 consecutive columns starting at a
// multiple of 4 are contiguous.
template <class OT, int K>
__host__ __device__ __forceinline__ int fimg(int r, int c) {
    constexpr int EPP = 16 / (int)sizeof(OT);  // elements per 16-byte piece
    constexpr int P = 8 / EPP;                 // pieces per lane and fragment
    static_assert(K % 32 == 0, "fragment images have whole 32-column blocks");
    const int lq = (c >> 3) & 3;
    const int slot = 16 * lq + ((r & 15) ^ (4 * (lq & 1)));
    const int frag = (r >> 4) * (K / 32) + (c >> 5);
    return ((frag * P + (c & 7) / EPP) * 64 + slot) * EPP + (c & 7) % EPP;
}
template <class XT, int K>
struct LImg {  // fragment image in LDS
    const lds_char* p;
    __device__ __forceinline__ int off(int r, int c) const { return fimg<XT, K>(r, c) * (int)sizeof(XT); }
};
// A row-K fragment (lane (li, lq): X[row0 + li][k0 + 8 lq + e]) stored into a fragment image
// in global memory: one contiguous kilobyte per piece (NT: non-temporal, see st4_nt).
template <class OT, int K, bool NT>
__device__ __forceinline__ void store_frag_img(OT* m, int row0, int k0, const typename Frag<OT>::type& f) {
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    if constexpr (sizeof(OT) == 2) {
        store_out<NT>((bf16x8*)(m + fimg<OT, K>(row0 + li, k0 + 8 * lq)), f);
    } else {
        const f32x4 x0 = __builtin_shufflevector(f, f, 0, 1, 2, 3), x1 = __builtin_shufflevector(f, f, 4, 5, 6, 7);
        store_out<NT>((f32x4*)(m + fimg<OT, K>(row0 + li, k0 + 8 * lq)), x0);
        store_out<NT>((f32x4*)(m + fimg<OT, K>(row0 + li, k0 + 8 * lq + 4)), x1);
    }
}
// Row-K fragment (as lfrag_rowk8) read straight from a fragment image in global memory.
template <class OT, int K>
__device__ __forceinline__ typename Frag<OT>::type gfrag_img(const OT* m, int row0, int k0) {
    const int l = lane_id(), li = l & 15, lq = l >> 4;
    if constexpr (sizeof(OT) == 2) {
        return *(const bf16x8*)(m + fimg<OT, K>(row0 + li, k0 + 8 * lq));
    } else {
        const f32x4 x0 = *(const f32x4*)(m + fimg<OT, K>(row0 + li, k0 + 8 * lq));
        const f32x4 x1 = *(const f32x4*)(m + fimg<OT, K>(row0 + li, k0 + 8 * lq + 4));
        return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}
// accumulator tile dump: 64 lanes x 4 elements (NT: non-temporal, see st4_nt)
template <class OT, bool NT = false>
__device__ __forceinline__ void store_tile(OT* base, const f32x4& d) {
    float t[4] = {d[0], d[1], d[2], d[3]};
    st4_out<NT>(base + lane_id() * 4, t);
}
template <class OT>
__device__ __forceinline__ f32x4 load_tile(const OT* base) {
    float t[4];
    ld4(base + lane_id() * 4, t);
    f32x4 d = {t[0], t[1], t[2], t[3]};
    return d;
}

// ----------------------------------------------------------------------------- wave scans
// inclusive prefix sum across the 16 lanes of each DPP row (lanes li = 0..15)
__device__ __forceinline__ float row_scan16(float x) {
    int v;
    v = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __int_as_float(v);
    v = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __int_as_float(v);
    v = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __int_as_float(v);
    v = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __int_as_float(v);
    return x;
}
// inclusive suffix sum across the 16 lanes of each DPP row (lane li gets the sum over
// lanes li .. 15)
__device__ __forceinline__ float row_suffix16(float x) {
    int v;
    v = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x101, 0xF, 0xF, false);  // row_shl:1
    x += __int_as_float(v);
    v = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x102, 0xF, 0xF, false);  // row_shl:2
    x += __int_as_float(v);
    v = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x104, 0xF, 0xF, false);  // row_shl:4
    x += __int_as_float(v);
    v = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x108, 0xF, 0xF, false);  // row_shl:8
    x += __int_as_float(v);
    return x;
}
// value of the next lane of the row (lane 15 gets 0): with row_suffix16 an exclusive suffix
// sum that never subtracts
__device__ __forceinline__ float row_shl1(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x101, 0xF, 0xF, false));
}
// value of the previous lane of the row (lane 0 gets 0): with row_scan16 an exclusive prefix
// sum that never subtracts
__device__ __forceinline__ float row_shr1(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, false));
}
// value held by lane SRC of the caller's 16-lane row (DPP row_newbcast, a VALU move)
template <int SRC>
__device__ __forceinline__ float row_bcast(float x) {
    static_assert(SRC >= 0 && SRC < 16, "a row has 16 lanes");
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + SRC, 0xF, 0xF, false));
}
// sum over the 16 lanes of a row (result in every lane of the row)
__device__ __forceinline__ float row_sum16(float x) {
    float s = row_scan16(x);
    return row_bcast<15>(s);
}

}  // namespace gdr2
