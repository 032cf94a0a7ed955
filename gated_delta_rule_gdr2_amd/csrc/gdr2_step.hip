// Recurrent (token-by-token) form of the Gated Delta Rule-2 operator on gfx950, for
// decoding with a constant-size state (chatpaper.ai abstract of "Gated DeltaNet-2":
// constant-memory decoding; anthology record LIT-802, takeaway 1, for the update):
//   S_t = (I - k_t (b_t * k_t)^T) diag(exp g_t) S_{t-1} + k_t (w_t * v_t)^T,
//   o_t = S_t^T q_t.
// With X = diag(exp g_t) S_{t-1} and u = X^T (b_t * k_t) the update is the rank-one
// correction S_t = X + k_t (w_t * v_t - u)^T, and the readout o_t = S_t^T q_t.
//
// k_step: one workgroup of two waves per (sequence, 64-column slice of the value axis).
// The state slice stays in registers in fp32 for all tokens of the call: lane l of wave
// w holds columns 64 j + 32 w + 4 (l % 8) .. + 3 of rows l / 8 + 8 i (i < d_k / 8), so
// each row segment a wave loads or stores is one 128-byte line. Per token the key-side
// vectors (k, b*k, q, exp g) and the slice's v, w are staged in LDS (the next token's
// are loaded while this one is computed); the two sums over the key axis (u and o) are
// in-lane over the lane's rows and then over the 8 row groups with lane shuffles.
// Gates passed as logits (ACT) are activated as they are staged.
#include "gdr2_device.hpp"
#include "gdr2_kernels.hpp"

namespace gdr2 {

constexpr int STEP_COLS = 64;  // value columns per workgroup

__device__ __forceinline__ f32x4 xor_sum_rows(f32x4 x) {  // sum over lanes l ^ 8, 16, 32
#pragma unroll
    for (int m = 8; m < 64; m <<= 1)
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] += __shfl_xor(x[j], m, 64);
    return x;
}

template <class OT, int DK, int DV, bool ACT, bool NT>
__global__ __launch_bounds__(128) void k_step(Args a) {
    constexpr int NI = DK / 8;  // state rows per lane
    __shared__ float sk[2][4][DK];             // per token: k, b*k, q, exp(g)
    __shared__ float sv[2][2][STEP_COLS];      // per token: v, w of the slice
    poison_lds((lds_char*)sk, sizeof(sk));
    poison_lds((lds_char*)sv, sizeof(sv));
    poison_lds_done();
    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, cq = l & 7, rg = l >> 3;
    const int NJ = DV / STEP_COLS;
    const int s = blockIdx.x / NJ, js = blockIdx.x % NJ;
    const int bidx = s / a.H, h = s % a.H;
    const int col = STEP_COLS * js + 32 * wv + 4 * cq;  // first of this lane's 4 columns
    float* hs = a.state + (size_t)s * DK * DV + col;

    f32x4 S[NI];  // S[i]: row rg + 8 i, columns col .. col + 3
#pragma unroll
    for (int i = 0; i < NI; ++i) S[i] = *(const f32x4*)(hs + (size_t)(rg + 8 * i) * DV);

    // this thread's share of a token's vectors: key channel tid (< DK), value column tid
    auto load = [&](int t, float (&x)[6]) {
        const size_t row = ((size_t)bidx * a.T + t) * a.H + h;
        if (tid < DK) {
            x[0] = to_f(((const OT*)a.k)[row * DK + tid]);
            x[1] = to_f(((const OT*)a.b)[row * DK + tid]);
            x[2] = to_f(((const OT*)a.q)[row * DK + tid]);
            x[3] = to_f(((const OT*)a.g)[row * DK + tid]);
        }
        if (tid < STEP_COLS) {
            x[4] = to_f(((const OT*)a.v)[row * DV + STEP_COLS * js + tid]);
            x[5] = to_f(((const OT*)a.w)[row * DV + STEP_COLS * js + tid]);
        }
    };
    float x[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    load(0, x);
    for (int t = 0; t < a.T; ++t) {
        const int p = t & 1;
        if (tid < DK) {
            const float b = ACT ? gate_act<OT, GATE_B>(x[1], a.g_scale, a.b_scale) : x[1];
            const float g = ACT ? gate_act<OT, GATE_G>(x[3], a.g_scale, a.b_scale) : x[3];
            sk[p][0][tid] = x[0];
            sk[p][1][tid] = b * x[0];
            sk[p][2][tid] = x[2];
            sk[p][3][tid] = __expf(g);
        }
        if (tid < STEP_COLS) {
            sv[p][0][tid] = x[4];
            sv[p][1][tid] = ACT ? gate_act<OT, GATE_W>(x[5], a.g_scale, a.b_scale) : x[5];
        }
        __syncthreads();  // token t staged; token t - 1's buffer (the other one) is free
        if (t + 1 < a.T) load(t + 1, x);
        // decay and the erase read-out u = X^T (b * k)
        f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = rg + 8 * i;
            const float e = sk[p][3][r], bk = sk[p][1][r];
            S[i] *= e;
            u += bk * S[i];
        }
        u = xor_sum_rows(u);
        const int c0 = 32 * wv + 4 * cq;
        f32x4 d;  // w * v - u
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = sv[p][1][c0 + j] * sv[p][0][c0 + j] - u[j];
        // S = X + k d^T and the readout o = S^T q
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int r = rg + 8 * i;
            S[i] += sk[p][0][r] * d;
            o += sk[p][2][r] * S[i];
        }
        o = xor_sum_rows(o);
        if (rg == 0) {
            const float ov[4] = {o[0], o[1], o[2], o[3]};
            st4((OT*)a.o + (((size_t)bidx * a.T + t) * a.H + h) * DV + col, ov);
        }
    }
    // a large state goes back with non-temporal stores: it is not read again within the call,
    // and they stream to HBM faster (a 512 MB state updated in place: 0.177 against 0.217 ms
    // per call; non-temporal loads, by contrast, are slower); a state the Infinity Cache can
    // hold stays cached for the next call
#pragma unroll
    for (int i = 0; i < NI; ++i) store_out<NT>((f32x4*)(hs + (size_t)(rg + 8 * i) * DV), S[i]);
}

template <class OT, int DK, int DV>
static hipError_t launch_step_t(const Args& a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.B * a.H * (DV / STEP_COLS)));
    if (a.nt_out) {
        if (a.act)
            hipLaunchKernelGGL((k_step<OT, DK, DV, true, true>), grid, dim3(128), 0, stream, a);
        else
            hipLaunchKernelGGL((k_step<OT, DK, DV, false, true>), grid, dim3(128), 0, stream, a);
    } else {
        if (a.act)
            hipLaunchKernelGGL((k_step<OT, DK, DV, true, false>), grid, dim3(128), 0, stream, a);
        else
            hipLaunchKernelGGL((k_step<OT, DK, DV, false, false>), grid, dim3(128), 0, stream, a);
    }
    return hipGetLastError();
}

// A call without tokens: the state passes through unchanged (or starts at zero), a plain
// vectorised copy -- a kernel rather than a memset or copy command, so that a caller may
// capture the call in a HIP graph.
__global__ __launch_bounds__(256) void k_state_pass(f32x4* dst, const f32x4* src, long long n4) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long long)gridDim.x * 256)
        dst[i] = src ? src[i] : z;
}

hipError_t launch_state_pass(float* dst, const float* src, long long n, hipStream_t stream) {
    const long long n4 = n / 4, blocks = (n4 + 255) / 256;
    const dim3 grid((unsigned)(blocks < 1024 ? blocks : 1024));
    hipLaunchKernelGGL(k_state_pass, grid, dim3(256), 0, stream, (f32x4*)dst, (const f32x4*)src, n4);
    return hipGetLastError();
}

hipError_t launch_step(const Args& a, bool bf16_, hipStream_t stream) {
    const int DK = a.L.DK, DV = a.L.DV;
    if (bf16_) {
        if (DK == 64 && DV == 64) return launch_step_t<bf16, 64, 64>(a, stream);
        if (DK == 64 && DV == 128) return launch_step_t<bf16, 64, 128>(a, stream);
        if (DK == 128 && DV == 64) return launch_step_t<bf16, 128, 64>(a, stream);
        if (DK == 128 && DV == 128) return launch_step_t<bf16, 128, 128>(a, stream);
    } else {
        if (DK == 64 && DV == 64) return launch_step_t<float, 64, 64>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr2
