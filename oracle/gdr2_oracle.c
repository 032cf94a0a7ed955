/*
 * Gated Delta Rule-2 (GDR-2) reference oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously-correct fp64 CPU definition of the operator. Only the
 * test suite, the package smoke check and the CPU-baseline leg of the benchmark
 * may load this file's library. The product path (the HIP library) never links,
 * calls or reads it, and it shares no code with it.
 *
 * Source of the definition ("Gated DeltaNet-2: Decoupling Erase and Write in
 * Linear Attention", Hatamizadeh, Choi and Kautz, 2026):
 *   - state update: anthology record LIT-802, "Key takeaways", first bullet
 *     (paper Sec. 3.1, Eqs. 8-10): S_t = (I - k_t (b_t * k_t)^T) D_t S_{t-1}
 *     + k_t (w_t * v_t)^T, D_t = diag(alpha_t). The same equation appears in
 *     the wispaper.ai summary, "Methodology" section, with the transpose
 *     extracted as "{)}^{o}p".
 *   - the read happens along b_t * k_t and the write along k_t (same bullet).
 *   - D_t multiplies S_{t-1} before the erase factor (operator order of the
 *     printed equation).
 *   - channel-wise decay on the key axis inherited from KDA (LIT-802,
 *     "Standing in the anthology").
 * Readings taken where the pages are silent (each is restated in the design
 * notes of the repository):
 *   - readout o_t = S_t^T q_t, taken after the update, no scale;
 *   - alpha_t = exp(g_t) with g_t the caller's log-decay, no clamping;
 *   - the gates b_t, w_t arrive already activated; nothing is normalised here.
 *
 * The backward pass is back-propagation through the token loop, derived by
 * hand from the forward steps below (one adjoint per forward step, in reverse
 * order). States are checkpointed every ORACLE_CKPT tokens and recomputed
 * inside each segment.
 *
 * Layouts (row-major, contiguous):
 *   q, k, g, b and their gradients: [B][T][H][DK]
 *   v, w, o, dout and their gradients: [B][T][H][DV]
 *   h0, ht, dht, dh0: [B][H][DK][DV]
 * Nullable: h0 (means 0), ht (not written), dht (means 0), dh0 (not written).
 *
 * Parallelism: OpenMP over the B*H independent sequences; each sequence runs
 * the plain token loop.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_CKPT 64

static inline size_t idx_tok(int bb, int t, int h, int d, int T, int H, int D) {
    return (((size_t)bb * T + t) * H + h) * (size_t)D + d;
}

/* One forward token step on a single sequence.
 * S (DK x DV, in/out): S_{t-1} on entry, S_t on exit.
 * Steps, in the order of the state equation:
 *   1. alpha = exp(g)              decay factors (key axis)
 *   2. P = diag(alpha) S           decay applied first
 *   3. c = b * k                   erase/read address
 *   4. r = P^T c                   what the erase address currently returns
 *   5. x = w * v ; u = x - r       gated write value minus the read
 *   6. S = P + k u^T               write along k
 */
static void token_step(int DK, int DV, const double* qt, const double* kt,
                       const double* vt, const double* gt, const double* bt,
                       const double* wt, double* S, double* r, double* u) {
    (void)qt;
    for (int i = 0; i < DK; ++i) {
        double a = exp(gt[i]);
        for (int j = 0; j < DV; ++j) S[i * DV + j] *= a;
    }
    for (int j = 0; j < DV; ++j) r[j] = 0.0;
    for (int i = 0; i < DK; ++i) {
        double c = bt[i] * kt[i];
        for (int j = 0; j < DV; ++j) r[j] += S[i * DV + j] * c;
    }
    for (int j = 0; j < DV; ++j) u[j] = wt[j] * vt[j] - r[j];
    for (int i = 0; i < DK; ++i)
        for (int j = 0; j < DV; ++j) S[i * DV + j] += kt[i] * u[j];
}

void gdr2_oracle_fwd(int B, int T, int H, int DK, int DV,
                     const double* q, const double* k, const double* v,
                     const double* g, const double* b, const double* w,
                     const double* h0, double* o, double* ht) {
    int nseq = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int s = 0; s < nseq; ++s) {
        int bb = s / H, h = s % H;
        double* S = (double*)malloc(sizeof(double) * DK * DV);
        double* r = (double*)malloc(sizeof(double) * DV);
        double* u = (double*)malloc(sizeof(double) * DV);
        if (h0)
            memcpy(S, h0 + (size_t)s * DK * DV, sizeof(double) * DK * DV);
        else
            memset(S, 0, sizeof(double) * DK * DV);
        for (int t = 0; t < T; ++t) {
            const double* qt = q + idx_tok(bb, t, h, 0, T, H, DK);
            const double* kt = k + idx_tok(bb, t, h, 0, T, H, DK);
            const double* gt = g + idx_tok(bb, t, h, 0, T, H, DK);
            const double* bt = b + idx_tok(bb, t, h, 0, T, H, DK);
            const double* vt = v + idx_tok(bb, t, h, 0, T, H, DV);
            const double* wt = w + idx_tok(bb, t, h, 0, T, H, DV);
            token_step(DK, DV, qt, kt, vt, gt, bt, wt, S, r, u);
            /* 7. readout after the update: o_t = S_t^T q_t */
            double* ot = o + idx_tok(bb, t, h, 0, T, H, DV);
            for (int j = 0; j < DV; ++j) ot[j] = 0.0;
            for (int i = 0; i < DK; ++i)
                for (int j = 0; j < DV; ++j) ot[j] += S[i * DV + j] * qt[i];
        }
        if (ht) memcpy(ht + (size_t)s * DK * DV, S, sizeof(double) * DK * DV);
        free(S);
        free(r);
        free(u);
    }
}

/* Backward through the token loop. For token t (reverse order), with
 * G = dL/dS_t accumulated so far and S_prev = S_{t-1} recomputed:
 *   readout   : G += q_t do_t^T ;           dq_t = S_t do_t
 *   write     : S_t = P + k u^T  ->  dP = G ; dk_t += G u ; du = G^T k
 *   x - r     : dx = du ; dr = -du
 *   gates     : dw_t = dx * v_t ; dv_t = dx * w_t
 *   read      : r = P^T c  ->  dP += c dr^T ; dc = P dr
 *   address   : db_t = dc * k_t ; dk_t += dc * b_t
 *   decay     : P = diag(alpha) S_prev -> dS_prev = diag(alpha) dP ;
 *               dalpha_i = sum_j dP_ij S_prev_ij ; dg_t = dalpha * alpha
 *   G <- dS_prev
 */
void gdr2_oracle_bwd(int B, int T, int H, int DK, int DV,
                     const double* q, const double* k, const double* v,
                     const double* g, const double* b, const double* w,
                     const double* h0, const double* dout, const double* dht,
                     double* dq, double* dk, double* dv, double* dg,
                     double* db, double* dw, double* dh0) {
    int nseq = B * H;
    int nck = (T + ORACLE_CKPT - 1) / ORACLE_CKPT;
#pragma omp parallel for schedule(dynamic, 1)
    for (int s = 0; s < nseq; ++s) {
        int bb = s / H, h = s % H;
        size_t SS = (size_t)DK * DV;
        double* ck = (double*)malloc(sizeof(double) * SS * (nck > 0 ? nck : 1));
        double* seg = (double*)malloc(sizeof(double) * SS * (ORACLE_CKPT + 1));
        double* G = (double*)malloc(sizeof(double) * SS);
        double* P = (double*)malloc(sizeof(double) * SS);
        double* r = (double*)malloc(sizeof(double) * DV);
        double* u = (double*)malloc(sizeof(double) * DV);
        double* du = (double*)malloc(sizeof(double) * DV);
        double* dc = (double*)malloc(sizeof(double) * DK);
        double* alpha = (double*)malloc(sizeof(double) * DK);
        double* S = (double*)malloc(sizeof(double) * SS);

        /* forward pass storing checkpoints S_{c*CKPT} */
        if (h0)
            memcpy(S, h0 + (size_t)s * SS, sizeof(double) * SS);
        else
            memset(S, 0, sizeof(double) * SS);
        for (int t = 0; t < T; ++t) {
            if (t % ORACLE_CKPT == 0) memcpy(ck + (size_t)(t / ORACLE_CKPT) * SS, S, sizeof(double) * SS);
            token_step(DK, DV, q + idx_tok(bb, t, h, 0, T, H, DK), k + idx_tok(bb, t, h, 0, T, H, DK),
                       v + idx_tok(bb, t, h, 0, T, H, DV), g + idx_tok(bb, t, h, 0, T, H, DK),
                       b + idx_tok(bb, t, h, 0, T, H, DK), w + idx_tok(bb, t, h, 0, T, H, DV), S, r, u);
        }
        if (dht)
            memcpy(G, dht + (size_t)s * SS, sizeof(double) * SS);
        else
            memset(G, 0, sizeof(double) * SS);

        for (int c = nck - 1; c >= 0; --c) {
            int t0 = c * ORACLE_CKPT;
            int t1 = t0 + ORACLE_CKPT < T ? t0 + ORACLE_CKPT : T;
            /* recompute the states of this segment: seg[j] = S_{t0+j} */
            memcpy(seg, ck + (size_t)c * SS, sizeof(double) * SS);
            for (int t = t0; t < t1; ++t) {
                memcpy(seg + (size_t)(t - t0 + 1) * SS, seg + (size_t)(t - t0) * SS, sizeof(double) * SS);
                token_step(DK, DV, q + idx_tok(bb, t, h, 0, T, H, DK), k + idx_tok(bb, t, h, 0, T, H, DK),
                           v + idx_tok(bb, t, h, 0, T, H, DV), g + idx_tok(bb, t, h, 0, T, H, DK),
                           b + idx_tok(bb, t, h, 0, T, H, DK), w + idx_tok(bb, t, h, 0, T, H, DV),
                           seg + (size_t)(t - t0 + 1) * SS, r, u);
            }
            for (int t = t1 - 1; t >= t0; --t) {
                const double* Sprev = seg + (size_t)(t - t0) * SS;
                const double* Scur = seg + (size_t)(t - t0 + 1) * SS;
                const double* qt = q + idx_tok(bb, t, h, 0, T, H, DK);
                const double* kt = k + idx_tok(bb, t, h, 0, T, H, DK);
                const double* gt = g + idx_tok(bb, t, h, 0, T, H, DK);
                const double* bt = b + idx_tok(bb, t, h, 0, T, H, DK);
                const double* vt = v + idx_tok(bb, t, h, 0, T, H, DV);
                const double* wt = w + idx_tok(bb, t, h, 0, T, H, DV);
                const double* dot = dout + idx_tok(bb, t, h, 0, T, H, DV);
                double* dqt = dq + idx_tok(bb, t, h, 0, T, H, DK);
                double* dkt = dk + idx_tok(bb, t, h, 0, T, H, DK);
                double* dgt = dg + idx_tok(bb, t, h, 0, T, H, DK);
                double* dbt = db + idx_tok(bb, t, h, 0, T, H, DK);
                double* dvt = dv + idx_tok(bb, t, h, 0, T, H, DV);
                double* dwt = dw + idx_tok(bb, t, h, 0, T, H, DV);

                /* readout o_t = S_t^T q_t */
                for (int i = 0; i < DK; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < DV; ++j) {
                        acc += Scur[i * DV + j] * dot[j];
                        G[i * DV + j] += qt[i] * dot[j];
                    }
                    dqt[i] = acc;
                }
                /* recompute the step's intermediates from S_{t-1} */
                for (int i = 0; i < DK; ++i) alpha[i] = exp(gt[i]);
                for (int i = 0; i < DK; ++i)
                    for (int j = 0; j < DV; ++j) P[i * DV + j] = alpha[i] * Sprev[i * DV + j];
                for (int j = 0; j < DV; ++j) r[j] = 0.0;
                for (int i = 0; i < DK; ++i) {
                    double ci = bt[i] * kt[i];
                    for (int j = 0; j < DV; ++j) r[j] += P[i * DV + j] * ci;
                }
                for (int j = 0; j < DV; ++j) u[j] = wt[j] * vt[j] - r[j];

                /* write: S_t = P + k u^T */
                for (int j = 0; j < DV; ++j) du[j] = 0.0;
                for (int i = 0; i < DK; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < DV; ++j) {
                        acc += G[i * DV + j] * u[j];
                        du[j] += G[i * DV + j] * kt[i];
                    }
                    dkt[i] = acc;
                }
                /* gates of the write value; dr = -du */
                for (int j = 0; j < DV; ++j) {
                    dwt[j] = du[j] * vt[j];
                    dvt[j] = du[j] * wt[j];
                }
                /* read r = P^T c: dP += c dr^T, dc = P dr (dr = -du) */
                for (int i = 0; i < DK; ++i) {
                    double ci = bt[i] * kt[i];
                    double acc = 0.0;
                    for (int j = 0; j < DV; ++j) {
                        acc -= P[i * DV + j] * du[j];
                        G[i * DV + j] -= ci * du[j];
                    }
                    dc[i] = acc;
                }
                for (int i = 0; i < DK; ++i) {
                    dbt[i] = dc[i] * kt[i];
                    dkt[i] += dc[i] * bt[i];
                }
                /* decay P = diag(alpha) S_{t-1} */
                for (int i = 0; i < DK; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < DV; ++j) {
                        acc += G[i * DV + j] * Sprev[i * DV + j];
                        G[i * DV + j] *= alpha[i];
                    }
                    dgt[i] = acc * alpha[i];
                }
            }
        }
        if (dh0) memcpy(dh0 + (size_t)s * SS, G, sizeof(double) * SS);
        free(ck); free(seg); free(G); free(P); free(r); free(u); free(du);
        free(dc); free(alpha); free(S);
    }
}

int gdr2_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
