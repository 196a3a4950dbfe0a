/*
 * hba_oracle.c -- plain fp64 CPU statement of block-hybrid attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the tests, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the HIP library; the two
 * meet only in the seeded inputs the tests hand to both.
 *
 * Source of every formula: "Retrofitting Linear Attention into Diffusion
 * Language Models" (arXiv 2608.06628), section 2.2 (softmax attention, linear
 * attention Eq. 1 and its recurrent state) and section 3.1 (within-block
 * softmax numerator/normaliser, Hedgehog feature map, the states S and Z and
 * their per-block update, the linear readout, the gated shared-normaliser
 * merge).  Each function below names the passage it writes out.
 *
 * Everything is fp64.  Inputs that are bf16 or fp32 on the device arrive here
 * widened exactly to fp64 by the caller.  Loops run in the order the formulas
 * are written; the only parallelism is an OpenMP split over independent
 * (request, head) pairs, which does not change any element's arithmetic.
 *
 * Layouts (row-major, C order):
 *   x, q, out         [B][H][L][d]        one block of L tokens per request
 *   k, v              [B][Hkv][L][d]      key/value heads; query head h reads
 *                                         key/value head h / (H / Hkv)
 *   W                 [H][d][F]           u = x W  (W is d x F, per head)
 *   gate              [H] or NULL         w = sigma(alpha); NULL means w = 1
 *   S pool            [n_slots][H][2F][d] S = sum phi(k) v^T
 *   Z pool            [n_slots][H][2F]    Z = sum phi(k)
 *   slot              [B] or NULL         request -> pool slot; NULL means b
 *   Kc, Vc            [B][Hkv][P][d]      full prefix cache for the comparator
 *
 * Query heads own W, the gate and the states (section 3.1, and section 3.3
 * on serving, keep them per query head).  When Hkv < H, consecutive
 * groups of H / Hkv query heads share one key/value head; Hkv == H is the
 * plain multi-head case.
 *
 * Parity of each function is pinned by the CPU tests against closed forms,
 * a hand-worked example, library softmax/SDPA and brute-force Eq. 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Key/value row block of query head h of request b. */
static int64_t kv_index(int b, int h, int H, int Hkv) {
    return (int64_t)b * Hkv + h / (H / Hkv);
}

/* Largest |score| for which exp() of the unshifted score stays far from fp64
 * overflow (exp(709) is the limit).  The step and comparator below use the
 * unshifted definition, so they refuse inputs beyond it. */
#define ORC_MAX_ABS_SCORE 700.0

/* Hedgehog feature map for one row (section 3.1, feature-map definition):
 *   u = x W,  phi(x) = [softmax(u), softmax(-u)]  in R^{2F}.
 * softmax(u)_f = exp(u_f) / sum_g exp(u_g).  The exponent is shifted by
 * max(u) (resp. max(-u) = -min(u)); the shift cancels between numerator and
 * denominator, so this is the definition itself, safe for any finite u. */
static void phi_row(int d, int F, const double *x, const double *W,
                    double *u, double *phi) {
    for (int f = 0; f < F; ++f) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i) acc += x[i] * W[(int64_t)i * F + f];
        u[f] = acc;
    }
    double mx = u[0], mn = u[0];
    for (int f = 1; f < F; ++f) {
        if (u[f] > mx) mx = u[f];
        if (u[f] < mn) mn = u[f];
    }
    double sp = 0.0, sn = 0.0;
    for (int f = 0; f < F; ++f) {
        sp += exp(u[f] - mx);
        sn += exp(-u[f] + mn);
    }
    for (int f = 0; f < F; ++f) {
        phi[f] = exp(u[f] - mx) / sp;
        phi[F + f] = exp(-u[f] + mn) / sn;
    }
}

static int threads_or_default(int nthreads) {
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Number of threads an OpenMP region with this request would use. */
int orc_threads(int nthreads) { return threads_or_default(nthreads); }

/* phi for n rows of x [n][H][d] with per-head W [H][d][F] -> phi [n][H][2F]. */
int orc_feature_map(int64_t n, int H, int d, int F, const double *x,
                    const double *W, double *phi, int nthreads) {
    if (n < 0 || H <= 0 || d <= 0 || F <= 0) return 1;
    int nt = threads_or_default(nthreads);
    #pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t r = 0; r < n * H; ++r) {
        int h = (int)(r % H);
        double *u = (double *)malloc(sizeof(double) * F);
        phi_row(d, F, x + r * d, W + (int64_t)h * d * F, u, phi + r * 2 * F);
        free(u);
    }
    return 0;
}

/* State commit (section 3.1, per-block state update):
 *   S_n = S_{n-1} + sum_{t in block} phi(k_t) v_t^T,
 *   Z_n = Z_{n-1} + sum_{t in block} phi(k_t).
 * Written token by token.  Request b folds its first n_valid[b] tokens
 * (all T when n_valid is NULL) into pool slot slot[b] (b when NULL). */
int orc_commit(int B, int H, int Hkv, int T, int d, int F, const int32_t *n_valid,
               const double *k, const double *v, const double *W,
               double *S_pool, double *Z_pool, const int32_t *slot,
               int nthreads) {
    if (B < 0 || H <= 0 || Hkv <= 0 || H % Hkv || T < 0 || d <= 0 || F <= 0) return 1;
    const int P2 = 2 * F;
    int nt = threads_or_default(nthreads);
    int bad = 0;
    #pragma omp parallel for num_threads(nt) schedule(dynamic) reduction(|:bad)
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        int b = (int)(bh / H), h = (int)(bh % H);
        int nv = n_valid ? n_valid[b] : T;
        if (nv < 0 || nv > T) { bad |= 1; continue; }
        int64_t s = slot ? slot[b] : b;
        double *S = S_pool + (s * H + h) * (int64_t)P2 * d;
        double *Z = Z_pool + (s * H + h) * (int64_t)P2;
        const double *Wh = W + (int64_t)h * d * F;
        const int64_t kvh = kv_index(b, h, H, Hkv);
        double *u = (double *)malloc(sizeof(double) * F);
        double *p = (double *)malloc(sizeof(double) * P2);
        for (int t = 0; t < nv; ++t) {
            const double *kt = k + (kvh * T + t) * (int64_t)d;
            const double *vt = v + (kvh * T + t) * (int64_t)d;
            phi_row(d, F, kt, Wh, u, p);
            for (int f = 0; f < P2; ++f) {
                Z[f] += p[f];
                for (int n = 0; n < d; ++n) S[(int64_t)f * d + n] += p[f] * vt[n];
            }
        }
        free(u);
        free(p);
    }
    return bad ? 2 : 0;
}

/* One denoising step of block-hybrid attention (section 3.1):
 *   within-block branch  a_j = exp(q.k_j / sqrt(d)),
 *                        sm_num = sum_j a_j v_j,  sm_den = sum_j a_j
 *                        (every query sees all L block tokens, no mask);
 *   linear readout       lin_num = phi(q)^T S,  lin_den = phi(q)^T Z;
 *   gated merge          out = (w sm_num + lin_num) / (w sm_den + lin_den).
 * Scores are used unshifted, exactly as written; |score| above
 * ORC_MAX_ABS_SCORE is refused (return 3) instead of overflowing. */
int orc_step(int B, int H, int Hkv, int L, int d, int F, const double *q,
             const double *k, const double *v, const double *W,
             const double *gate, const double *S_pool, const double *Z_pool,
             const int32_t *slot, double *out, int nthreads) {
    if (B < 0 || H <= 0 || Hkv <= 0 || H % Hkv || L <= 0 || d <= 0 || F <= 0) return 1;
    const int P2 = 2 * F;
    const double scale = 1.0 / sqrt((double)d);
    int nt = threads_or_default(nthreads);
    int bad = 0;
    #pragma omp parallel for num_threads(nt) schedule(dynamic) reduction(|:bad)
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        int b = (int)(bh / H), h = (int)(bh % H);
        int64_t s = slot ? slot[b] : b;
        const double *S = S_pool + (s * H + h) * (int64_t)P2 * d;
        const double *Z = Z_pool + (s * H + h) * (int64_t)P2;
        const double *Wh = W + (int64_t)h * d * F;
        const double w = gate ? gate[h] : 1.0;
        const int64_t kvh = kv_index(b, h, H, Hkv);
        const double *qb = q + bh * (int64_t)L * d;
        const double *kb = k + kvh * (int64_t)L * d;
        const double *vb = v + kvh * (int64_t)L * d;
        double *ob = out + bh * (int64_t)L * d;
        double *u = (double *)malloc(sizeof(double) * F);
        double *p = (double *)malloc(sizeof(double) * P2);
        double *num = (double *)malloc(sizeof(double) * d);
        for (int i = 0; i < L; ++i) {
            const double *qi = qb + (int64_t)i * d;
            /* within-block softmax branch */
            double sm_den = 0.0;
            for (int n = 0; n < d; ++n) num[n] = 0.0;
            for (int j = 0; j < L; ++j) {
                double sc = 0.0;
                for (int n = 0; n < d; ++n) sc += qi[n] * kb[(int64_t)j * d + n];
                sc *= scale;
                if (!(fabs(sc) <= ORC_MAX_ABS_SCORE)) bad |= 4;
                double a = exp(sc);
                sm_den += a;
                for (int n = 0; n < d; ++n) num[n] += w * a * vb[(int64_t)j * d + n];
            }
            /* linear readout of the committed context */
            phi_row(d, F, qi, Wh, u, p);
            double lin_den = 0.0;
            for (int f = 0; f < P2; ++f) lin_den += p[f] * Z[f];
            for (int n = 0; n < d; ++n) {
                double lin = 0.0;
                for (int f = 0; f < P2; ++f) lin += p[f] * S[(int64_t)f * d + n];
                num[n] += lin;
            }
            /* shared normaliser */
            double den = w * sm_den + lin_den;
            for (int n = 0; n < d; ++n) ob[(int64_t)i * d + n] = num[n] / den;
        }
        free(u);
        free(p);
        free(num);
    }
    return bad ? 3 : 0;
}

/* Full softmax attention of the active block's queries over the prefix cache
 * and the block itself (section 2.2, softmax attention, with every prefix and
 * block key visible to the block's queries): the comparator the hybrid
 * layer replaces.  Request b uses the first prefix_len[b] cached tokens
 * (max_prefix when NULL). */
int orc_prefix_softmax(int B, int H, int Hkv, int L, int d, int max_prefix,
                       const int32_t *prefix_len, const double *q,
                       const double *k, const double *v, const double *Kc,
                       const double *Vc, double *out, int nthreads) {
    if (B < 0 || H <= 0 || Hkv <= 0 || H % Hkv || L <= 0 || d <= 0 || max_prefix < 0) return 1;
    const double scale = 1.0 / sqrt((double)d);
    int nt = threads_or_default(nthreads);
    int bad = 0;
    #pragma omp parallel for num_threads(nt) schedule(dynamic) reduction(|:bad)
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        int b = (int)(bh / H), h = (int)(bh % H);
        int P = prefix_len ? prefix_len[b] : max_prefix;
        if (P < 0 || P > max_prefix) { bad |= 2; continue; }
        const int64_t kvh = kv_index(b, h, H, Hkv);
        const double *qb = q + bh * (int64_t)L * d;
        const double *kb = k + kvh * (int64_t)L * d;
        const double *vb = v + kvh * (int64_t)L * d;
        const double *Kb = Kc + kvh * (int64_t)max_prefix * d;
        const double *Vb = Vc + kvh * (int64_t)max_prefix * d;
        double *ob = out + bh * (int64_t)L * d;
        double *num = (double *)malloc(sizeof(double) * d);
        for (int i = 0; i < L; ++i) {
            const double *qi = qb + (int64_t)i * d;
            double den = 0.0;
            for (int n = 0; n < d; ++n) num[n] = 0.0;
            for (int j = 0; j < P + L; ++j) {
                const double *kj = j < P ? Kb + (int64_t)j * d : kb + (int64_t)(j - P) * d;
                const double *vj = j < P ? Vb + (int64_t)j * d : vb + (int64_t)(j - P) * d;
                double sc = 0.0;
                for (int n = 0; n < d; ++n) sc += qi[n] * kj[n];
                sc *= scale;
                if (!(fabs(sc) <= ORC_MAX_ABS_SCORE)) bad |= 4;
                double a = exp(sc);
                den += a;
                for (int n = 0; n < d; ++n) num[n] += a * vj[n];
            }
            for (int n = 0; n < d; ++n) ob[(int64_t)i * d + n] = num[n] / den;
        }
        free(num);
    }
    return bad ? 3 : 0;
}

/* Stage-1 attention transfer (section 3.2): the layer's hybrid output over a
 * whole training sequence of N = n_blocks * L tokens, its squared error
 * against the softmax teacher's output, and the gradient of that error with
 * respect to the layer's own parameters W and alpha (the backbone, hence q,
 * k, v and the teacher, is frozen).
 *
 * Forward (section 3.1 over the sequence): the queries of block n use exact
 * softmax over block n, the states S_{n-1}, Z_{n-1} of blocks 0..n-1, and
 *   o_i = (w sm_num_i + phi(q_i)^T S_{n-1}) / (w sm_den_i + phi(q_i)^T Z_{n-1}),
 * w = sigma(alpha[h]).  Loss: L = sum over b, h, i, c of (o_ic - target_ic)^2,
 * the squared L2 norm of the section 3.2 objective for one layer and batch.
 *
 * Backward, by the chain rule, with g_i = dL/do_i = 2 (o_i - t_i):
 *   dL/dnum_i = g_i / den_i,   dL/dden_i = -(g_i . o_i) / den_i
 *   dL/dw     = sum_i dL/dnum_i . sm_num_i + dL/dden_i sm_den_i,
 *   dL/dalpha = dL/dw * w (1 - w)
 *   dL/dphi(q_i) = S_{n-1} dL/dnum_i + Z_{n-1} dL/dden_i
 *   dL/dphi(k_t) (t in block m) = G_m v_t + Gz_m, where G_m and Gz_m sum
 *       phi(q_i) dL/dnum_i^T and phi(q_i) dL/dden_i over the queries i of
 *       all blocks after m (those whose states contain k_t)
 *   phi = [p, p'] with p = softmax(u), p' = softmax(-u), u = x W:
 *   dL/du_f = p_f (dp_f - p . dp) - p'_f (dp'_f - p' . dp')
 *   dL/dW  += x dL/du^T for every query row x = q_i and key row x = k_t.
 * Layouts: q, target, out [B][H][N][d]; k, v [B][Hkv][N][d]; W, dW
 * [H][d][F]; alpha, dalpha [H]; out may be NULL.  dW, dalpha and loss are
 * overwritten.  The per-(request, head) parts are summed over requests in
 * request order. */
static void phi_backward(int F, const double *phi, const double *dphi, double *du) {
    double sp = 0.0, sn = 0.0;
    for (int f = 0; f < F; ++f) {
        sp += phi[f] * dphi[f];
        sn += phi[F + f] * dphi[F + f];
    }
    for (int f = 0; f < F; ++f)
        du[f] = phi[f] * (dphi[f] - sp) - phi[F + f] * (dphi[F + f] - sn);
}

int orc_transfer(int B, int H, int Hkv, int n_blocks, int L, int d, int F,
                 const double *q, const double *k, const double *v,
                 const double *W, const double *alpha, const double *target,
                 double *out, double *loss, double *dW, double *dalpha,
                 int nthreads) {
    if (B < 0 || H <= 0 || Hkv <= 0 || H % Hkv || n_blocks < 0 || L <= 0 || d <= 0 || F <= 0) return 1;
    const int P2 = 2 * F;
    const int64_t N = (int64_t)n_blocks * L;
    const double scale = 1.0 / sqrt((double)d);
    const int64_t nbh = (int64_t)B * H;
    /* per-(request, head) parts, summed in request order at the end */
    double *pW = (double *)calloc((size_t)(nbh > 0 ? nbh : 1) * d * F, sizeof(double));
    double *pw = (double *)calloc((size_t)(nbh > 0 ? nbh : 1), sizeof(double));
    double *pl = (double *)calloc((size_t)(nbh > 0 ? nbh : 1), sizeof(double));
    int nt = threads_or_default(nthreads);
    int bad = 0;
    #pragma omp parallel for num_threads(nt) schedule(dynamic) reduction(|:bad)
    for (int64_t bh = 0; bh < nbh; ++bh) {
        int b = (int)(bh / H), h = (int)(bh % H);
        const int64_t kvh = kv_index(b, h, H, Hkv);
        const double *Wh = W + (int64_t)h * d * F;
        const double w = 1.0 / (1.0 + exp(-alpha[h]));
        const double *qb = q + bh * N * d, *tb = target + bh * N * d;
        const double *kb = k + kvh * N * d, *vb = v + kvh * N * d;
        double *S = (double *)calloc((size_t)P2 * d, sizeof(double));
        double *Z = (double *)calloc((size_t)P2, sizeof(double));
        double *phq = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * P2);
        double *dnum = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * d);
        double *dden = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double *u = (double *)malloc(sizeof(double) * F);
        double *p = (double *)malloc(sizeof(double) * P2);
        double *dp = (double *)malloc(sizeof(double) * P2);
        double *du = (double *)malloc(sizeof(double) * F);
        double *smn = (double *)malloc(sizeof(double) * d);
        double *o = (double *)malloc(sizeof(double) * d);
        double *gW = pW + bh * d * F;
        for (int n = 0; n < n_blocks; ++n) {
            const int64_t i0 = (int64_t)n * L;
            for (int64_t i = i0; i < i0 + L; ++i) {
                const double *qi = qb + i * d;
                /* within-block softmax branch */
                double smd = 0.0;
                for (int c = 0; c < d; ++c) smn[c] = 0.0;
                for (int64_t j = i0; j < i0 + L; ++j) {
                    double sc = 0.0;
                    for (int c = 0; c < d; ++c) sc += qi[c] * kb[j * d + c];
                    sc *= scale;
                    if (!(fabs(sc) <= ORC_MAX_ABS_SCORE)) bad |= 4;
                    double a = exp(sc);
                    smd += a;
                    for (int c = 0; c < d; ++c) smn[c] += a * vb[j * d + c];
                }
                /* linear readout of blocks 0..n-1 and the shared normaliser */
                double *ph = phq + i * P2;
                phi_row(d, F, qi, Wh, u, ph);
                double den = w * smd;
                for (int f = 0; f < P2; ++f) den += ph[f] * Z[f];
                for (int c = 0; c < d; ++c) {
                    double lin = 0.0;
                    for (int f = 0; f < P2; ++f) lin += ph[f] * S[(int64_t)f * d + c];
                    o[c] = (w * smn[c] + lin) / den;
                }
                if (out)
                    for (int c = 0; c < d; ++c) out[(bh * N + i) * d + c] = o[c];
                /* loss and the gradient at the merge */
                double go = 0.0;
                for (int c = 0; c < d; ++c) {
                    const double e = o[c] - tb[i * d + c];
                    pl[bh] += e * e;
                    go += 2.0 * e * o[c];
                }
                dden[i] = -go / den;
                for (int c = 0; c < d; ++c) dnum[i * d + c] = 2.0 * (o[c] - tb[i * d + c]) / den;
                double gw = dden[i] * smd;
                for (int c = 0; c < d; ++c) gw += dnum[i * d + c] * smn[c];
                pw[bh] += gw;
                /* through phi(q_i) into W */
                for (int f = 0; f < P2; ++f) {
                    double acc = Z[f] * dden[i];
                    for (int c = 0; c < d; ++c) acc += S[(int64_t)f * d + c] * dnum[i * d + c];
                    dp[f] = acc;
                }
                phi_backward(F, ph, dp, du);
                for (int r = 0; r < d; ++r)
                    for (int f = 0; f < F; ++f) gW[(int64_t)r * F + f] += qi[r] * du[f];
            }
            /* commit block n */
            for (int64_t t = i0; t < i0 + L; ++t) {
                phi_row(d, F, kb + t * d, Wh, u, p);
                for (int f = 0; f < P2; ++f) {
                    Z[f] += p[f];
                    for (int c = 0; c < d; ++c) S[(int64_t)f * d + c] += p[f] * vb[t * d + c];
                }
            }
        }
        /* keys: G, Gz hold the blocks after m, so walk the blocks backwards */
        double *G = S, *Gz = Z;
        memset(G, 0, sizeof(double) * (size_t)P2 * d);
        memset(Gz, 0, sizeof(double) * (size_t)P2);
        for (int m = n_blocks - 1; m >= 0; --m) {
            const int64_t t0 = (int64_t)m * L;
            for (int64_t t = t0; t < t0 + L; ++t) {
                const double *kt = kb + t * d, *vt = vb + t * d;
                phi_row(d, F, kt, Wh, u, p);
                for (int f = 0; f < P2; ++f) {
                    double acc = Gz[f];
                    for (int c = 0; c < d; ++c) acc += G[(int64_t)f * d + c] * vt[c];
                    dp[f] = acc;
                }
                phi_backward(F, p, dp, du);
                for (int r = 0; r < d; ++r)
                    for (int f = 0; f < F; ++f) gW[(int64_t)r * F + f] += kt[r] * du[f];
            }
            for (int64_t i = t0; i < t0 + L; ++i) {
                const double *ph = phq + i * P2;
                for (int f = 0; f < P2; ++f) {
                    Gz[f] += ph[f] * dden[i];
                    for (int c = 0; c < d; ++c) G[(int64_t)f * d + c] += ph[f] * dnum[i * d + c];
                }
            }
        }
        pw[bh] *= w * (1.0 - w);
        free(S); free(Z); free(phq); free(dnum); free(dden);
        free(u); free(p); free(dp); free(du); free(smn); free(o);
    }
    double total = 0.0;
    memset(dW, 0, sizeof(double) * (size_t)H * d * F);
    memset(dalpha, 0, sizeof(double) * (size_t)H);
    for (int64_t bh = 0; bh < nbh; ++bh) {
        int h = (int)(bh % H);
        total += pl[bh];
        dalpha[h] += pw[bh];
        for (int64_t e = 0; e < (int64_t)d * F; ++e) dW[(int64_t)h * d * F + e] += pW[bh * d * F + e];
    }
    *loss = total;
    free(pW); free(pw); free(pl);
    return bad ? 3 : 0;
}
