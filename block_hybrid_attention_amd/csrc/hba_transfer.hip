// hba_transfer.hip -- stage-1 attention transfer: loss and gradients.
//
// "Retrofitting Linear Attention into Diffusion Language Models", section 3.2
// (attention transfer) trains only the hybrid layer's own parameters W and
// alpha against the frozen softmax teacher's output; the layer is the one of
// section 3.1, run over a whole training sequence: the queries of block n see
// exact softmax over block n plus the linear-attention states of blocks
// 0..n-1 through the shared normaliser.  For a sequence of n_blocks blocks
// per (request, head), these kernels compute
//   L = sum (o - target)^2,  dL/dW [H][d][F],  dL/dalpha [H].
//
// With g_i = 2 (o_i - t_i) and den_i the true shared denominator:
//   dnum_i = g_i / den_i,  dden_i = -(g_i . o_i) / den_i,
//   dL/dw  = sum_i dnum_i . sm_num_i + dden_i sm_den_i,  dL/dalpha = w (1-w) dL/dw,
//   dphi(q_i) = S_{n-1} dnum_i + Z_{n-1} dden_i,
//   dphi(k_t) = G_m v_t + Gz_m  (t in block m; G_m, Gz_m sum phi(q_i) dnum_i^T
//               and phi(q_i) dden_i over the queries of the blocks after m),
//   du = p (dp - p.dp) - p' (dp' - p'.dp')  for phi = [p, p'] = [softmax(u), softmax(-u)],
//   dW += x du^T for every query row and key row x.
//
// This file holds the fp32-input path and the launcher; bf16 inputs run the
// kernels of hba_transfer_bf16.hip (same sweeps, phi computed inside them,
// bf16 MFMA with split operands).  The fp32 path makes six launches:
//   0. the feature map (hba_feature_map's kernels) of every query and key
//      row into the workspace, fully parallel over rows.  The three sweeps
//      below stage phi from there instead of computing it per block.
// then one workgroup of eight waves per (request, head) for the three sweeps
// over the blocks:
//   1. forward sweep: output, loss, dnum and dden (stored to the workspace)
//      and dL/dw.  S (2F x d) lives in registers split by value column,
//      the layout in which phi(q) S contracts over features.
//   2. query sweep, forward: dphi(q) = dnum S^T + dden Z, through the feature
//      map into dW.  Here S^T lives in registers split by feature, the
//      layout in which the contraction over value columns runs.
//   3. key sweep, backward over the blocks: dphi(k) = v G^T + Gz, G updated
//      after each block with phi(q)^T dnum; into dW.
//   4. reduction of the per-(request, head) parts over requests, in request
//      order (deterministic; shared by both paths).
// Every product of these sweeps runs on fp32 MFMA (v_mfma_f32_16x16x4f32).
// Token tiles that MFMA reads with the token index on the 16-lane axis are
// staged transposed in LDS ([column][32 tokens + 4]); that stride puts the
// 64 lanes of an operand read on 64 different banks.
#include "hba_device.h"
#include "hba_internal.h"
#include "hba_transfer.h"

namespace hba {

template <int F>
struct XferGeom {
    static constexpr int D = kXferD, P2 = 2 * F;
    static constexpr int XLD = D + 4;   // row-major token tiles [32][XLD]
    static constexpr int TLD = 36;      // transposed tiles [columns][TLD]
    static constexpr int x_f = kRows * XLD;
    static constexpr int vT_f = D * TLD;
    static constexpr int ph_f = P2 * TLD;
    static constexpr int pm_f = kRows * TLD;
    static constexpr int red_f = 8 * kRows;           // [wave][row] partial sums
    // forward sweep
    static constexpr int f_xq = 0, f_xk = f_xq + x_f, f_vT = f_xk + x_f, f_phq = f_vT + vT_f,
                         f_phk = f_phq + ph_f, f_pm = f_phk + ph_f, f_z = f_pm + pm_f, f_red = f_z + P2,
                         f_row = f_red + red_f, f_sc = f_row + 8 * kRows * 2, f_total = f_sc + kRows * 8;
    // gradient sweeps
    // a gradient sweep stages only the side whose gradient it takes, so the
    // q and k tiles share one region
    static constexpr int s_xq = 0, s_xk = 0, s_vT = x_f, s_dnT = s_vT + vT_f,
                         s_phq = s_dnT + vT_f, s_phk = s_phq + ph_f, s_z = s_phk + ph_f, s_dd = s_z + P2,
                         s_red = s_dd + kRows, s_total = s_red + red_f;
};

int64_t transfer_workspace_floats(int64_t BH, int64_t N, int F) { return xfer_ws(BH, N, F).total; }

// Eight consecutive elements of one of the 32 rows of a token tile
// (512 threads: row = tid / 16, columns 8 (tid % 16) ..), zero past nrows.
__device__ __forceinline__ void load8(const float *__restrict__ rows, int nrows, int tid, float (&x)[8]) {
    const int row = tid >> 4, c0 = (tid & 15) * 8;
    if (row < nrows) {
        const float *p = rows + (int64_t)row * kXferD + c0;
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
}

template <int XLD>
__device__ __forceinline__ void stage_rows_f32(const float *__restrict__ rows, int nrows, float *dst, int tid) {
    float x[8];
    load8(rows, nrows, tid, x);
    float *p = dst + (tid >> 4) * XLD + (tid & 15) * 8;
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

template <int TLD>
__device__ __forceinline__ void stage_cols_f32(const float *__restrict__ rows, int nrows, float *dstT, int tid) {
    float x[8];
    load8(rows, nrows, tid, x);
    const int row = tid >> 4, c0 = (tid & 15) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) dstT[(c0 + e) * TLD + row] = x[e];
}

// 32 fp32 rows of COLS columns (row stride COLS) into the transposed tile
// dstT[COLS][TLD]; rows >= nrows become zero.
template <int COLS, int TLD>
__device__ __forceinline__ void stage_colsT_f32(const float *__restrict__ rows, int nrows, float *dstT, int tid) {
    constexpr int TPR = COLS / 8;                  // threads per row, eight columns each
    constexpr int RPP = kXferThreads / TPR;        // rows per pass
#pragma unroll
    for (int p = 0; p < kRows / RPP; ++p) {
        const int row = p * RPP + tid / TPR, c0 = (tid % TPR) * 8;
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
        if (row < nrows) {
            a = *reinterpret_cast<const float4 *>(rows + (int64_t)row * COLS + c0);
            b = *reinterpret_cast<const float4 *>(rows + (int64_t)row * COLS + c0 + 4);
        }
        const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) dstT[(c0 + e) * TLD + row] = x[e];
    }
}

// 1. Forward sweep.
template <int F>
__global__ __launch_bounds__(kXferThreads, 1) void transfer_forward_kernel(TransferArgs a) {
    using G = XferGeom<F>;
    constexpr int D = kXferD, P2 = 2 * F, NFT = P2 / 16, TLD = G::TLD;
    __shared__ __attribute__((aligned(16))) float sm[G::f_total];
    float *xq = sm + G::f_xq, *xk = sm + G::f_xk, *vT = sm + G::f_vT, *phqT = sm + G::f_phq,
          *phkT = sm + G::f_phk, *pm = sm + G::f_pm, *Zs = sm + G::f_z, *red = sm + G::f_red,
          *rowp = sm + G::f_row, *rsc = sm + G::f_sc;

    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % a.H);
    const int L = a.L;
    const int64_t N = (int64_t)a.nb * L;
    const float *qg = static_cast<const float *>(a.q) + bh * N * D;
    const float *kg = static_cast<const float *>(a.k) + (bh / a.G) * N * D;
    const float *vg = static_cast<const float *>(a.v) + (bh / a.G) * N * D;
    const float *tg = a.target + bh * N * D;
    const float w = 1.f / (1.f + __expf(-a.alpha[h]));
    const float log2w = __log2f(w);
    constexpr float kScaleLog2 = 0.08838834764831845f * 1.4426950408889634f;   // log2(e) / sqrt(128)
    const XferWs ws = xfer_ws((int64_t)a.B * a.H, N, F);

    const float *pqg = a.ws + ws.phq + bh * N * P2;
    const float *pkg = a.ws + ws.phk + bh * N * P2;
    floatx4 S[NFT];   // S[16 ft + 4 lg + r][16 wave + li]
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) S[ft] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (tid < P2) Zs[tid] = 0.f;
    const int c0 = 16 * wave;
    float loss = 0.f, dw = 0.f;

#pragma unroll 1
    for (int n = 0; n < a.nb; ++n) {
        const int64_t t0 = (int64_t)n * L;
        stage_rows_f32<G::XLD>(qg + t0 * D, L, xq, tid);
        stage_rows_f32<G::XLD>(kg + t0 * D, L, xk, tid);
        stage_cols_f32<TLD>(vg + t0 * D, L, vT, tid);
        stage_colsT_f32<P2, TLD>(pqg + t0 * P2, L, phqT, tid);
        stage_colsT_f32<P2, TLD>(pkg + t0 * P2, L, phkT, tid);
        // this lane's teacher outputs (rows 16 rt + 4 lg + r, column c0 + li),
        // requested with the staging so their latency is not exposed later
        float tv[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rt + 4 * lg + r;
                tv[rt][r] = row < L ? tg[(t0 + row) * D + c0 + li] : 0.f;
            }
        __syncthreads();
        if (wave < 4) {
            // scores of query tile it against key tile jt, in log2 units; keys >= L masked
            const int it = wave >> 1, jt = wave & 1;
            floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 4; ++ks) {
                s = mfma_f32(xq[(16 * it + li) * G::XLD + 4 * ks + lg], xk[(16 * jt + li) * G::XLD + 4 * ks + lg], s);
                if ((ks & 7) == 7) fence();
            }
            const bool key_ok = 16 * jt + li < L;
#pragma unroll
            for (int r = 0; r < 4; ++r) pm[(16 * it + 4 * lg + r) * TLD + 16 * jt + li] = key_ok ? s[r] * kScaleLog2 : -INFINITY;
        } else {
            // lin_den = phi(q) . Z for the 32 rows: eight lanes per row
            const int t = tid - 256, row = t >> 3, part = t & 7;
            float acc = 0.f;
            for (int f = part * (P2 / 8); f < (part + 1) * (P2 / 8); ++f) acc += phqT[f * TLD + row] * Zs[f];
            acc += __shfl_xor(acc, 1, kWave);
            acc += __shfl_xor(acc, 2, kWave);
            acc += __shfl_xor(acc, 4, kWave);
            if (part == 0) rsc[row * 8 + 0] = acc;
        }
        __syncthreads();
        {
            // per row: block max M, probabilities 2^(s - M), their sum, and the
            // shared shift c = max(M + log2 w, log2 lin_den) (log2 units)
            const int row = tid >> 4, j = (tid & 15) * 2;
            const float x0 = pm[row * TLD + j], x1 = pm[row * TLD + j + 1];
            const float M = row16_max(fmaxf(x0, x1));   // finite: key 0 is always valid
            const float p0 = fast_exp2(x0 - M), p1 = fast_exp2(x1 - M);
            const float smd = row16_sum(p0 + p1);
            pm[row * TLD + j] = p0;
            pm[row * TLD + j + 1] = p1;
            if ((tid & 15) == 0) {
                const float lden = rsc[row * 8 + 0];
                const float c2 = fmaxf(M + log2w, __log2f(lden));
                const float esm = fast_exp2(M + log2w - c2), elin = fast_exp2(-c2);
                const float den = esm * smd + elin * lden;
                rsc[row * 8 + 1] = esm;
                rsc[row * 8 + 2] = elin;
                rsc[row * 8 + 3] = den;
                rsc[row * 8 + 4] = smd;
            }
        }
        __syncthreads();
        // block softmax numerator and linear readout for this wave's 16 columns
        floatx4 smv[2], lin[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < kRows / 4; ++ks)
                acc = mfma_f32(pm[(16 * rt + li) * TLD + 4 * ks + lg], vT[(c0 + li) * TLD + 4 * ks + lg], acc);
            smv[rt] = acc;
            floatx4 acl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) {
#pragma unroll
                for (int r = 0; r < 4; ++r) acl = mfma_f32(phqT[(16 * ft + 4 * lg + r) * TLD + 16 * rt + li], S[ft][r], acl);
                if ((ft & 1) == 1) fence();
            }
            lin[rt] = acl;
        }
        // output, loss, and the row sums g.o and g.smv
        floatx4 o[2], gg[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rt + 4 * lg + r;
                const float esm = rsc[row * 8 + 1], elin = rsc[row * 8 + 2], den = rsc[row * 8 + 3];
                const float ov = (esm * smv[rt][r] + elin * lin[rt][r]) / den;
                o[rt][r] = ov;
                float g = 0.f;
                if (row < L) {
                    const float e = ov - tv[rt][r];
                    loss += e * e;
                    g = 2.f * e;
                    if (a.out) a.out[(bh * N + t0 + row) * D + c0 + li] = ov;
                }
                gg[rt][r] = g;
                const float go = row16_sum(g * ov), gs = row16_sum(g * smv[rt][r]);
                if (li == 0) {
                    rowp[(wave * kRows + row) * 2 + 0] = go;
                    rowp[(wave * kRows + row) * 2 + 1] = gs;
                }
            }
        // Z of blocks 0..n-1 is no longer read in this block: fold block n in
        __syncthreads();
        if (tid < P2) {
            float z = Zs[tid];
#pragma unroll 8
            for (int t = 0; t < kRows; ++t) z += phkT[tid * TLD + t];
            Zs[tid] = z;
        } else if (tid >= 256 && tid < 256 + kRows) {
            // per row: g.o and g.smv over the eight waves' columns, 1/den,
            // dden and the row's share of dL/dw
            const int row = tid - 256;
            float go = 0.f, gs = 0.f;
#pragma unroll
            for (int ww = 0; ww < 8; ++ww) {
                go += rowp[(ww * kRows + row) * 2 + 0];
                gs += rowp[(ww * kRows + row) * 2 + 1];
            }
            const float esm = rsc[row * 8 + 1], elin = rsc[row * 8 + 2], den = rsc[row * 8 + 3];
            const float rho = elin / den;   // 1 / (true denominator)
            rsc[row * 8 + 5] = rho;
            if (row < L) {
                a.ws[ws.dden + bh * ((N + 3) & ~int64_t(3)) + t0 + row] = -go * rho;
                dw += (esm / w) / den * (gs - go * rsc[row * 8 + 4]);
            }
        }
        __syncthreads();
        // dnum = g / den
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rt + 4 * lg + r;
                if (row < L) a.ws[ws.dnum + (bh * N + t0 + row) * D + c0 + li] = gg[rt][r] * rsc[row * 8 + 5];
            }
        // commit block n: S[f][c] += sum_t phi(k_t)[f] v_t[c] for this wave's columns
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
#pragma unroll
            for (int ks = 0; ks < kRows / 4; ++ks)
                S[ft] = mfma_f32(phkT[(16 * ft + li) * TLD + 4 * ks + lg], vT[(c0 + li) * TLD + 4 * ks + lg], S[ft]);
            fence();
        }
        __syncthreads();
    }
    // per-(request, head) loss and dL/dw (dw lives in the lanes of threads 256 .. 287)
    loss = wave_sum(loss);
    dw = wave_sum(dw);
    if (lane == 0) {
        red[wave] = loss;
        red[8 + wave] = dw;
    }
    __syncthreads();
    if (tid == 0) {
        float s = 0.f, sw = 0.f;
        for (int ww = 0; ww < 8; ++ww) {
            s += red[ww];
            sw += red[8 + ww];
        }
        a.ws[ws.scal + bh * 4 + 0] = s;
        a.ws[ws.scal + bh * 4 + 1] = sw;
    }
}

// 2./3. Gradient sweeps.  KEYS = false: queries, blocks in order,
//   dphi(q) = dnum S^T + dden Z, then S^T += V^T phi(K), Z += sum phi(k).
// KEYS = true: keys, blocks in reverse order,
//   dphi(k) = V G^T + Gz, then G^T += dnum^T phi(Q), Gz += sum dden phi(q).
// The state X^T [d][2F] lives in registers split by feature: wave w holds
// features fb .. fb + 2F/8 - 1 (fb = w 2F/8) for all d value columns.
template <int F, bool KEYS>
__global__ __launch_bounds__(kXferThreads, 1) void transfer_sweep_kernel(TransferArgs a) {
    using G = XferGeom<F>;
    constexpr int D = kXferD, P2 = 2 * F, TLD = G::TLD;
    constexpr int FS = P2 / 8, FT = FS / 16;          // features per wave, their 16-tiles
    constexpr int DWT = F == 128 ? 8 : 4;             // dW tiles per wave
    __shared__ __attribute__((aligned(16))) float sm[G::s_total];
    float *xq = sm + G::s_xq, *xk = sm + G::s_xk, *vT = sm + G::s_vT, *dnT = sm + G::s_dnT,
          *phqT = sm + G::s_phq, *phkT = sm + G::s_phk, *Zs = sm + G::s_z, *dd = sm + G::s_dd,
          *red = sm + G::s_red;

    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % a.H);
    const int L = a.L;
    const int64_t N = (int64_t)a.nb * L;
    const int64_t npad = (N + 3) & ~int64_t(3);
    const float *qg = static_cast<const float *>(a.q) + bh * N * D;
    const float *kg = static_cast<const float *>(a.k) + (bh / a.G) * N * D;
    const float *vg = static_cast<const float *>(a.v) + (bh / a.G) * N * D;
    const XferWs ws = xfer_ws((int64_t)a.B * a.H, N, F);
    const float *dng = a.ws + ws.dnum + bh * N * D;
    const float *ddg = a.ws + ws.dden + bh * npad;
    const float *pqg = a.ws + ws.phq + bh * N * P2;
    const float *pkg = a.ws + ws.phk + bh * N * P2;
    (void)h;
    const int fb = wave * FS;
    floatx4 X[D / 16][FT];   // X^T[16 ct + 4 lg + r][fb + 16 j + li]
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
        for (int j = 0; j < FT; ++j) X[ct][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    const int wft = F == 128 ? wave : (wave & 3);              // dW feature tile
    const int wd0 = F == 128 ? 0 : 4 * (wave >> 2);            // first dW row tile
    floatx4 dW[DWT];   // dW[16 (wd0 + m) + 4 lg + r][16 wft + li]
#pragma unroll
    for (int m = 0; m < DWT; ++m) dW[m] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (tid < P2) Zs[tid] = 0.f;

#pragma unroll 1
    for (int it_ = 0; it_ < a.nb; ++it_) {
        const int n = KEYS ? a.nb - 1 - it_ : it_;
        const int64_t t0 = (int64_t)n * L;
        // only the side whose gradient this sweep takes needs its rows
        if (KEYS)
            stage_rows_f32<G::XLD>(kg + t0 * D, L, xk, tid);
        else
            stage_rows_f32<G::XLD>(qg + t0 * D, L, xq, tid);
        stage_cols_f32<TLD>(vg + t0 * D, L, vT, tid);
        stage_cols_f32<TLD>(dng + t0 * D, L, dnT, tid);
        stage_colsT_f32<P2, TLD>(pqg + t0 * P2, L, phqT, tid);
        stage_colsT_f32<P2, TLD>(pkg + t0 * P2, L, phkT, tid);
        if (tid < kRows) dd[tid] = tid < L ? ddg[t0 + tid] : 0.f;
        __syncthreads();

        float *phx = KEYS ? phkT : phqT;        // the side whose gradient this sweep takes
        const float *phy = KEYS ? phqT : phkT;  // the side folded into the state
        const float *xs = KEYS ? xk : xq;
        const float *cT = KEYS ? vT : dnT;      // contracted with the state
        const float *uT = KEYS ? dnT : vT;      // folded into the state
        // dphi^T[f][i] for this wave's features f and all 32 rows i
        floatx4 dp[FT][2];
#pragma unroll
        for (int j = 0; j < FT; ++j)
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ct = 0; ct < D / 16; ++ct) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc = mfma_f32(X[ct][j][r], cT[(16 * ct + 4 * lg + r) * TLD + 16 * it + li], acc);
                    if ((ct & 1) == 1) fence();
                }
                dp[j][it] = acc;
            }
        // + Z[f] s_i with s_i = dden_i (queries) or 1 for valid keys
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int i = 16 * it + li;
            const float s = KEYS ? (i < L ? 1.f : 0.f) : dd[i];
#pragma unroll
            for (int j = 0; j < FT; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) dp[j][it][r] += Zs[fb + 16 * j + 4 * lg + r] * s;
        }
        // p . dp per row over this wave's features, then over the wave's half
        float part[2];
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < FT; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc += phx[(fb + 16 * j + 4 * lg + r) * TLD + 16 * it + li] * dp[j][it][r];
            acc = xrow_sum(acc);
            part[it] = acc;
        }
        if (lg == 0) {
            red[wave * kRows + li] = part[0];
            red[wave * kRows + 16 + li] = part[1];
        }
        __syncthreads();
        // du for this wave's features: +p (dp - p.dp) in the first half, -p'(dp' - p'.dp') in the second
        const int w0 = wave < 4 ? 0 : 4;
        const float sgn = wave < 4 ? 1.f : -1.f;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int i = 16 * it + li;
            const float tot = red[(w0 + 0) * kRows + i] + red[(w0 + 1) * kRows + i] + red[(w0 + 2) * kRows + i] +
                              red[(w0 + 3) * kRows + i];
#pragma unroll
            for (int j = 0; j < FT; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dp[j][it][r] = sgn * phx[(fb + 16 * j + 4 * lg + r) * TLD + i] * (dp[j][it][r] - tot);
        }
        // du = du+ - du- into phx rows 0..F-1 (the first half's own rows; the
        // second half adds after a barrier)
        if (wave < 4) {
#pragma unroll
            for (int it = 0; it < 2; ++it)
#pragma unroll
                for (int j = 0; j < FT; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) phx[(fb + 16 * j + 4 * lg + r) * TLD + 16 * it + li] = dp[j][it][r];
        }
        __syncthreads();
        if (wave >= 4) {
#pragma unroll
            for (int it = 0; it < 2; ++it)
#pragma unroll
                for (int j = 0; j < FT; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) phx[(fb - F + 16 * j + 4 * lg + r) * TLD + 16 * it + li] += dp[j][it][r];
        }
        __syncthreads();
        // dW[d][f] += sum_t x[t][d] du[t][f]
#pragma unroll
        for (int m = 0; m < DWT; ++m) {
#pragma unroll
            for (int ks = 0; ks < kRows / 4; ++ks)
                dW[m] = mfma_f32(xs[(4 * ks + lg) * G::XLD + 16 * (wd0 + m) + li], phx[(16 * wft + li) * TLD + 4 * ks + lg], dW[m]);
            fence();
        }
        // fold this block into the state: X^T[c][f] += sum_t u[t][c] phy[t][f]
#pragma unroll
        for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
            for (int j = 0; j < FT; ++j) {
#pragma unroll
                for (int ks = 0; ks < kRows / 4; ++ks)
                    X[ct][j] = mfma_f32(uT[(16 * ct + li) * TLD + 4 * ks + lg], phy[(fb + 16 * j + li) * TLD + 4 * ks + lg], X[ct][j]);
                fence();
            }
        if (tid < P2) {
            float z = Zs[tid];
#pragma unroll 8
            for (int t = 0; t < kRows; ++t) z += phy[tid * TLD + t] * (KEYS ? dd[t] : 1.f);
            Zs[tid] = z;
        }
        __syncthreads();
    }
    float *dWg = a.ws + (KEYS ? ws.dWk : ws.dWq) + bh * D * F;
#pragma unroll
    for (int m = 0; m < DWT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) dWg[(int64_t)(16 * (wd0 + m) + 4 * lg + r) * F + 16 * wft + li] = dW[m][r];
}

// 4. Sum the per-(request, head) parts over requests, in request order.
// Grid (H, d F / (4 kThreads)); workgroup (h, 0) also writes dL/dalpha[h],
// and workgroup (0, 0) the total loss.
template <int F>
__global__ __launch_bounds__(kThreads) void transfer_reduce_kernel(TransferArgs a) {
    constexpr int D = kXferD;
    const int h = (int)blockIdx.x, tid = (int)threadIdx.x;
    const int64_t N = (int64_t)a.nb * a.L;
    const XferWs ws = xfer_ws((int64_t)a.B * a.H, N, F);
    const int e = 4 * ((int)blockIdx.y * kThreads + tid);
    if (e < D * F) {
        floatx4 s = {0.f, 0.f, 0.f, 0.f};
        for (int b = 0; b < a.B; ++b) {
            const int64_t p = (int64_t)b * a.H + h;
            s += *reinterpret_cast<const floatx4 *>(a.ws + ws.dWq + p * D * F + e);
            s += *reinterpret_cast<const floatx4 *>(a.ws + ws.dWk + p * D * F + e);
        }
        *reinterpret_cast<floatx4 *>(a.dW + (int64_t)h * D * F + e) = s;
    }
    if (blockIdx.y == 0 && tid == 0) {
        const float w = 1.f / (1.f + __expf(-a.alpha[h]));
        float s = 0.f;
        for (int b = 0; b < a.B; ++b) s += a.ws[ws.scal + ((int64_t)b * a.H + h) * 4 + 1];
        a.dalpha[h] = s * w * (1.f - w);
    }
    if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
        float s = 0.f;
        for (int64_t p = 0; p < (int64_t)a.B * a.H; ++p) s += a.ws[ws.scal + p * 4 + 0];
        a.loss[0] = s;
    }
}

template <typename T, int F>
static hipError_t launch_transfer_t(const TransferArgs &a, hipStream_t stream) {
    const int64_t pairs = (int64_t)a.B * a.H;
    hipError_t e = hipSuccess;
    if (pairs > 0 && a.nb > 0) {
        if constexpr (sizeof(T) == 2) {
            // bf16 inputs: hba_transfer_bf16.hip, phi computed inside the sweeps
            e = launch_transfer_forward_bf16(a, F, stream);
            if (e == hipSuccess) e = launch_transfer_sweeps_bf16(a, F, stream);
        } else {
            // phi(q) and phi(k) of every token first, fully parallel, into the
            // workspace rows [B H][N][2F]; the three sweeps stage them from there
            const int64_t N = (int64_t)a.nb * a.L, D = kXferD, P2 = 2 * F;
            const XferWs ws = xfer_ws(pairs, N, F);
            const FeatureMapArgs fq{a.q, a.W, a.ws + ws.phq, N, a.H, D, N * D, (int64_t)a.H * N * D,
                                    P2, N * P2, (int64_t)a.H * N * P2, 1};
            const FeatureMapArgs fk{a.k, a.W, a.ws + ws.phk, N, a.H, D, N * D, (int64_t)(a.H / a.G) * N * D,
                                    P2, N * P2, (int64_t)a.H * N * P2, a.G};
            e = launch_feature_map(fq, false, (int)D, F, stream, a.B);
            if (e == hipSuccess) e = launch_feature_map(fk, false, (int)D, F, stream, a.B);
            const dim3 grid((unsigned)pairs), block(kXferThreads);
            if (e == hipSuccess) e = launch_kernel(transfer_forward_kernel<F>, grid, block, a, stream);
            if (e == hipSuccess) e = launch_kernel(transfer_sweep_kernel<F, false>, grid, block, a, stream);
            if (e == hipSuccess) e = launch_kernel(transfer_sweep_kernel<F, true>, grid, block, a, stream);
        }
    }
    if (e != hipSuccess) return e;
    TransferArgs r = a;
    if (a.nb == 0) r.B = 0;   // nothing was computed: the sums are empty
    const dim3 rgrid((unsigned)a.H, (unsigned)(kXferD * F / 4 / kThreads));
    return launch_kernel(transfer_reduce_kernel<F>, rgrid, dim3(kThreads), r, stream);
}

hipError_t launch_transfer(const TransferArgs &a, bool bf16, int F, hipStream_t stream) {
    if (F == 128) return bf16 ? launch_transfer_t<uint16_t, 128>(a, stream) : launch_transfer_t<float, 128>(a, stream);
    if (F == 64) return bf16 ? launch_transfer_t<uint16_t, 64>(a, stream) : launch_transfer_t<float, 64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace hba
