// hba_step.hip -- one denoising step of block-hybrid attention.
//
// "Retrofitting Linear Attention into Diffusion Language Models", section 3.1:
// for each query q_i of the active block,
//   out_i = (w sum_j exp(q_i.k_j/sqrt d) v_j + phi(q_i)^T S)
//         / (w sum_j exp(q_i.k_j/sqrt d)     + phi(q_i)^T Z).
//
// One workgroup (4 waves) per (request, head).  The step is bound by HBM
// bandwidth: the fp32 state S (2F x d, 128 KB at F = d = 128) is read once and
// dominates the bytes.  Both kernels below:
//   * give every wave d/4 output columns and stream its column slice of S
//     through registers, with part of the stream requested at kernel entry,
//     so the state's latency overlaps the staging and the prologue;
//   * stage q, k and W in LDS (W transposed in registers on the way), then
//     form phi(q), phi(q).Z and the block softmax weights in the MFMA
//     accumulator layout, with exponentials in the base-2 domain;
//   * apply one exponent shift per query, c_i = max(m_i + ln w, ln lin_den_i),
//     to both branches, so w exp(s - c) <= 1 and e^{-c} lin_den <= 1;
//   * run both numerators as ONE contraction
//       [w e^{s_i - c_i} | e^{-c_i} phi(q_i)]  x  [V ; S]     (K = L + 2F)
//     whose A operand reuses the LDS of the staged q, k and W, and apply the
//     shared denominator at the store.
// step_kernel_f32 (fp32 inputs) streams S in 4-row K-steps, 24 in flight,
// spreads the prologue over all four waves (two per query row, swapping
// partial maxima and sums through LDS) and contracts on fp32 MFMA.
// step_kernel_bf16 (bf16 inputs, the serving path) streams S in 32-row
// chunks, two to four in flight; waves 0-1 form phi(q) and waves 2-3 the
// block scores; the contraction runs on bf16 MFMA with split operands (see
// the note above that kernel).
#include "hba_device.h"
#include "hba_internal.h"

namespace hba {

template <typename T, int D, int F>
struct StepGeom {
    using P = ProjGeom<T, D, F>;
    static constexpr int KROWS = kRows + 2 * F;   // rows of the merged contraction
    // q tile, k tile and W are dead once waves 0-1 hold u and the scores in
    // registers; the merged A operand [KROWS][32] fp32 then reuses their LDS
    static constexpr int q_off = 0;
    static constexpr int k_off = P::x_bytes;
    static constexpr int w_off = 2 * P::x_bytes;
    static constexpr int in_bytes = 2 * P::x_bytes + P::w_bytes;
    static constexpr int a_bytes = KROWS * 32 * 4;
    static constexpr int r1 = in_bytes > a_bytes ? in_bytes : a_bytes;
    static constexpr int den_off = r1;                // shared denominator per query
    static constexpr int z_off = den_off + kRows * 4;  // Z of this (request, head)
    static constexpr int NX = 4;                       // partial row statistics swapped per wave
    static constexpr int x_off = z_off + 2 * F * 4;    // [4 waves][NX][16 rows]
    static constexpr int bytes = x_off + 4 * NX * 16 * 4;
};

// Common exponent shift of both branches for one query (section 3.1 merge),
// in base 2: c = max(m + log2 w, log2 lin_den), floored at -120 so 2^{-c}
// stays finite.
__device__ __forceinline__ float exp2_shift(float m2, float lw2, float lin_den) {
    float c = m2 + lw2;
    if (lin_den > 0.f) c = fmaxf(c, __log2f(lin_den));
    return fmaxf(c, -120.f);
}

// Row k of the merged A operand holds the 32 queries interleaved as
// (i, i + 16) pairs, XOR-swizzled by k so that both the per-query column
// writes and the MFMA pair reads avoid LDS bank conflicts.
__device__ __forceinline__ int a_index(int k, int i) {
    return k * 32 + ((2 * (i & 15) + (i >> 4)) ^ (2 * (k & 15)));
}
__device__ __forceinline__ int a_pair(int k, int li) {
    return k * 32 + ((2 * li) ^ (2 * (k & 15)));
}

// EPL consecutive block values of one row held in the input type; get(e)
// widens element e to fp32 (exact).  Rows past the block read as zero.
template <typename T, int EPL>
struct VRow;
template <>
struct VRow<uint16_t, 2> {
    uint32_t w;
    __device__ __forceinline__ void load(const uint16_t *p, bool ok) {
        const uint32_t t = *reinterpret_cast<const uint32_t *>(p);
        w = ok ? t : 0u;
    }
    __device__ __forceinline__ float get(int e) const { return __uint_as_float(e ? (w & 0xffff0000u) : (w << 16)); }
};
template <>
struct VRow<uint16_t, 1> {
    uint32_t w;
    __device__ __forceinline__ void load(const uint16_t *p, bool ok) {
        const uint32_t t = *p;
        w = ok ? t : 0u;
    }
    __device__ __forceinline__ float get(int) const { return __uint_as_float(w << 16); }
};
template <int EPL>
struct VRow<float, EPL> {
    float f[EPL];
    __device__ __forceinline__ void load(const float *p, bool ok) {
        if constexpr (EPL == 2) {
            const float2 t = *reinterpret_cast<const float2 *>(p);
            f[0] = ok ? t.x : 0.f;
            f[1] = ok ? t.y : 0.f;
        } else {
            const float t = *p;
            f[0] = ok ? t : 0.f;
        }
    }
    __device__ __forceinline__ float get(int e) const { return f[e]; }
};

// One 16x16 tile of the block scores q k^T (unscaled), computed by one wave:
// s[r] = q[row0 + 4(l/16) + r] . k[16 nt + l%16].
template <typename T, int D>
__device__ __forceinline__ void project_scores16(const T *__restrict__ qs, const T *__restrict__ ks,
                                                 int row0, int nt, floatx4 &s) {
    constexpr bool kBf16 = sizeof(T) == 2;
    constexpr int XLD = kBf16 ? D + 8 : D + 4;
    const int lane = (int)threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    s = floatx4{0.f, 0.f, 0.f, 0.f};
    if constexpr (kBf16) {
#pragma unroll
        for (int ks_ = 0; ks_ < D / 32; ++ks_) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(qs + (row0 + li) * XLD + 32 * ks_ + 8 * lg);
            const bf16x8 b = *reinterpret_cast<const bf16x8 *>(ks + (16 * nt + li) * XLD + 32 * ks_ + 8 * lg);
            s = mfma_bf16(a, b, s);
        }
    } else {
#pragma unroll 4
        for (int ks_ = 0; ks_ < D / 4; ++ks_)
            s = mfma_f32(qs[(row0 + li) * XLD + 4 * ks_ + lg], ks[(16 * nt + li) * XLD + 4 * ks_ + lg], s);
    }
}

// fp32 inputs: every product on fp32 MFMA.
template <typename T, int D, int F>
__global__ __launch_bounds__(kThreads, 3) void step_kernel_f32(StepArgs a) {
    using G = StepGeom<T, D, F>;
    constexpr int EPL = D / 64;       // columns per lane per MFMA column group
    constexpr int NCOL = D / 4;       // output columns owned by one wave
    constexpr int KS = 2 * F / 4;     // 4-row K-steps over the state
    constexpr int RING = KS < 24 ? KS : 24;   // state K-steps kept in flight
    constexpr int NTH = F / 32;       // 16-feature tiles of u per wave (half of F)
    constexpr float kScale = D == 128 ? 0.08838834764831845f : 0.125f;   // 1/sqrt(d)

    __shared__ __attribute__((aligned(16))) char smem[G::bytes];
    T *qs = reinterpret_cast<T *>(smem + G::q_off);
    T *ks = reinterpret_cast<T *>(smem + G::k_off);
    T *ws = reinterpret_cast<T *>(smem + G::w_off);
    float *As = reinterpret_cast<float *>(smem);
    float *dens = reinterpret_cast<float *>(smem + G::den_off);
    float *zs = reinterpret_cast<float *>(smem + G::z_off);
    float *xs_ = reinterpret_cast<float *>(smem + G::x_off);

    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int bh = (int)blockIdx.x;
    const int b = bh / a.H, h = bh - b * a.H;
    const int L = a.L;
    const int64_t slot = a.slot ? (int64_t)a.slot[b] : (int64_t)b;

    const T *qg = static_cast<const T *>(a.q) + (int64_t)bh * L * D;
    const T *kg = static_cast<const T *>(a.k) + (int64_t)(bh / a.G) * L * D;
    const T *vg = static_cast<const T *>(a.v) + (int64_t)(bh / a.G) * L * D;
    const T *Wg = static_cast<const T *>(a.W) + (int64_t)h * D * F;
    const float *Sg = a.S + (slot * a.H + h) * (int64_t)(2 * F) * D;
    const float *Zg = a.Z + (slot * a.H + h) * (int64_t)(2 * F);

    // 1. small operands first: q, k rows and W (written to LDS below)
    RowChunks<T, D> qc, kc;
    load_rows<T, D>(qg, D, L, qc);
    load_rows<T, D>(kg, D, L, kc);
    WChunks<T, D, F> wc;
    load_w<T, D, F>(Wg, wc);
    constexpr int ZQ = 2 * F / 4;   // float4 chunks of Z
    float4 zq = make_float4(0.f, 0.f, 0.f, 0.f);
    if ((int)threadIdx.x < ZQ) zq = reinterpret_cast<const float4 *>(Zg)[threadIdx.x];

    // 2. open the state stream: the first RING 4-row steps of this wave's slice
    const int c0 = wave * NCOL + EPL * li;
    const float *s_lane = Sg + (int64_t)lg * D + c0;
    float sreg[KS][EPL];
    auto load_s = [&](int kk) {
        const float *p = s_lane + (int64_t)(4 * kk) * D;
        if constexpr (EPL == 2) {
            const floatx2 t = __builtin_nontemporal_load(reinterpret_cast<const floatx2 *>(p));
            sreg[kk][0] = t[0];
            sreg[kk][1] = t[1];
        } else {
            sreg[kk][0] = __builtin_nontemporal_load(p);
        }
    };
#pragma unroll
    for (int kk = 0; kk < RING; ++kk) load_s(kk);
    const float lw2 = a.gate ? __log2f(a.gate[h]) : 0.f;   // log2 w

    // 3. stage q, k, W
    store_rows<T, D, F>(qc, qs);
    store_rows<T, D, F>(kc, ks);
    store_w<T, D, F>(wc, ws);
    if ((int)threadIdx.x < ZQ) reinterpret_cast<float4 *>(zs)[threadIdx.x] = zq;
    __syncthreads();

    // 4. wave w: rows 16 mt .. +15 (mt = w/2), feature half fh = w%2 of u, and
    //    the block scores of those rows against all 32 keys
    const int mt = wave >> 1, fh = wave & 1;
    const int row0 = 16 * mt;
    floatx4 u[NTH], sc[2];
    project_rows16_part<T, D, F, NTH>(qs, ws, row0, NTH * fh, u);
    project_scores16<T, D>(qs, ks, row0, 0, sc[0]);
    project_scores16<T, D>(qs, ks, row0, 1, sc[1]);
    // base-2 logits; keys past the block are masked
    const bool kv0 = li < L, kv1 = (16 + li) < L;
    float pmx[4], pmn[4], m2[4], ssum[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float mx_ = -INFINITY, mn_ = INFINITY;
#pragma unroll
        for (int j = 0; j < NTH; ++j) {
            u[j][r] *= kLog2e;
            mx_ = fmaxf(mx_, u[j][r]);
            mn_ = fminf(mn_, u[j][r]);
        }
        pmx[r] = row16_max(mx_);
        pmn[r] = row16_min(mn_);
        sc[0][r] = kv0 ? sc[0][r] * (kScale * kLog2e) : -INFINITY;
        sc[1][r] = kv1 ? sc[1][r] * (kScale * kLog2e) : -INFINITY;
        m2[r] = row16_max(fmaxf(sc[0][r], sc[1][r]));
        sc[0][r] = kv0 ? fast_exp2(sc[0][r] - m2[r]) : 0.f;   // <= 1
        sc[1][r] = kv1 ? fast_exp2(sc[1][r] - m2[r]) : 0.f;
        ssum[r] = row16_sum(sc[0][r] + sc[1][r]);
    }
    float *xw = xs_ + wave * (G::NX * 16);           // this wave's partials
    const float *xp = xs_ + (wave ^ 1) * (G::NX * 16);  // the partner's
    if (li == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            xw[0 * 16 + 4 * lg + r] = pmx[r];
            xw[1 * 16 + 4 * lg + r] = pmn[r];
        }
    }
    __syncthreads();   // q, k, W are dead from here: their LDS becomes the A operand

    // 5. row maxima/minima complete; exponentials, partial sums and Z-dots
    float mx[4], mn[4], sp[4], sn[4], zd[4], ps[4];
    floatx4 en[NTH];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        mx[r] = fmaxf(pmx[r], xp[0 * 16 + 4 * lg + r]);
        mn[r] = fminf(pmn[r], xp[1 * 16 + 4 * lg + r]);
        float a_ = 0.f, b_ = 0.f, zp_ = 0.f, zn_ = 0.f;
#pragma unroll
        for (int j = 0; j < NTH; ++j) {
            const int f = 16 * (NTH * fh + j) + li;
            const float x = u[j][r];
            u[j][r] = fast_exp2(x - mx[r]);    // <= 1
            en[j][r] = fast_exp2(mn[r] - x);   // <= 1
            a_ += u[j][r];
            b_ += en[j][r];
            zp_ += u[j][r] * zs[f];
            zn_ += en[j][r] * zs[F + f];
        }
        sp[r] = row16_sum(a_);
        sn[r] = row16_sum(b_);
        // Z-dots of the two halves are kept apart: each is scaled by its own sum
        zd[r] = row16_sum(zp_);
        ps[r] = row16_sum(zn_);
    }
    __syncthreads();   // partner partials of step 4 consumed before overwrite
    if (li == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            xw[0 * 16 + 4 * lg + r] = sp[r];
            xw[1 * 16 + 4 * lg + r] = sn[r];
            xw[2 * 16 + 4 * lg + r] = zd[r];
            xw[3 * 16 + 4 * lg + r] = ps[r];
        }
    }
    __syncthreads();

    // 6. totals, the shared shift, and the merged A operand rows
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = row0 + 4 * lg + r;
        const float SP = sp[r] + xp[0 * 16 + 4 * lg + r];
        const float SN = sn[r] + xp[1 * 16 + 4 * lg + r];
        const float ZP = zd[r] + xp[2 * 16 + 4 * lg + r];
        const float ZN = ps[r] + xp[3 * 16 + 4 * lg + r];
        const float ip = 1.0f / SP, in_ = 1.0f / SN;
        const float ld = ZP * ip + ZN * in_;               // lin_den = phi(q).Z
        const float c = exp2_shift(m2[r], lw2, ld);
        const float elin = ld > 0.f ? fast_exp2(-c) : 0.f;
        const float fp = fast_exp2(m2[r] + lw2 - c);       // w 2^{m - c} <= 1
        As[a_index(16 * fh + li, i)] = sc[fh][r] * fp;   // each wave of the pair writes 16 keys
        if (fh == 0 && li == 0) dens[i] = ssum[r] * fp + elin * ld;
        const float ep = ip * elin, enn = in_ * elin;
#pragma unroll
        for (int j = 0; j < NTH; ++j) {
            const int f = 16 * (NTH * fh + j) + li;
            As[a_index(kRows + f, i)] = u[j][r] * ep;
            As[a_index(kRows + F + f, i)] = en[j][r] * enn;
        }
    }
    __syncthreads();

    // 7. merged contraction [w P | e^{-c} phi(q)] x [V ; S] on fp32 MFMA:
    //    the state rows first (the stream is already in flight), then the
    //    block values, requested now and kept in the input type until use
    VRow<T, EPL> vreg[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const int j = 4 * kk + lg;
        vreg[kk].load(vg + (int64_t)(j < L ? j : L - 1) * D + c0, j < L);
    }
    floatx4 acc[2][EPL];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[t][e] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        if (kk + RING < KS) load_s(kk + RING);   // keep the ring full
        const floatx2 av = *reinterpret_cast<const floatx2 *>(As + a_pair(kRows + 4 * kk + lg, li));
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            acc[0][e] = mfma_f32(av[0], sreg[kk][e], acc[0][e]);
            acc[1][e] = mfma_f32(av[1], sreg[kk][e], acc[1][e]);
        }
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const floatx2 av = *reinterpret_cast<const floatx2 *>(As + a_pair(4 * kk + lg, li));
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const float bv = vreg[kk].get(e);
            acc[0][e] = mfma_f32(av[0], bv, acc[0][e]);
            acc[1][e] = mfma_f32(av[1], bv, acc[1][e]);
        }
    }

    // 8. shared normaliser and store
    float *og = a.out + (int64_t)bh * L * D;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * t + 4 * lg + r;
            if (i < L) {
                const float inv = 1.0f / dens[i];
                float *o = og + (int64_t)i * D + c0;
                if constexpr (EPL == 2) {
                    *reinterpret_cast<float2 *>(o) = make_float2(acc[t][0][r] * inv, acc[t][1][r] * inv);
                } else {
                    o[0] = acc[t][0][r] * inv;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 inputs.  The contraction over the fp32 state runs on bf16 MFMA with
// both operands split into a bf16 high part and a bf16 residual,
//   A B ~= A_hi B_hi + A_hi B_lo + A_lo B_hi,
// which keeps about 16 mantissa bits of every product (the dropped A_lo B_lo
// term is ~2^-17 relative) at a fifth of the fp32 MFMA cycles.  phi(q) is
// formed in the transposed accumulator layout (a lane holds features of one
// query, so its row reductions are mostly in-register), and the two branches
// are merged at the store from per-query scalars, so the phi waves and the
// score waves share nothing before the contraction.
template <int D, int F>
struct StepGeomBf16 {
    using P = ProjGeom<uint16_t, D, F>;
    static constexpr int KA = kRows + 2 * F;   // K of the merged contraction
    static constexpr int KP = KA + 8;          // A row stride in bf16 (16-byte aligned rows)
    static constexpr int q_off = 0;
    static constexpr int k_off = P::x_bytes;
    static constexpr int w_off = 2 * P::x_bytes;
    static constexpr int in_bytes = 2 * P::x_bytes + P::w_bytes;
    static constexpr int a_bytes = 2 * kRows * KP * 2;   // A_hi then A_lo, [32][KP] bf16
    static constexpr int r1 = in_bytes > a_bytes ? in_bytes : a_bytes;
    static constexpr int alo_off = kRows * KP * 2;
    static constexpr int z_off = r1;                    // Z [2F] fp32
    static constexpr int row_off = z_off + 2 * F * 4;   // per query: lin_den, max, block sum
    static constexpr int bytes = row_off + 3 * kRows * 4;
};


template <int D, int F, int NSPLIT>
__global__ __launch_bounds__(kThreads, 3) void step_kernel_bf16(StepArgs a) {
    using T = uint16_t;
    using P = ProjGeom<T, D, F>;
    using G = StepGeomBf16<D, F>;
    // NSPLIT workgroups per (request, head), each owning D/NSPLIT output
    // columns (small batches: more workgroups than (request, head) pairs;
    // each recomputes the prologue, and none needs another's results)
    constexpr int EPL = D / (64 * NSPLIT);   // columns per lane per N-tile
    constexpr int NCOL = D / (4 * NSPLIT);   // output columns owned by one wave
    static_assert(EPL >= 1, "a wave needs at least one 16-column N-tile");
    constexpr int NCH = 2 * F / 32;   // 32-row chunks of the state
    constexpr int RING = NCH < 2 ? NCH : 2;   // chunks in flight
    constexpr int PRE = NCH < 4 ? NCH : 4;    // chunks requested before the contraction
    constexpr int NT = F / 16;        // 16-feature tiles of u^T
    constexpr float kS2 = (D == 128 ? 0.08838834764831845f : 0.125f) * kLog2e;   // log2(e)/sqrt(d)

    __shared__ __attribute__((aligned(16))) char smem[G::bytes];
    T *qs = reinterpret_cast<T *>(smem + G::q_off);
    T *ks = reinterpret_cast<T *>(smem + G::k_off);
    T *ws = reinterpret_cast<T *>(smem + G::w_off);
    T *Ahi = reinterpret_cast<T *>(smem);
    T *Alo = reinterpret_cast<T *>(smem + G::alo_off);
    float *zs = reinterpret_cast<float *>(smem + G::z_off);
    float *r_ld = reinterpret_cast<float *>(smem + G::row_off);
    float *r_m = r_ld + kRows;
    float *r_a = r_m + kRows;

    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int bh = (int)blockIdx.x / NSPLIT, part = (int)blockIdx.x - bh * NSPLIT;
    const int b = bh / a.H, h = bh - b * a.H;
    const int L = a.L;
    const int64_t slot = a.slot ? (int64_t)a.slot[b] : (int64_t)b;

    const T *qg = static_cast<const T *>(a.q) + (int64_t)bh * L * D;
    const T *kg = static_cast<const T *>(a.k) + (int64_t)(bh / a.G) * L * D;
    const T *vg = static_cast<const T *>(a.v) + (int64_t)(bh / a.G) * L * D;
    const T *Wg = static_cast<const T *>(a.W) + (int64_t)h * D * F;
    const float *Sg = a.S + (slot * a.H + h) * (int64_t)(2 * F) * D;
    const float *Zg = a.Z + (slot * a.H + h) * (int64_t)(2 * F);

    // 1. small operands first: q, k rows, W and Z (written to LDS below)
    RowChunks<T, D> qc, kc;
    load_rows<T, D>(qg, D, L, qc);
    load_rows<T, D>(kg, D, L, kc);
    WChunks<T, D, F> wc;
    load_w<T, D, F>(Wg, wc);
    constexpr int ZQ = 2 * F / 4;
    float4 zq = make_float4(0.f, 0.f, 0.f, 0.f);
    if ((int)threadIdx.x < ZQ) zq = reinterpret_cast<const float4 *>(Zg)[threadIdx.x];

    // 2. open the state stream: chunk c holds rows 32c + 8 lg + t (t < 8) of
    //    this wave's column slice, in the K order of the bf16 MFMA B operand
    const int c0 = part * (D / NSPLIT) + wave * NCOL + EPL * li;
    const float *s_lane = Sg + (int64_t)(8 * lg) * D + c0;
    float sreg[NCH][8][EPL];
    // Non-temporal loads when the state streams from HBM at full rate (one
    // workgroup per pair: 58.6-59.0 against 65.1-65.3 us at B = 128 with
    // plain loads); plain loads in the latency-bound two-way split (8.65-8.7
    // against 9.1 us at B = 8, 7.95 against 8.5 us at B = 4)
    auto load_chunk = [&](int c) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float *p = s_lane + (int64_t)(32 * c + t) * D;
            if constexpr (NSPLIT == 2) {
                sreg[c][t][0] = *p;
            } else if constexpr (EPL == 2) {
                const floatx2 v = __builtin_nontemporal_load(reinterpret_cast<const floatx2 *>(p));
                sreg[c][t][0] = v[0];
                sreg[c][t][1] = v[1];
            } else {
                sreg[c][t][0] = __builtin_nontemporal_load(p);
            }
        }
    };
#pragma unroll
    for (int c = 0; c < RING; ++c) load_chunk(c);
    const float lw2 = a.gate ? __log2f(a.gate[h]) : 0.f;   // log2 w

    // 3. stage q, k, W, Z
    store_rows<T, D, F>(qc, qs);
    store_rows<T, D, F>(kc, ks);
    store_w<T, D, F>(wc, ws);
    if ((int)threadIdx.x < ZQ) reinterpret_cast<float4 *>(zs)[threadIdx.x] = zq;
    __syncthreads();
    // more of the stream goes out while the prologue computes
#pragma unroll
    for (int c = RING; c < PRE; ++c) load_chunk(c);
    __builtin_amdgcn_sched_barrier(0);

    // 4. waves 0-1: u^T = W^T q^T for queries 16w .. 16w+15 (all F features):
    //    acc[m][r] = u[16w + l%16][16m + 4(l/16) + r].
    //    waves 2-3: block scores of queries 16(w-2) .. +15 against all keys.
    floatx4 acc[NT];
#pragma unroll
    for (int m = 0; m < NT; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (wave < 2) {
#pragma unroll
        for (int ks_ = 0; ks_ < D / 32; ++ks_) {
            const bf16x8 bq = *reinterpret_cast<const bf16x8 *>(qs + (16 * wave + li) * P::XLD + 32 * ks_ + 8 * lg);
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                const bf16x8 aw = *reinterpret_cast<const bf16x8 *>(ws + wt_off<D>(16 * m + li, 4 * ks_ + lg));
                acc[m] = mfma_bf16(aw, bq, acc[m]);
            }
        }
    } else {
        project_scores16<T, D>(qs, ks, 16 * (wave - 2), 0, acc[0]);
        project_scores16<T, D>(qs, ks, 16 * (wave - 2), 1, acc[1]);
    }
    __syncthreads();   // q, k, W are dead: their LDS becomes the A operand

    // 5. A operand rows (bf16 high parts and residuals) and per-query scalars
    if (wave < 2) {
        const int qi = 16 * wave + li;
        float mx = -INFINITY, mn = INFINITY;
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[m][r] *= kLog2e;
                mx = fmaxf(mx, acc[m][r]);
                mn = fminf(mn, acc[m][r]);
            }
        // the query's F features are spread over the four lane groups
        mx = xrow_max(mx);
        mn = xrow_min(mn);
        float sp = 0.f, sn = 0.f;
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sp += fast_exp2(acc[m][r] - mx);
                sn += fast_exp2(mn - acc[m][r]);
            }
        sp = xrow_sum(sp);
        sn = xrow_sum(sn);
        const float ip = 1.0f / sp, in_ = 1.0f / sn;
        float zd = 0.f;
        T *ah = Ahi + qi * G::KP + kRows + 4 * lg;
        T *al = Alo + qi * G::KP + kRows + 4 * lg;
#pragma unroll
        for (int m = 0; m < NT; ++m) {
            const float4 zp4 = *reinterpret_cast<const float4 *>(zs + 16 * m + 4 * lg);
            const float4 zn4 = *reinterpret_cast<const float4 *>(zs + F + 16 * m + 4 * lg);
            const float zp[4] = {zp4.x, zp4.y, zp4.z, zp4.w}, zn[4] = {zn4.x, zn4.y, zn4.z, zn4.w};
            float ep[4], en[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                ep[r] = fast_exp2(acc[m][r] - mx) * ip;   // softmax(u)_f
                en[r] = fast_exp2(mn - acc[m][r]) * in_;  // softmax(-u)_f
                zd += ep[r] * zp[r] + en[r] * zn[r];
            }
            uint32_t hp[2], lp[2], hn[2], ln[2];
            split_pk_bf16(ep[0], ep[1], hp[0], lp[0]);
            split_pk_bf16(ep[2], ep[3], hp[1], lp[1]);
            split_pk_bf16(en[0], en[1], hn[0], ln[0]);
            split_pk_bf16(en[2], en[3], hn[1], ln[1]);
            *reinterpret_cast<uint2 *>(ah + 16 * m) = make_uint2(hp[0], hp[1]);
            *reinterpret_cast<uint2 *>(al + 16 * m) = make_uint2(lp[0], lp[1]);
            *reinterpret_cast<uint2 *>(ah + F + 16 * m) = make_uint2(hn[0], hn[1]);
            *reinterpret_cast<uint2 *>(al + F + 16 * m) = make_uint2(ln[0], ln[1]);
        }
        zd = xrow_sum(zd);
        if (lg == 0) r_ld[qi] = zd;   // lin_den = phi(q).Z
    } else {
        const int row0 = 16 * (wave - 2);
        const bool kv0 = li < L, kv1 = (16 + li) < L;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = row0 + 4 * lg + r;
            const float s0 = kv0 ? acc[0][r] * kS2 : -INFINITY;
            const float s1 = kv1 ? acc[1][r] * kS2 : -INFINITY;
            const float m2 = row16_max(fmaxf(s0, s1));
            const float p0 = kv0 ? fast_exp2(s0 - m2) : 0.f;   // <= 1
            const float p1 = kv1 ? fast_exp2(s1 - m2) : 0.f;
            const float as = row16_sum(p0 + p1);
            Ahi[i * G::KP + li] = __builtin_bit_cast(uint16_t, (__bf16)p0);
            Ahi[i * G::KP + 16 + li] = __builtin_bit_cast(uint16_t, (__bf16)p1);
            Alo[i * G::KP + li] = __builtin_bit_cast(uint16_t, (__bf16)bf16_residual(p0));
            Alo[i * G::KP + 16 + li] = __builtin_bit_cast(uint16_t, (__bf16)bf16_residual(p1));
            if (li == 0) {
                r_m[i] = m2;
                r_a[i] = as;
            }
        }
    }
    __syncthreads();

    // 6. the contraction: state rows through the ring, then the block values
    floatx4 accS[2][EPL], accV[2][EPL];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < EPL; ++e) accS[t][e] = accV[t][e] = floatx4{0.f, 0.f, 0.f, 0.f};
    // block values for keys 8 lg + t, requested now (after the ring head)
    uint32_t vw[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int j = 8 * lg + t;
        const T *p = vg + (int64_t)(j < L ? j : L - 1) * D + c0;
        const uint32_t w_ = EPL == 2 ? *reinterpret_cast<const uint32_t *>(p) : (uint32_t)*p;
        vw[t] = w_;   // keys j >= L carry probability exactly 0
    }
    __builtin_amdgcn_sched_barrier(0);   // issue the block values before the stream is consumed
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        if (c + RING < NCH && c + RING >= PRE) load_chunk(c + RING);
        __builtin_amdgcn_sched_barrier(0);   // the refill stays ahead of the waits for chunk c
        bf16x8 bh_[EPL], bl_[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) split_pk_bf16(sreg[c][2 * j][e], sreg[c][2 * j + 1][e], hw[j], lw[j]);
            bh_[e] = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
            bl_[e] = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
        }
        const int k0 = kRows + 32 * c + 8 * lg;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(Ahi + (16 * mt + li) * G::KP + k0);
            const bf16x8 al = *reinterpret_cast<const bf16x8 *>(Alo + (16 * mt + li) * G::KP + k0);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                accS[mt][e] = mfma_bf16(ah, bh_[e], accS[mt][e]);
                accS[mt][e] = mfma_bf16(ah, bl_[e], accS[mt][e]);
                accS[mt][e] = mfma_bf16(al, bh_[e], accS[mt][e]);
            }
        }
    }
    {
        bf16x8 bv[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            uint32_t pk[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                pk[j] = __builtin_amdgcn_perm(vw[2 * j + 1], vw[2 * j], e ? 0x07060302u : 0x05040100u);
            bv[e] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(Ahi + (16 * mt + li) * G::KP + 8 * lg);
            const bf16x8 al = *reinterpret_cast<const bf16x8 *>(Alo + (16 * mt + li) * G::KP + 8 * lg);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                accV[mt][e] = mfma_bf16(ah, bv[e], accV[mt][e]);
                accV[mt][e] = mfma_bf16(al, bv[e], accV[mt][e]);
            }
        }
    }

    // 7. merge with one shift per query and store:
    //    out = (w 2^m2 V-part + phi.S) / (w 2^m2 a + lin_den), computed as
    //    (sv accV + ss accS) / (sv a + ss ld) with c = max(m2 + log2 w, log2 ld)
    float *og = a.out + (int64_t)bh * L * D;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * mt + 4 * lg + r;
            if (i < L) {
                const float ld = r_ld[i], g2 = r_m[i] + lw2, as = r_a[i];
                float c = g2;
                if (ld > 0.f) c = fmaxf(c, __log2f(ld));
                c = fmaxf(c, -120.f);
                const float sv = fast_exp2(g2 - c);
                const float ss = ld > 0.f ? fast_exp2(-c) : 0.f;
                const float inv = __builtin_amdgcn_rcpf(sv * as + ss * ld);
                float *o = og + (int64_t)i * D + c0;
                if constexpr (EPL == 2) {
                    __builtin_nontemporal_store(floatx2{(sv * accV[mt][0][r] + ss * accS[mt][0][r]) * inv,
                                                        (sv * accV[mt][1][r] + ss * accS[mt][1][r]) * inv},
                                                reinterpret_cast<floatx2 *>(o));
                } else {
                    __builtin_nontemporal_store((sv * accV[mt][0][r] + ss * accS[mt][0][r]) * inv, o);
                }
            }
        }
    }
}

template <typename T, int D, int F>
static hipError_t launch_step_t(const StepArgs &a, hipStream_t stream) {
    if constexpr (sizeof(T) == 2) {
        const int64_t items = (int64_t)a.B * a.H;
        if constexpr (D == 128) {
            // at most half a workgroup per CU: split the output columns over
            // two workgroups per pair.  Measured per launch from a HIP graph
            // at H = 16: 9.8 -> 9.05 us at B = 8 and 8.65 -> 7.4 us at B = 1;
            // between half and all of the CUs one workgroup per pair is
            // faster (10.1-11.1 against 11.9-13.0 us at B = 9..15)
            const int64_t cus = device_cus();
            if (cus > 0 && 2 * items <= cus)
                return launch_kernel(step_kernel_bf16<D, F, 2>, dim3((unsigned)(2 * items)), dim3(kThreads), a, stream);
        }
        return launch_kernel(step_kernel_bf16<D, F, 1>, dim3((unsigned)items), dim3(kThreads), a, stream);
    } else {
        return launch_kernel(step_kernel_f32<T, D, F>, dim3((unsigned)(a.B * a.H)), dim3(kThreads), a, stream);
    }
}

hipError_t launch_step(const StepArgs &a, bool bf16, int d, int F, hipStream_t stream) {
#define HBA_STEP_CASE(DD, FF)                                                              \
    if (d == DD && F == FF)                                                                \
        return bf16 ? launch_step_t<uint16_t, DD, FF>(a, stream)                           \
                    : launch_step_t<float, DD, FF>(a, stream);
    HBA_STEP_CASE(64, 64)
    HBA_STEP_CASE(64, 128)
    HBA_STEP_CASE(128, 64)
    HBA_STEP_CASE(128, 128)
#undef HBA_STEP_CASE
    return hipErrorInvalidValue;
}

}  // namespace hba
