// hba_step.hip -- one denoising step of block-hybrid attention.
//
// "Retrofitting Linear Attention into Diffusion Language Models", section 3.1:
// for each query q_i of the active block,
//   out_i = (w sum_j exp(q_i.k_j/sqrt d) v_j + phi(q_i)^T S)
//         / (w sum_j exp(q_i.k_j/sqrt d)     + phi(q_i)^T Z).
//
// One workgroup (4 waves) per (request, head).  The step is bound by HBM
// bandwidth: the fp32 state S (2F x d, 128 KB at F = d = 128) is read once and
// dominates the bytes.  Design:
//   * Every wave owns d/4 output columns and streams its column slice of S
//     through a ring of registers: the first kRing 4-row steps are requested
//     at kernel entry, and each step consumed in the main loop requests the
//     step kRing ahead, so ~16 KB per wave stay in flight from the first
//     instruction to the last.
//   * q, k and W are staged in LDS (W transposed in registers on the way).
//     Waves 0 and 1 each own 16 query rows end to end: u = q W and the block
//     scores on MFMA (bf16 MFMA for bf16 inputs: exact products, fp32
//     accumulation; fp32 MFMA for fp32 inputs), then phi(q), phi(q).Z and the
//     softmax weights in the accumulator layout, where a query row sits in
//     one 16-lane DPP row and every reduction is four DPP steps.
//   * Per query the exponent shift c_i = max(m_i + ln w, ln lin_den_i) is
//     applied to both branches, so w exp(s - c) <= 1 and e^{-c} lin_den <= 1.
//   * Both numerators become ONE contraction
//       [w e^{s_i - c_i} | e^{-c_i} phi(q_i)]  x  [V ; S]     (K = L + 2F)
//     on fp32 MFMA; its A operand reuses the LDS of the staged q, k and W.
//     The shared denominator is applied at the store.
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
    static constexpr int bytes = z_off + 2 * F * 4;
};

// Common exponent shift of both branches for one query (section 3.1 merge):
// c = max(m + ln w, ln lin_den), floored at -80 so e^{-c} stays finite.
__device__ __forceinline__ float exp_shift(float m, float lnw, float lin_den) {
    float c = m + lnw;
    if (lin_den > 0.f) c = fmaxf(c, __logf(lin_den));
    return fmaxf(c, -80.f);
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

// Block scores q k^T (unscaled) for 16 query rows row0.. and all 32 keys,
// computed by one wave: s[nt][r] = q[row0 + 4(l/16) + r] . k[16 nt + l%16].
template <typename T, int D, int F>
__device__ __forceinline__ void block_scores16(const T *__restrict__ qs, const T *__restrict__ ks,
                                               int row0, floatx4 (&s)[2]) {
    using P = ProjGeom<T, D, F>;
    const int lane = (int)threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    s[0] = s[1] = floatx4{0.f, 0.f, 0.f, 0.f};
    if constexpr (P::kBf16) {
#pragma unroll
        for (int ks_ = 0; ks_ < D / 32; ++ks_) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(qs + (row0 + li) * P::XLD + 32 * ks_ + 8 * lg);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const bf16x8 b = *reinterpret_cast<const bf16x8 *>(ks + (16 * nt + li) * P::XLD + 32 * ks_ + 8 * lg);
                s[nt] = mfma_bf16(a, b, s[nt]);
            }
        }
    } else {
#pragma unroll 4
        for (int ks_ = 0; ks_ < D / 4; ++ks_) {
            const float a = qs[(row0 + li) * P::XLD + 4 * ks_ + lg];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) s[nt] = mfma_f32(a, ks[(16 * nt + li) * P::XLD + 4 * ks_ + lg], s[nt]);
        }
    }
}

template <typename T, int D, int F>
__global__ __launch_bounds__(kThreads, 3) void step_kernel(StepArgs a) {
    using G = StepGeom<T, D, F>;
    constexpr int EPL = D / 64;       // columns per lane per MFMA column group
    constexpr int NCOL = D / 4;       // output columns owned by one wave
    constexpr int KS = 2 * F / 4;     // 4-row K-steps over the state
    constexpr int RING = KS < 24 ? KS : 24;   // state K-steps kept in flight
    constexpr int NT = F / 16;        // 16-feature tiles of phi
    constexpr float kScale = D == 128 ? 0.08838834764831845f : 0.125f;   // 1/sqrt(d)

    __shared__ __attribute__((aligned(16))) char smem[G::bytes];
    T *qs = reinterpret_cast<T *>(smem + G::q_off);
    T *ks = reinterpret_cast<T *>(smem + G::k_off);
    T *ws = reinterpret_cast<T *>(smem + G::w_off);
    float *As = reinterpret_cast<float *>(smem);
    float *dens = reinterpret_cast<float *>(smem + G::den_off);
    float *zs = reinterpret_cast<float *>(smem + G::z_off);

    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int bh = (int)blockIdx.x;
    const int b = bh / a.H, h = bh - b * a.H;
    const int L = a.L;
    const int64_t slot = a.slot ? (int64_t)a.slot[b] : (int64_t)b;

    const T *qg = static_cast<const T *>(a.q) + (int64_t)bh * L * D;
    const T *kg = static_cast<const T *>(a.k) + (int64_t)bh * L * D;
    const T *vg = static_cast<const T *>(a.v) + (int64_t)bh * L * D;
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
    const float *sp = Sg + (int64_t)lg * D + c0;
    float sreg[KS][EPL];
    auto load_s = [&](int kk) {
        const float *p = sp + (int64_t)(4 * kk) * D;
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
    const float lnw = a.gate ? __logf(a.gate[h]) : 0.f;

    // 3. stage q, k, W
    store_rows<T, D, F>(qc, qs);
    store_rows<T, D, F>(kc, ks);
    store_w<T, D, F>(wc, ws);
    if ((int)threadIdx.x < ZQ) reinterpret_cast<float4 *>(zs)[threadIdx.x] = zq;
    __syncthreads();

    // 4. waves 0-1: u = q W and block scores for query rows 16w .. 16w+15
    const int row0 = 16 * wave;
    floatx4 u[NT], sc[2];
    if (wave < 2) {
        project_rows16<T, D, F>(qs, ws, row0, u);
        block_scores16<T, D, F>(qs, ks, row0, sc);
    }
    __syncthreads();   // q, k, W are dead: their LDS becomes the A operand

    // 5. waves 0-1: per query the shift, block weights and scaled phi(q),
    //    one of the lane's four rows at a time
    if (wave < 2) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = row0 + 4 * lg + r;
            float mx = u[0][r], mn = u[0][r];
#pragma unroll
            for (int nt = 1; nt < NT; ++nt) {
                mx = fmaxf(mx, u[nt][r]);
                mn = fminf(mn, u[nt][r]);
            }
            mx = row16_max(mx);
            mn = row16_min(mn);
            // phi(q) = [softmax(u), softmax(-u)]: sums first, values recomputed
            float sp_ = 0.f, sn_ = 0.f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                sp_ += fast_exp(u[nt][r] - mx);
                sn_ += fast_exp(mn - u[nt][r]);
            }
            const float ip = 1.0f / row16_sum(sp_), in_ = 1.0f / row16_sum(sn_);
            float t = 0.f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                t += fast_exp(u[nt][r] - mx) * ip * zs[16 * nt + li] +
                     fast_exp(mn - u[nt][r]) * in_ * zs[F + 16 * nt + li];
            const float ld = row16_sum(t);   // lin_den = phi(q).Z
            const float s0 = li < L ? sc[0][r] * kScale : -INFINITY;
            const float s1 = (16 + li) < L ? sc[1][r] * kScale : -INFINITY;
            const float m = row16_max(fmaxf(s0, s1));
            const float c = exp_shift(m, lnw, ld);
            const float elin = ld > 0.f ? fast_exp(-c) : 0.f;
            const float p0 = li < L ? fast_exp(s0 + lnw - c) : 0.f;
            const float p1 = (16 + li) < L ? fast_exp(s1 + lnw - c) : 0.f;
            As[a_index(li, i)] = p0;
            As[a_index(16 + li, i)] = p1;
            const float psum = row16_sum(p0 + p1);
            if (li == 0) dens[i] = psum + elin * ld;
            const float ep = ip * elin, en = in_ * elin;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                As[a_index(kRows + 16 * nt + li, i)] = fast_exp(u[nt][r] - mx) * ep;
                As[a_index(kRows + F + 16 * nt + li, i)] = fast_exp(mn - u[nt][r]) * en;
            }
        }
    }
    __syncthreads();

    // 6. merged contraction [w P | e^{-c} phi(q)] x [V ; S] on fp32 MFMA:
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

    // 7. shared normaliser and store
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

template <typename T, int D, int F>
static hipError_t launch_step_t(const StepArgs &a, hipStream_t stream) {
    return launch_kernel(step_kernel<T, D, F>, dim3((unsigned)(a.B * a.H)), dim3(kThreads), a, stream);
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
