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
//     for all 2F rows straight into registers at kernel entry, before any
//     other work, so the whole state read is in flight during the prologue.
//   * q, k and W go through LDS; u = q W and the block scores q k^T run on
//     bf16 MFMA (exact products, fp32 accumulation) or fp32 MFMA for fp32
//     inputs.
//   * Per query the exponent shift c_i = max(m_i + ln w, ln lin_den_i) is
//     applied to both branches, so w exp(s - c) <= 1 and e^{-c} lin_den <= 1.
//   * Both numerators become ONE contraction
//       [w e^{s_i - c_i} | e^{-c_i} phi(q_i)]  x  [V ; S]     (K = L + 2F)
//     on fp32 MFMA, with the shared denominator applied at the store.
#include "hba_device.h"
#include "hba_internal.h"

namespace hba {

template <typename T, int D, int F>
struct StepGeom {
    using P = ProjGeom<T, D, F>;
    static constexpr int KROWS = kRows + 2 * F;   // rows of the merged contraction
    static constexpr int SLD = 36;                // score tile row stride (floats)
    // region 1: q tile, k tile, W  -- dead after the projections, then reused
    // for the merged A operand [KROWS][32] fp32
    static constexpr int q_off = 0;
    static constexpr int k_off = P::x_bytes;
    static constexpr int w_off = 2 * P::x_bytes;
    static constexpr int r1_in = 2 * P::x_bytes + P::w_bytes;
    static constexpr int a_bytes = KROWS * 32 * 4;
    static constexpr int r1 = r1_in > a_bytes ? r1_in : a_bytes;
    static constexpr int u_off = r1;
    static constexpr int s_off = u_off + P::u_bytes;
    static constexpr int den_off = s_off + kRows * SLD * 4;
    static constexpr int bytes = den_off + kRows * 4;
};

// Row k of the merged A operand holds the 32 queries interleaved as
// (i, i + 16) pairs, XOR-swizzled by k so that both the per-query column
// writes and the MFMA pair reads avoid LDS bank conflicts.
__device__ __forceinline__ int a_index(int k, int i) {
    return k * 32 + ((2 * (i & 15) + (i >> 4)) ^ (2 * (k & 15)));
}
__device__ __forceinline__ int a_pair(int k, int li) {
    return k * 32 + ((2 * li) ^ (2 * (k & 15)));
}

// Load n consecutive input elements and widen to fp32.
template <typename T, int N>
__device__ __forceinline__ void load_widen(const T *__restrict__ p, float (&o)[N]) {
    if constexpr (sizeof(T) == 4) {
        if constexpr (N == 2) {
            const float2 t = *reinterpret_cast<const float2 *>(p);
            o[0] = t.x;
            o[1] = t.y;
        } else {
#pragma unroll
            for (int e = 0; e < N; ++e) o[e] = p[e];
        }
    } else {
        if constexpr (N == 2) {
            const uint32_t t = *reinterpret_cast<const uint32_t *>(p);
            o[0] = bf16_bits_to_f32(t & 0xffffu);
            o[1] = bf16_bits_to_f32(t >> 16);
        } else {
#pragma unroll
            for (int e = 0; e < N; ++e) o[e] = to_f32(p[e]);
        }
    }
}

// s = q k^T (unscaled) for the 32x32 block; wave w computes 16x16 tile w.
template <typename T, int D, int F>
__device__ __forceinline__ void block_scores(const T *__restrict__ qs, const T *__restrict__ ks,
                                             float *__restrict__ ss) {
    using P = ProjGeom<T, D, F>;
    using G = StepGeom<T, D, F>;
    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int mt = wave >> 1, nt = wave & 1;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (P::kBf16) {
#pragma unroll
        for (int ks_ = 0; ks_ < D / 32; ++ks_) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(qs + (16 * mt + li) * P::XLD + 32 * ks_ + 8 * lg);
            const bf16x8 b = *reinterpret_cast<const bf16x8 *>(ks + (16 * nt + li) * P::XLD + 32 * ks_ + 8 * lg);
            acc = mfma_bf16(a, b, acc);
        }
    } else {
#pragma unroll
        for (int ks_ = 0; ks_ < D / 4; ++ks_) {
            acc = mfma_f32(qs[(16 * mt + li) * P::XLD + 4 * ks_ + lg],
                           ks[(16 * nt + li) * P::XLD + 4 * ks_ + lg], acc);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) ss[(16 * mt + 4 * lg + r) * G::SLD + 16 * nt + li] = acc[r];
}

template <typename T, int D, int F>
__global__ __launch_bounds__(kThreads) void step_kernel(StepArgs a) {
    using P = ProjGeom<T, D, F>;
    using G = StepGeom<T, D, F>;
    constexpr int EPL = D / 64;       // columns per lane per MFMA column group
    constexpr int NCOL = D / 4;       // output columns owned by one wave
    constexpr int KS = 2 * F / 4;     // 4-row K-steps over the state
    constexpr int FM = F / 64;
    constexpr float kScale = D == 128 ? 0.08838834764831845f : 0.125f;   // 1/sqrt(d)

    __shared__ __attribute__((aligned(16))) char smem[G::bytes];
    T *qs = reinterpret_cast<T *>(smem + G::q_off);
    T *ks = reinterpret_cast<T *>(smem + G::k_off);
    T *ws = reinterpret_cast<T *>(smem + G::w_off);
    float *As = reinterpret_cast<float *>(smem);
    float *us = reinterpret_cast<float *>(smem + G::u_off);
    float *ss = reinterpret_cast<float *>(smem + G::s_off);
    float *dens = reinterpret_cast<float *>(smem + G::den_off);

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

    // 2. the state stream: this wave's column slice of S, all 2F rows
    const int c0 = wave * NCOL + EPL * li;
    float sreg[KS][EPL];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const float *p = Sg + (int64_t)(4 * kk + lg) * D + c0;
        if constexpr (EPL == 2) {
            const floatx2 t = __builtin_nontemporal_load(reinterpret_cast<const floatx2 *>(p));
            sreg[kk][0] = t[0];
            sreg[kk][1] = t[1];
        } else {
            sreg[kk][0] = __builtin_nontemporal_load(p);
        }
    }
    // block values (B operand rows 0..31 of the merged contraction)
    float vreg[8][EPL];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const int j = 4 * kk + lg;
        load_widen<T, EPL>(vg + (int64_t)(j < L ? j : L - 1) * D + c0, vreg[kk]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) vreg[kk][e] = j < L ? vreg[kk][e] : 0.f;
    }
    float zr[2 * FM];
#pragma unroll
    for (int m = 0; m < 2 * FM; ++m) zr[m] = Zg[lane + 64 * m];
    const float lnw = a.gate ? __logf(a.gate[h]) : 0.f;

    // 3. stage q, k, W
    store_rows<T, D, F>(qc, qs);
    store_rows<T, D, F>(kc, ks);
    store_w<T, D, F>(wc, ws);
    __syncthreads();

    // 4. u = q W and s = q k^T
    project_tile<T, D, F>(qs, ws, us);
    block_scores<T, D, F>(qs, ks, ss);
    __syncthreads();

    // 5. per query: phi(q), lin_den, shared shift, merged A operand row
#pragma unroll 1
    for (int ii = 0; ii < 8; ++ii) {
        const int i = 8 * wave + ii;
        if (i >= L) break;
        float pp[FM], pn[FM];
        phi_of_row<F>(us + i * P::ULD, lane, pp, pn);
        float ld = 0.f;
#pragma unroll
        for (int m = 0; m < FM; ++m) ld += pp[m] * zr[m] + pn[m] * zr[FM + m];
        const float lin_den = wave_sum(ld);
        const float sj = lane < L ? ss[i * G::SLD + lane] * kScale : -INFINITY;
        const float mx = wave_max(sj);
        float c = mx + lnw;
        if (lin_den > 0.f) c = fmaxf(c, __logf(lin_den));
        c = fmaxf(c, -80.f);
        const float p = lane < L ? fast_exp(sj + lnw - c) : 0.f;
        const float sm_den = wave_sum(p);
        const float elin = lin_den > 0.f ? fast_exp(-c) : 0.f;
        if (lane < 32) As[a_index(lane, i)] = p;
#pragma unroll
        for (int m = 0; m < FM; ++m) {
            As[a_index(kRows + lane + 64 * m, i)] = pp[m] * elin;
            As[a_index(kRows + F + lane + 64 * m, i)] = pn[m] * elin;
        }
        if (lane == 0) dens[i] = sm_den + elin * lin_den;
    }
    __syncthreads();

    // 6. merged contraction [w P | e^{-c} phi(q)] x [V ; S] on fp32 MFMA
    floatx4 acc[2][EPL];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[t][e] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        const float2 av = *reinterpret_cast<const float2 *>(As + a_pair(4 * kk + lg, li));
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            acc[0][e] = mfma_f32(av.x, vreg[kk][e], acc[0][e]);
            acc[1][e] = mfma_f32(av.y, vreg[kk][e], acc[1][e]);
        }
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const float2 av = *reinterpret_cast<const float2 *>(As + a_pair(kRows + 4 * kk + lg, li));
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            acc[0][e] = mfma_f32(av.x, sreg[kk][e], acc[0][e]);
            acc[1][e] = mfma_f32(av.y, sreg[kk][e], acc[1][e]);
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
