// hba_step_commit.hip -- the last denoising step of a block fused with the
// commit of that block.
//
// "Retrofitting Linear Attention into Diffusion Language Models", section 3.1
// (the step and the state update) and section 3.3 (one launch per hybrid
// layer with its causal state update): out is the block-hybrid step on the
// state as it was, then the block's keys and values are folded into S and Z,
//   S += phi(K)^T V,  Z += sum_t phi(k_t)   (tokens t < n_valid).
// One pass reads S once and writes S + phi(K)^T V once; a separate step and
// commit read it twice.
//
// bf16 inputs, d = 128: one workgroup of eight waves per (request, head).
//   * Waves 0-3 stage q, k and W^T in LDS.  Waves 0-3 then form phi(q) (waves
//     0-1 the softmax(u) half, 2-3 the softmax(-u) half, as u^T = W^T q^T so
//     a lane holds features of one query) and waves 2-3 the block softmax;
//     waves 4-7 form phi(K) as u = K W, so a lane holds four consecutive
//     tokens of one feature: phi(K)^T goes to LDS as a bf16 high part and
//     residual in [feature][token] order, and the per-feature token sums for
//     Z are taken in registers.
//   * Every wave owns 16 output columns and streams its column slice of S
//     through a register ring.  Per 32-row chunk it runs the step's
//     contraction and then dS = phi(K)^T V on bf16 MFMA, whose B operand is
//     the block values it already holds for the step; the A rows are taken
//     in the order that makes dS land in exactly the lanes and rows that
//     hold the streamed chunk, so S + dS is stored in place at once.
// Other dtypes and shapes run the step kernel, then the commit kernel.
#include "hba_device.h"
#include "hba_internal.h"

namespace hba {

template <int D, int F>
struct FusedGeom {
    using P = ProjGeom<uint16_t, D, F>;
    static constexpr int KP = kRows + 2 * F + 8;           // step A operand row stride (bf16)
    static constexpr int a_bytes = 2 * kRows * KP * 2;     // step A operand: hi rows, then lo rows
    static constexpr int KT = kRows + 8;                   // phi(K)^T row stride (bf16): tokens + pad
    static constexpr int kt_off = a_bytes;                 // phi(K)^T: hi rows [2F][KT], then lo rows
    static constexpr int kt_bytes = 2 * (2 * F) * KT * 2;
    static constexpr int in_bytes = 2 * P::x_bytes + P::w_bytes;   // q, k, W^T staging
    static constexpr int r1 = in_bytes > kt_off + kt_bytes ? in_bytes : kt_off + kt_bytes;
    static constexpr int z_off = r1;                        // old Z [2F]
    static constexpr int zk_off = z_off + 2 * F * 4;        // sum over 16 tokens of phi(k_t) [2][2F]
    // per query i: phi+.Z+, phi-.Z-, block max, block sum live in the 16-byte
    // pad at the end of A_hi row i (columns kRows + 2F .. KP, never an MFMA
    // operand), which keeps the whole layout at 80 KB: two workgroups per CU
    static constexpr int row_pad = kRows + 2 * F;
    static constexpr int bytes = zk_off + 2 * 2 * F * 4;
    static_assert(KP - row_pad == 8, "four floats per A_hi row pad");
};
constexpr int kFusedThreads = 512;

template <int D, int F>
__global__ __launch_bounds__(kFusedThreads, 2) void step_commit_kernel_bf16(StepCommitArgs a) {
    using T = uint16_t;
    using P = ProjGeom<T, D, F>;
    using G = FusedGeom<D, F>;
    static_assert(D == 128, "eight waves of 16 output columns");
    constexpr int NCH = 2 * F / 32;   // 32-row chunks of the state
    constexpr int RING = NCH / 2 < 2 ? NCH / 2 : 2;
    constexpr int PRE = NCH / 2;   // every chunk is requested before the contraction
                                // (measured: 150.3 -> 147.6 us at B=128, 39.6 -> 36.4 us at B=32)
    constexpr int NT = F / 16;        // 16-feature tiles
    constexpr int KS = D / 32;        // K-steps of the projections
    constexpr int ZQ = 2 * F / 4;
    constexpr float kS2 = 0.08838834764831845f * kLog2e;   // log2(e)/sqrt(128)

    __shared__ __attribute__((aligned(16))) char smem[G::bytes];
    T *qs = reinterpret_cast<T *>(smem);
    T *ks = reinterpret_cast<T *>(smem + P::x_bytes);
    T *ws = reinterpret_cast<T *>(smem + 2 * P::x_bytes);
    T *Ahi = reinterpret_cast<T *>(smem);
    T *Alo = Ahi + kRows * G::KP;
    T *Khi = reinterpret_cast<T *>(smem + G::kt_off);
    T *Klo = Khi + 2 * F * G::KT;
    float *zs = reinterpret_cast<float *>(smem + G::z_off);
    float *zk = reinterpret_cast<float *>(smem + G::zk_off);
    auto rowv = [&](int i) { return reinterpret_cast<float *>(Ahi + i * G::KP + G::row_pad); };

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int bh = (int)blockIdx.x;
    const int b = bh / a.H, h = bh - b * a.H;
    const int L = a.L;
    int nv = a.n_valid ? a.n_valid[b] : L;
    nv = nv < 0 ? 0 : (nv > L ? L : nv);
    const int64_t slot = a.slot ? (int64_t)a.slot[b] : (int64_t)b;

    const T *qg = static_cast<const T *>(a.q) + (int64_t)bh * L * D;
    const T *kg = static_cast<const T *>(a.k) + (int64_t)(bh / a.G) * L * D;
    const T *vg = static_cast<const T *>(a.v) + (int64_t)(bh / a.G) * L * D;
    const T *Wg = static_cast<const T *>(a.W) + (int64_t)h * D * F;
    float *Sg = a.S + (slot * a.H + h) * (int64_t)(2 * F) * D;
    float *Zg = a.Z + (slot * a.H + h) * (int64_t)(2 * F);

    // 1. q, k, W (waves 0-3) and Z, then the ring head of every wave's column
    //    slice: chunk c holds rows 32c + 8 lg + t (t < 8) of column c0
    RowChunks<T, D> qc, kc;
    WChunks<T, D, F> wc;
    if (wave < 4) {
        load_rows<T, D>(qg, D, L, qc);
        load_rows<T, D>(kg, D, L, kc);
        load_w<T, D, F>(Wg, wc);
    }
    float4 zq = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < ZQ) zq = reinterpret_cast<const float4 *>(Zg)[tid];
    // streaming layout: wave w owns columns 32 (w mod 4) .. +31 (two per
    // lane: c0, c0 + 1) of state rows 128 (w / 4) .. +127 (F = 128); the two
    // row halves' partial step sums meet in LDS at the end
    constexpr int NCHW = NCH / 2;                // chunks per wave
    const int cp = wave & 3, rh = wave >> 2;
    const int c0 = 32 * cp + 2 * li;
    float sreg[NCHW][8][2];
    auto load_chunk = [&](int cl) {
        const int c = rh * NCHW + cl;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const floatx2 v2 = __builtin_nontemporal_load(reinterpret_cast<const floatx2 *>(Sg + (int64_t)(32 * c + 8 * lg + t) * D + c0));
            sreg[cl][t][0] = v2[0];
            sreg[cl][t][1] = v2[1];
        }
    };
#pragma unroll
    for (int c = 0; c < RING; ++c) load_chunk(c);
    const float lw2 = a.gate ? __log2f(a.gate[h]) : 0.f;   // log2 w
    // block values of keys 8 lg + t, columns c0 and c0 + 1, requested with
    // the other small inputs: the first chunk's dS needs them
    uint32_t vw[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int j = 8 * lg + t;
        vw[t] = *reinterpret_cast<const uint32_t *>(vg + (j < L ? j : L - 1) * D + c0);
    }

    if (wave < 4) {
        store_rows<T, D, F>(qc, qs);
        store_rows<T, D, F>(kc, ks);
        store_w<T, D, F>(wc, ws);
    }
    if (tid < ZQ) reinterpret_cast<float4 *>(zs)[tid] = zq;
    __syncthreads();
#pragma unroll
    for (int c = RING; c < PRE; ++c) load_chunk(c);
    __builtin_amdgcn_sched_barrier(0);

    // 2. projections.  waves 0-3: u_q^T for queries 16 (w mod 2) .. +15,
    //    acc[m][r] = u[query 16 g + l%16][feature 16m + 4(l/16) + r]; waves 2-3
    //    also the block scores of those queries.  waves 4-7: u_k = K W for
    //    tokens 16 (w mod 2) .. +15, acc[m][r] = u[token 16 g + 4(l/16) + r][feature 16m + l%16]
    const int grp = wave & 1;
    floatx4 acc[NT], sc[2];
#pragma unroll
    for (int m = 0; m < NT; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (wave < 4) {
#pragma unroll
        for (int ks_ = 0; ks_ < KS; ++ks_) {
            const bf16x8 bq = *reinterpret_cast<const bf16x8 *>(qs + (16 * grp + li) * P::XLD + 32 * ks_ + 8 * lg);
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                const bf16x8 aw = *reinterpret_cast<const bf16x8 *>(ws + wt_off<D>(16 * m + li, 4 * ks_ + lg));
                acc[m] = mfma_bf16(aw, bq, acc[m]);
            }
        }
        if (wave >= 2) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                sc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks_ = 0; ks_ < KS; ++ks_) {
                    const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(qs + (16 * grp + li) * P::XLD + 32 * ks_ + 8 * lg);
                    const bf16x8 bk = *reinterpret_cast<const bf16x8 *>(ks + (16 * nt + li) * P::XLD + 32 * ks_ + 8 * lg);
                    sc[nt] = mfma_bf16(aq, bk, sc[nt]);
                }
            }
        }
    } else {
#pragma unroll
        for (int ks_ = 0; ks_ < KS; ++ks_) {
            const bf16x8 ak = *reinterpret_cast<const bf16x8 *>(ks + (16 * grp + li) * P::XLD + 32 * ks_ + 8 * lg);
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                const bf16x8 bw = *reinterpret_cast<const bf16x8 *>(ws + wt_off<D>(16 * m + li, 4 * ks_ + lg));
                acc[m] = mfma_bf16(ak, bw, acc[m]);
            }
        }
    }
    __syncthreads();   // q, k and W^T are dead: their LDS becomes the operands below

    // 3. operands in LDS
    if (wave < 4) {
        // this wave's half of phi(q_i) = softmax(sgn u_i) and of lin_den = phi(q_i).Z
        const int qi = 16 * grp + li;
        const int half = wave >> 1;
        const float sgn2 = half ? -kLog2e : kLog2e;
        float mx = -INFINITY;
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[m][r] *= sgn2;
                mx = fmaxf(mx, acc[m][r]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        float sm = 0.f;
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[m][r] = fast_exp2(acc[m][r] - mx);
                sm += acc[m][r];
            }
        sm += __shfl_xor(sm, 16, kWave);
        sm += __shfl_xor(sm, 32, kWave);
        const float is = 1.0f / sm;
        float zd = 0.f;
        T *ah = Ahi + qi * G::KP + kRows + half * F + 4 * lg;
        T *al = Alo + qi * G::KP + kRows + half * F + 4 * lg;
        const float *zh = zs + half * F + 4 * lg;
#pragma unroll
        for (int m = 0; m < NT; ++m) {
            const float4 z4 = *reinterpret_cast<const float4 *>(zh + 16 * m);
            const float e0 = acc[m][0] * is, e1 = acc[m][1] * is, e2 = acc[m][2] * is, e3 = acc[m][3] * is;
            zd += e0 * z4.x + e1 * z4.y + e2 * z4.z + e3 * z4.w;
            uint32_t hw[2], lw[2];
            split_pk_bf16(e0, e1, hw[0], lw[0]);
            split_pk_bf16(e2, e3, hw[1], lw[1]);
            *reinterpret_cast<uint2 *>(ah + 16 * m) = make_uint2(hw[0], hw[1]);
            *reinterpret_cast<uint2 *>(al + 16 * m) = make_uint2(lw[0], lw[1]);
        }
        zd += __shfl_xor(zd, 16, kWave);
        zd += __shfl_xor(zd, 32, kWave);
        if (lg == 0) rowv(qi)[half] = zd;
        if (wave >= 2) {
            // block softmax of the same queries, relative to the row maximum
            const bool kv0 = li < L, kv1 = (16 + li) < L;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * grp + 4 * lg + r;
                const float s0 = kv0 ? sc[0][r] * kS2 : -INFINITY;
                const float s1 = kv1 ? sc[1][r] * kS2 : -INFINITY;
                const float m2 = row16_max(fmaxf(s0, s1));
                const float p0 = kv0 ? fast_exp2(s0 - m2) : 0.f;
                const float p1 = kv1 ? fast_exp2(s1 - m2) : 0.f;
                const float as = row16_sum(p0 + p1);
                Ahi[i * G::KP + li] = __builtin_bit_cast(uint16_t, (__bf16)p0);
                Ahi[i * G::KP + 16 + li] = __builtin_bit_cast(uint16_t, (__bf16)p1);
                Alo[i * G::KP + li] = __builtin_bit_cast(uint16_t, (__bf16)bf16_residual(p0));
                Alo[i * G::KP + 16 + li] = __builtin_bit_cast(uint16_t, (__bf16)bf16_residual(p1));
                if (li == 0) {
                    rowv(i)[2] = m2;
                    rowv(i)[3] = as;
                }
            }
        }
    } else {
        // this wave's half of phi(k_t) for tokens 16 g + 4(l/16) + r, feature
        // half F + 16m + l%16; tokens past n_valid get phi = 0
        const int half = (wave >> 1) & 1;
        const float sgn2 = half ? -kLog2e : kLog2e;
        float mx[4], is[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float m0 = -INFINITY;
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                acc[m][r] *= sgn2;
                m0 = fmaxf(m0, acc[m][r]);
            }
            mx[r] = row16_max(m0);   // over the 16 lanes holding this token's features
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float s0 = 0.f;
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                acc[m][r] = fast_exp2(acc[m][r] - mx[r]);
                s0 += acc[m][r];
            }
            const bool ok = 16 * grp + 4 * lg + r < nv;
            is[r] = ok ? 1.0f / row16_sum(s0) : 0.f;
        }
        const int t0 = 16 * grp + 4 * lg;
#pragma unroll
        for (int m = 0; m < NT; ++m) {
            const int f = half * F + 16 * m + li;
            const float e0 = acc[m][0] * is[0], e1 = acc[m][1] * is[1], e2 = acc[m][2] * is[2], e3 = acc[m][3] * is[3];
            uint32_t hw[2], lw[2];
            split_pk_bf16(e0, e1, hw[0], lw[0]);
            split_pk_bf16(e2, e3, hw[1], lw[1]);
            *reinterpret_cast<uint2 *>(Khi + f * G::KT + t0) = make_uint2(hw[0], hw[1]);
            *reinterpret_cast<uint2 *>(Klo + f * G::KT + t0) = make_uint2(lw[0], lw[1]);
            float zt = (e0 + e1) + (e2 + e3);   // this lane's four tokens
            zt += __shfl_xor(zt, 16, kWave);
            zt += __shfl_xor(zt, 32, kWave);
            if (lg == 0) zk[grp * 2 * F + f] = zt;
        }
    }
    __syncthreads();

    // 4. the stream: step contraction, then S + phi(K)^T V stored in place
    floatx4 accS[2][2], accV[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 2; ++e) accS[t][e] = accV[t][e] = floatx4{0.f, 0.f, 0.f, 0.f};
    // block values of keys 8 lg + t, columns c0 and c0 + 1: the B operands of
    // both the step's V part and dS (keys past the block repeat row L-1;
    // their weights and phi are exactly 0)
    bf16x8 bv[2];
    {
        uint32_t p0[4], p1[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p0[j] = __builtin_amdgcn_perm(vw[2 * j + 1], vw[2 * j], 0x05040100u);
            p1[j] = __builtin_amdgcn_perm(vw[2 * j + 1], vw[2 * j], 0x07060302u);
        }
        bv[0] = __builtin_bit_cast(bf16x8, make_uint4(p0[0], p0[1], p0[2], p0[3]));
        bv[1] = __builtin_bit_cast(bf16x8, make_uint4(p1[0], p1[1], p1[2], p1[3]));
    }
    const bool commit = nv > 0;   // nothing to fold: the state is left untouched
#pragma unroll
    for (int cl = 0; cl < NCHW; ++cl) {
        if (cl + RING < NCHW && cl + RING >= PRE) load_chunk(cl + RING);
        __builtin_amdgcn_sched_barrier(0);
        const int c = rh * NCHW + cl;
        bf16x8 bh_[2], bl_[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) split_pk_bf16(sreg[cl][2 * j][e], sreg[cl][2 * j + 1][e], hw[j], lw[j]);
            bh_[e] = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
            bl_[e] = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
        }
        const int k0 = kRows + 32 * c + 8 * lg;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(Ahi + (16 * mt + li) * G::KP + k0);
            const bf16x8 al = *reinterpret_cast<const bf16x8 *>(Alo + (16 * mt + li) * G::KP + k0);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                accS[mt][e] = mfma_bf16(ah, bh_[e], accS[mt][e]);
                accS[mt][e] = mfma_bf16(ah, bl_[e], accS[mt][e]);
                accS[mt][e] = mfma_bf16(al, bh_[e], accS[mt][e]);
            }
        }
        if (commit) {
            // dS tile mt, row 4(l/16) + r = chunk row 8(l/16) + 4 mt + r: the A
            // operand row of lane l%16 = 4 g + r' is state row 32c + 8g + 4mt + r'
            const int frow = 32 * c + 8 * (li >> 2) + (li & 3);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const bf16x8 kh = *reinterpret_cast<const bf16x8 *>(Khi + (frow + 4 * mt) * G::KT + 8 * lg);
                const bf16x8 kl = *reinterpret_cast<const bf16x8 *>(Klo + (frow + 4 * mt) * G::KT + 8 * lg);
                floatx4 ds[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    ds[e] = mfma_bf16(kh, bv[e], floatx4{0.f, 0.f, 0.f, 0.f});
                    ds[e] = mfma_bf16(kl, bv[e], ds[e]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const floatx2 o2 = {sreg[cl][4 * mt + r][0] + ds[0][r], sreg[cl][4 * mt + r][1] + ds[1][r]};
                    __builtin_nontemporal_store(o2, reinterpret_cast<floatx2 *>(Sg + (int64_t)(32 * c + 8 * lg + 4 * mt + r) * D + c0));
                }
            }
        }
    }
    if (rh == 0) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(Ahi + (16 * mt + li) * G::KP + 8 * lg);
            const bf16x8 al = *reinterpret_cast<const bf16x8 *>(Alo + (16 * mt + li) * G::KP + 8 * lg);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                accV[mt][e] = mfma_bf16(ah, bv[e], accV[mt][e]);
                accV[mt][e] = mfma_bf16(al, bv[e], accV[mt][e]);
            }
        }
    }
    // the second row half's partial sums through LDS (phi(K)^T is dead)
    __syncthreads();
    floatx4 *xs = reinterpret_cast<floatx4 *>(Khi) + (cp * kWave + lane) * 4;
    if (rh == 1) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int e = 0; e < 2; ++e) xs[2 * mt + e] = accS[mt][e];
    }
    __syncthreads();

    // 5. merge with one shift per query, out = (sv accV + ss accS) / (sv a + ss ld)
    if (rh == 0) {
        float *og = a.out + (int64_t)bh * L * D;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const floatx4 o0 = accS[mt][0] + xs[2 * mt + 0], o1 = accS[mt][1] + xs[2 * mt + 1];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * mt + 4 * lg + r;
                if (i < L) {
                    const float4 rv = *reinterpret_cast<const float4 *>(rowv(i));
                    const float ld = rv.x + rv.y, g2 = rv.z + lw2, as = rv.w;
                    float cc = g2;
                    if (ld > 0.f) cc = fmaxf(cc, __log2f(ld));
                    cc = fmaxf(cc, -120.f);
                    const float sv = fast_exp2(g2 - cc);
                    const float ss = ld > 0.f ? fast_exp2(-cc) : 0.f;
                    const float inv = __builtin_amdgcn_rcpf(sv * as + ss * ld);
                    const floatx2 v2 = {(sv * accV[mt][0][r] + ss * o0[r]) * inv, (sv * accV[mt][1][r] + ss * o1[r]) * inv};
                    __builtin_nontemporal_store(v2, reinterpret_cast<floatx2 *>(og + (int64_t)i * D + c0));
                }
            }
        }
    }
    // 6. Z += sum_t phi(k_t)
    if (commit && tid < 2 * F) __builtin_nontemporal_store(zs[tid] + zk[tid] + zk[2 * F + tid], Zg + tid);
}

hipError_t launch_step_commit(const StepCommitArgs &a, bool bf16, int d, int F, hipStream_t stream) {
    if (bf16 && d == 128) {
        if (F == 128)
            return launch_kernel(step_commit_kernel_bf16<128, 128>, dim3((unsigned)(a.B * a.H)), dim3(kFusedThreads), a, stream);
        if (F == 64)
            return launch_kernel(step_commit_kernel_bf16<128, 64>, dim3((unsigned)(a.B * a.H)), dim3(kFusedThreads), a, stream);
    }
    // other shapes: the step on the current state, then the commit
    const StepArgs s{a.q, a.k, a.v, a.W, a.gate, a.S, a.Z, a.slot, a.out, a.B, a.H, a.L, a.G};
    hipError_t e = launch_step(s, bf16, d, F, stream);
    if (e != hipSuccess) return e;
    const CommitArgs c{a.n_valid, a.k, a.v, a.W, a.S, a.Z, a.slot, a.B, a.H, a.L, a.G};
    return launch_commit(c, bf16, d, F, stream);
}

}  // namespace hba
