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
// bf16 inputs, d = 128: one workgroup of four waves per (request, head), two
// workgroups per CU (80 KB of LDS at F = 128), so that one pair's prologue
// overlaps another pair's state stream.
//   * All four waves stage q, k and W^T in LDS.  Waves 0-1 then form phi(q)
//     of 16 queries each, both signs (u^T = W^T q^T, so a lane holds features
//     of one query); waves 2-3 form the block scores and softmax of the same
//     queries, then phi(K) of 16 tokens each, both signs, as u = K W (a lane
//     holds four consecutive tokens of one feature): phi(K)^T goes to LDS as
//     a bf16 high part and residual in [feature][token] order, and the
//     per-feature token sums for Z are taken in registers.
//   * Wave w owns the F state rows of feature half w / 2 and the value
//     columns of column block w mod 2 (64 columns, four per lane, or 32 with
//     two workgroups per pair), and holds that slice in registers, requested
//     before the prologue: every state access is a 16-byte (8-byte) access,
//     a 256-byte (128-byte) row segment per 16 lanes.  Per 32-row chunk it
//     runs its part of the step's contraction (this half's features) and
//     then dS = phi(K)^T V on bf16 MFMA, whose B operand is the block values
//     it already holds for the step; the A rows are taken in the order that
//     makes dS land in exactly the lanes and rows that hold the streamed
//     chunk, so S + dS is stored in place at once.
//   * The two halves' step partials of a column block meet in LDS; the wave
//     of the first half adds the block-softmax part, merges and stores.
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

template <int D, int F, int NSPLIT>
__global__ __launch_bounds__(kThreads, 2) void step_commit_kernel_bf16(StepCommitArgs a) {
    using T = uint16_t;
    using P = ProjGeom<T, D, F>;
    using G = FusedGeom<D, F>;
    // NSPLIT workgroups per (request, head), each owning D/NSPLIT value
    // columns of the output and the state; each forms the whole prologue
    static_assert(D == 128 && (NSPLIT == 1 || NSPLIT == 2), "two column blocks of 64 or 32 value columns");
    constexpr int EPL = 4 / NSPLIT;   // columns per lane (N-tiles of the state contraction)
    constexpr int CB = 16 * EPL;      // columns per wave
    constexpr int NCH = F / 32;       // 32-row chunks of this wave's feature half
    constexpr int RING = 1;           // chunks requested at entry (the rest after staging)
    constexpr int NT = F / 16;
    constexpr int KS = D / 32;
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
    const int bh = (int)blockIdx.x / NSPLIT, part = (int)blockIdx.x - bh * NSPLIT;
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

    // 1. q, k, W, Z, then the ring head of the state
    RowChunks<T, D> qc, kc;
    WChunks<T, D, F> wc;
    load_rows<T, D>(qg, D, L, qc);
    load_rows<T, D>(kg, D, L, kc);
    load_w<T, D, F>(Wg, wc);
    float4 zq = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < ZQ) zq = reinterpret_cast<const float4 *>(Zg)[tid];
    const int sh = wave >> 1;   // feature half of this wave's state rows
    const int c0 = part * (D / NSPLIT) + CB * (wave & 1) + EPL * li;   // its columns c0 .. c0 + EPL - 1
    // chunk c holds rows sh F + 32 c + 8 lg + t (t < 8); 32-bit element
    // offsets from the uniform state base
    const int lofs = (sh * F + 8 * lg) * D + c0;
    float sreg[NCH][8][EPL];
    auto load_chunk = [&](int c) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if constexpr (EPL == 4) {
                const floatx4 v4 = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(Sg + (lofs + (32 * c + t) * D)));
#pragma unroll
                for (int e = 0; e < 4; ++e) sreg[c][t][e] = v4[e];
            } else {
                const floatx2 v2 = __builtin_nontemporal_load(reinterpret_cast<const floatx2 *>(Sg + (lofs + (32 * c + t) * D)));
                sreg[c][t][0] = v2[0];
                sreg[c][t][1] = v2[1];
            }
        }
    };
#pragma unroll
    for (int c = 0; c < RING; ++c) load_chunk(c);
    const float lw2 = a.gate ? __log2f(a.gate[h]) : 0.f;   // log2 w
    uint32_t vw[8][EPL / 2];   // tokens 8 lg + t, columns c0 .. (two per word)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int j = 8 * lg + t;
        const T *p = vg + (j < L ? j : L - 1) * D + c0;
        if constexpr (EPL == 4) {
            const uint2 w2 = *reinterpret_cast<const uint2 *>(p);
            vw[t][0] = w2.x;
            vw[t][1] = w2.y;
        } else {
            vw[t][0] = *reinterpret_cast<const uint32_t *>(p);
        }
    }
    store_rows<T, D, F>(qc, qs);
    store_rows<T, D, F>(kc, ks);
    store_w<T, D, F>(wc, ws);
    if (tid < ZQ) reinterpret_cast<float4 *>(zs)[tid] = zq;
    __syncthreads();
#pragma unroll
    for (int c = RING; c < NCH; ++c) load_chunk(c);
    __builtin_amdgcn_sched_barrier(0);

    // 2. projections: waves 0-1 u_q^T (acc[m][r] = u[query 16 g + l%16][feature
    //    16m + 4(l/16) + r]); waves 2-3 the block scores, then u_k = K W
    //    (acc[m][r] = u[token 16 g + 4(l/16) + r][feature 16m + l%16])
    const int grp = wave & 1;
    floatx4 acc[NT], sc[2];
#pragma unroll
    for (int m = 0; m < NT; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (wave < 2) {
#pragma unroll
        for (int ks_ = 0; ks_ < KS; ++ks_) {
            const bf16x8 bq = *reinterpret_cast<const bf16x8 *>(qs + (16 * grp + li) * P::XLD + 32 * ks_ + 8 * lg);
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                const bf16x8 aw = *reinterpret_cast<const bf16x8 *>(ws + wt_off<D>(16 * m + li, 4 * ks_ + lg));
                acc[m] = mfma_bf16(aw, bq, acc[m]);
            }
        }
    } else {
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
    if (wave < 2) {
        // phi(q_i) = [softmax(u_i), softmax(-u_i)] and both halves of lin_den
        const int qi = 16 * grp + li;
        float mx = -INFINITY, mn = INFINITY;
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[m][r] *= kLog2e;
                mx = fmaxf(mx, acc[m][r]);
                mn = fminf(mn, acc[m][r]);
            }
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
        float zdp = 0.f, zdn = 0.f;
        T *ah = Ahi + qi * G::KP + kRows + 4 * lg;
        T *al = Alo + qi * G::KP + kRows + 4 * lg;
#pragma unroll
        for (int m = 0; m < NT; ++m) {
            const float4 zp4 = *reinterpret_cast<const float4 *>(zs + 16 * m + 4 * lg);
            const float4 zn4 = *reinterpret_cast<const float4 *>(zs + F + 16 * m + 4 * lg);
            float ep[4], en[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                ep[r] = fast_exp2(acc[m][r] - mx) * ip;
                en[r] = fast_exp2(mn - acc[m][r]) * in_;
            }
            zdp += ep[0] * zp4.x + ep[1] * zp4.y + ep[2] * zp4.z + ep[3] * zp4.w;
            zdn += en[0] * zn4.x + en[1] * zn4.y + en[2] * zn4.z + en[3] * zn4.w;
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
        zdp = xrow_sum(zdp);
        zdn = xrow_sum(zdn);
        if (lg == 0) {
            rowv(qi)[0] = zdp;
            rowv(qi)[1] = zdn;
        }
    } else {
        // block softmax of queries 16 g .. +15, relative to the row maximum
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
        // phi(k_t) for tokens 16 g + 4(l/16) + r, both halves (features
        // half F + 16m + l%16); tokens past n_valid get phi = 0
        const int t0 = 16 * grp + 4 * lg;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const float sgn2 = half ? -kLog2e : kLog2e;
            float mx[4], is[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float m0 = -INFINITY;
#pragma unroll
                for (int m = 0; m < NT; ++m) m0 = fmaxf(m0, acc[m][r] * sgn2);
                mx[r] = row16_max(m0);   // over the 16 lanes holding this token's features
            }
            floatx4 ex[NT];   // this sign's numerators, each exponential once
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float s0 = 0.f;
#pragma unroll
                for (int m = 0; m < NT; ++m) {
                    ex[m][r] = fast_exp2(acc[m][r] * sgn2 - mx[r]);
                    s0 += ex[m][r];
                }
                const bool ok = t0 + r < nv;
                is[r] = ok ? 1.0f / row16_sum(s0) : 0.f;
            }
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                const int f = half * F + 16 * m + li;
                const float e0 = ex[m][0] * is[0], e1 = ex[m][1] * is[1], e2 = ex[m][2] * is[2], e3 = ex[m][3] * is[3];
                uint32_t hw[2], lw[2];
                split_pk_bf16(e0, e1, hw[0], lw[0]);
                split_pk_bf16(e2, e3, hw[1], lw[1]);
                *reinterpret_cast<uint2 *>(Khi + f * G::KT + t0) = make_uint2(hw[0], hw[1]);
                *reinterpret_cast<uint2 *>(Klo + f * G::KT + t0) = make_uint2(lw[0], lw[1]);
                float zt = (e0 + e1) + (e2 + e3);   // this lane's four tokens
                zt = xrow_sum(zt);
                if (lg == 0) zk[grp * 2 * F + f] = zt;
            }
        }
    }
    __syncthreads();

    // 4. the stream: this half's step contraction, then S + phi(K)^T V
    //    stored in place
    floatx4 accS[2][EPL];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < EPL; ++e) accS[t][e] = floatx4{0.f, 0.f, 0.f, 0.f};
    // N-tile e: lane l%16 supplies column c0 + e of tokens 8(l/16) ..
    bf16x8 bv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        uint32_t pk[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            pk[j] = __builtin_amdgcn_perm(vw[2 * j + 1][e >> 1], vw[2 * j][e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
        bv[e] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }
    const bool commit = nv > 0;   // nothing to fold: the state is left untouched
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int k0 = kRows + sh * F + 32 * c + 8 * lg;
        bf16x8 ah[2], al[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            ah[mt] = *reinterpret_cast<const bf16x8 *>(Ahi + (16 * mt + li) * G::KP + k0);
            al[mt] = *reinterpret_cast<const bf16x8 *>(Alo + (16 * mt + li) * G::KP + k0);
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            // column c0 + e of the chunk's rows 8 lg + t, split
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) split_pk_bf16(sreg[c][2 * j][e], sreg[c][2 * j + 1][e], hw[j], lw[j]);
            const bf16x8 bh_ = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
            const bf16x8 bl_ = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                accS[mt][e] = mfma_bf16(ah[mt], bh_, accS[mt][e]);
                accS[mt][e] = mfma_bf16(ah[mt], bl_, accS[mt][e]);
                accS[mt][e] = mfma_bf16(al[mt], bh_, accS[mt][e]);
            }
        }
        if (commit) {
            // dS tile mt, row 4(l/16) + r = chunk row 8(l/16) + 4 mt + r: the A
            // operand row of lane l%16 = 4 g + r' is state row sh F + 32c + 8g + 4mt + r'
            const int frow = sh * F + 32 * c + 8 * (li >> 2) + (li & 3);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const bf16x8 kh = *reinterpret_cast<const bf16x8 *>(Khi + (frow + 4 * mt) * G::KT + 8 * lg);
                const bf16x8 kl = *reinterpret_cast<const bf16x8 *>(Klo + (frow + 4 * mt) * G::KT + 8 * lg);
                floatx4 ds[EPL];
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    ds[e] = mfma_bf16(kh, bv[e], floatx4{0.f, 0.f, 0.f, 0.f});
                    ds[e] = mfma_bf16(kl, bv[e], ds[e]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float *o = Sg + (lofs + (32 * c + 4 * mt + r) * D);
                    if constexpr (EPL == 4) {
                        const floatx4 o4 = {sreg[c][4 * mt + r][0] + ds[0][r], sreg[c][4 * mt + r][1] + ds[1][r],
                                            sreg[c][4 * mt + r][2] + ds[2][r], sreg[c][4 * mt + r][3] + ds[3][r]};
                        __builtin_nontemporal_store(o4, reinterpret_cast<floatx4 *>(o));
                    } else {
                        const floatx2 o2 = {sreg[c][4 * mt + r][0] + ds[0][r], sreg[c][4 * mt + r][1] + ds[1][r]};
                        __builtin_nontemporal_store(o2, reinterpret_cast<floatx2 *>(o));
                    }
                }
            }
        }
    }

    // 5. the second half's partials meet the first half's in LDS (over
    //    phi(K)^T, dead after the stream); the first half's wave adds the
    //    block-softmax part, merges with one shift per query and stores:
    //    out = (sv accV + ss accS) / (sv a + ss ld)
    constexpr int RLD = CB + 4;   // partial tile row stride (floats)
    static_assert(2 * kRows * RLD * 4 <= G::kt_bytes, "partials fit the phi(K)^T area");
    float *red = reinterpret_cast<float *>(smem + G::kt_off) + (wave & 1) * kRows * RLD;
    __syncthreads();   // every wave is done with phi(K)^T
    if (sh == 1) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float *rp = red + (16 * mt + 4 * lg + r) * RLD + EPL * li;
                if constexpr (EPL == 4)
                    *reinterpret_cast<floatx4 *>(rp) = floatx4{accS[mt][0][r], accS[mt][1][r], accS[mt][2][r], accS[mt][3][r]};
                else
                    *reinterpret_cast<floatx2 *>(rp) = floatx2{accS[mt][0][r], accS[mt][1][r]};
            }
    }
    __syncthreads();
    if (sh == 0) {
        floatx4 accV[2][EPL];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(Ahi + (16 * mt + li) * G::KP + 8 * lg);
            const bf16x8 al = *reinterpret_cast<const bf16x8 *>(Alo + (16 * mt + li) * G::KP + 8 * lg);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                accV[mt][e] = mfma_bf16(ah, bv[e], floatx4{0.f, 0.f, 0.f, 0.f});
                accV[mt][e] = mfma_bf16(al, bv[e], accV[mt][e]);
            }
        }
        float *og = a.out + (int64_t)bh * L * D;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * mt + 4 * lg + r;
                const float *rp = red + i * RLD + EPL * li;
                float pv[EPL];
                if constexpr (EPL == 4) {
                    const floatx4 p4 = *reinterpret_cast<const floatx4 *>(rp);
#pragma unroll
                    for (int e = 0; e < 4; ++e) pv[e] = p4[e];
                } else {
                    const floatx2 p2 = *reinterpret_cast<const floatx2 *>(rp);
                    pv[0] = p2[0];
                    pv[1] = p2[1];
                }
                if (i < L) {
                    const float4 rv = *reinterpret_cast<const float4 *>(rowv(i));
                    const float ld = rv.x + rv.y, g2 = rv.z + lw2, as = rv.w;
                    float cc = g2;
                    if (ld > 0.f) cc = fmaxf(cc, __log2f(ld));
                    cc = fmaxf(cc, -120.f);
                    const float sv = fast_exp2(g2 - cc);
                    const float ss = ld > 0.f ? fast_exp2(-cc) : 0.f;
                    const float inv = __builtin_amdgcn_rcpf(sv * as + ss * ld);
                    float ov[EPL];
#pragma unroll
                    for (int e = 0; e < EPL; ++e) ov[e] = (sv * accV[mt][e][r] + ss * (accS[mt][e][r] + pv[e])) * inv;
                    float *o = og + (int64_t)i * D + c0;
                    if constexpr (EPL == 4)
                        __builtin_nontemporal_store(floatx4{ov[0], ov[1], ov[2], ov[3]}, reinterpret_cast<floatx4 *>(o));
                    else
                        __builtin_nontemporal_store(floatx2{ov[0], ov[1]}, reinterpret_cast<floatx2 *>(o));
                }
            }
        }
    }
    // 6. Z += sum_t phi(k_t), by the first workgroup of the pair
    if (commit && part == 0 && tid < 2 * F) __builtin_nontemporal_store(zs[tid] + zk[tid] + zk[2 * F + tid], Zg + tid);
}

hipError_t launch_step_commit(const StepCommitArgs &a, bool bf16, int d, int F, hipStream_t stream) {
    if (bf16 && d == 128) {
        // at most half a workgroup per CU: split the value columns over two
        // workgroups per pair (13.7 -> 12.8 us at B = 8, H = 16; slower at
        // B = 12 and 16, 14.4 -> 17.6 and 16.6 -> 18.6 us)
        const int64_t items = (int64_t)a.B * a.H, cus = device_cus();
        const bool split = cus > 0 && 2 * items <= cus;
        const dim3 grid((unsigned)(split ? 2 * items : items));
        if (F == 128)
            return split ? launch_kernel(step_commit_kernel_bf16<128, 128, 2>, grid, dim3(kThreads), a, stream)
                         : launch_kernel(step_commit_kernel_bf16<128, 128, 1>, grid, dim3(kThreads), a, stream);
        if (F == 64)
            return split ? launch_kernel(step_commit_kernel_bf16<128, 64, 2>, grid, dim3(kThreads), a, stream)
                         : launch_kernel(step_commit_kernel_bf16<128, 64, 1>, grid, dim3(kThreads), a, stream);
    }
    // other shapes: the step on the current state, then the commit
    const StepArgs s{a.q, a.k, a.v, a.W, a.gate, a.S, a.Z, a.slot, a.out, a.B, a.H, a.L, a.G};
    hipError_t e = launch_step(s, bf16, d, F, stream);
    if (e != hipSuccess) return e;
    const CommitArgs c{a.n_valid, a.k, a.v, a.W, a.S, a.Z, a.slot, a.B, a.H, a.L, a.G};
    return launch_commit(c, bf16, d, F, stream);
}

}  // namespace hba
