// hba_transfer_bf16.hip -- stage-1 attention transfer, bf16 inputs.
//
// Same quantities as the fp32 path in hba_transfer.hip ("Retrofitting Linear
// Attention into Diffusion Language Models", section 3.2, over the layer of
// section 3.1): per (request, head) one workgroup of eight waves sweeps the
// blocks of the sequence and keeps the state in registers.  What differs:
//   - phi(q) and phi(k) are computed inside the sweep, per block, on bf16
//     MFMA (products of bf16 values are exact in fp32) from W^T staged once;
//     nothing reads phi from memory.
//   - Every product with an fp32 operand runs on v_mfma_f32_16x16x32_bf16
//     with that operand split into a bf16 high part and a bf16 residual
//     (x = hi + lo + O(2^-17 |x|)): hi*hi + hi*lo + lo*hi for two fp32
//     operands, hi*b + lo*b when the other operand is an exact bf16 input.
//     Accumulation is fp32.
//   - The next block's q, k, v rows and teacher outputs are requested while
//     the current block computes, so their latency is covered.
//
// Operand layouts of the 16x16x32 MFMA: lane l supplies A[l%16][8(l/16) + e]
// and B[8(l/16) + e][l%16], e = 0..7; the result lands as D[4(l/16) + r][l%16].
// The contraction index may be permuted freely as long as A and B agree.  A
// state held in result layout (rows 16t + 4(l/16) + r of tile t) serves as a
// B operand over pairs of tiles (2m, 2m+1) with the permutation
//   slot e of lane group g  <->  row 32m + 16(e/4) + 4g + e%4,
// and the phi(q) rows are stored in LDS in that order, so the matching A
// operand is one 16-byte read.
#include "hba_device.h"
#include "hba_internal.h"
#include "hba_transfer.h"

namespace hba {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int F>
struct XbGeom {
    static constexpr int D = kXferD, P2 = 2 * F, NFT = F / 16, NPT = P2 / 16;
    static constexpr int XLD = ProjGeom<uint16_t, kXferD, F>::XLD;   // bf16 row tiles [32][XLD]
    static constexpr int WLD = ProjGeom<uint16_t, kXferD, F>::WLD;   // W^T [F][WLD]
    // bf16 tiles with the token index contiguous, [column][TLD]: 80-byte
    // rows (16-byte aligned operand reads).  The 96-byte stride that avoids
    // LDS bank conflicts on these reads measured no faster.
    static constexpr int TLD = kRows + 8;
    static constexpr int PQLD = P2 + 8;   // phi(q) rows [32][PQLD], permuted per 32 features
    // byte offsets
    static constexpr int xq = 0, xk = xq + kRows * XLD * 2, vT = xk + kRows * XLD * 2, wt = vT + D * TLD * 2,
                         pqh = wt + F * WLD * 2, pql = pqh + kRows * PQLD * 2, pkh = pql + kRows * PQLD * 2,
                         pkl = pkh + P2 * TLD * 2, pph = pkl + P2 * TLD * 2, ppl = pph + kRows * TLD * 2,
                         z = ppl + kRows * TLD * 2, zp = z + P2 * 4, rs = zp + 8 * P2 * 4,
                         rowp = rs + kRows * 4 * 4, red = rowp + 8 * kRows * 2 * 4, total = red + 16 * 4;
    static_assert(xk % 16 == 0 && vT % 16 == 0 && wt % 16 == 0 && pqh % 16 == 0 && pql % 16 == 0 &&
                      pkh % 16 == 0 && pkl % 16 == 0 && pph % 16 == 0 && ppl % 16 == 0 && z % 16 == 0 &&
                      zp % 16 == 0 && rs % 16 == 0,
                  "LDS tiles must stay 16-byte aligned");
    static_assert(total <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_bit_cast(bf16x8, u32x4{a, b, c, d});
}
__device__ __forceinline__ bf16x8 lds_bf16x8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// Four fp32 values -> bf16 high parts and residuals, written as 8 bytes each.
__device__ __forceinline__ void store_split4(uint16_t *hi, uint16_t *lo, float v0, float v1, float v2, float v3) {
    uint32_t h0, l0, h1, l1;
    split_pk_bf16(v0, v1, h0, l0);
    split_pk_bf16(v2, v3, h1, l1);
    *reinterpret_cast<uint2 *>(hi) = make_uint2(h0, h1);
    *reinterpret_cast<uint2 *>(lo) = make_uint2(l0, l1);
}

// The B operand of a contraction over 32 state rows: tiles 2m and 2m+1 of a
// state held in result layout, split into high parts and residuals.
__device__ __forceinline__ void split_state_pair(const floatx4 &s0, const floatx4 &s1, bf16x8 &hi, bf16x8 &lo) {
    uint32_t h[4], l[4];
    split_pk_bf16(s0[0], s0[1], h[0], l[0]);
    split_pk_bf16(s0[2], s0[3], h[1], l[1]);
    split_pk_bf16(s1[0], s1[1], h[2], l[2]);
    split_pk_bf16(s1[2], s1[3], h[3], l[3]);
    hi = as_bf16x8(h[0], h[1], h[2], h[3]);
    lo = as_bf16x8(l[0], l[1], l[2], l[3]);
}

// One 16-byte chunk (8 bf16) of a 32-row tile per thread: row tid/16,
// columns 8 (tid % 16) ..  Rows >= nrows repeat row nrows - 1 (the row is
// clamped, no branch); they are zeroed where the chunk is staged, one block
// later.  Zeroing here would place the selects, and with them the wait for
// the load, right after the load, and the next block's loads would no
// longer overlap the current block.
__device__ __forceinline__ uint4 load_chunk(const uint16_t *__restrict__ rows, int nrows, int tid) {
    const int row = tid >> 4, c0 = (tid & 15) * 8;
    const int rr = row < nrows ? row : nrows - 1;
    return *reinterpret_cast<const uint4 *>(rows + (rr * kXferD + c0));
}

// The same chunk of v for the transposed tile vT[column][token]: row tid % 32,
// columns 8 (tid / 32) ..  Each wave then covers all 32 rows of two column
// chunks (its 2-byte writes into vT measured free of bank conflicts).
__device__ __forceinline__ uint4 load_chunk_t(const uint16_t *__restrict__ rows, int nrows, int tid) {
    const int row = tid & 31, c0 = (tid >> 5) * 8;
    const int rr = row < nrows ? row : nrows - 1;
    return *reinterpret_cast<const uint4 *>(rows + (rr * kXferD + c0));
}

__device__ __forceinline__ uint4 zero_unless(const uint4 &v, bool ok) {
    return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}
__device__ __forceinline__ float4 zero_unless(const float4 &v, bool ok) {
    return ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
}

// 1. Forward sweep, bf16 inputs.  Per block, after the staging barrier, each
// wave takes one sign of phi for one 16-row tile (the projection u of that
// tile is formed by both waves of the pair):
//   waves 0-3  phi(q) of query tile w/2, sign w%2, its share of phi(q) . Z,
//              phi(q) to LDS; waves 1 and 3 also the scores of their query
//              tile against all keys, row max and sum, P to LDS;
//   waves 4-7  phi(k) of key tile (w-4)/2, sign w%2, phi(k)^T to LDS, its
//              partial column sums for Z.
// Then every wave, for its 16 value columns: P V and phi(q) S, the output,
// loss, dnum; after a barrier the commit S += phi(k)^T V, while wave 7 forms
// each row's dden and share of dL/dw.  S [2F][d] lives in registers in
// result layout: S[pt][r] = S[16 pt + 4(l/16) + r][16 w + l%16].
template <int F>
__global__ __launch_bounds__(kXferThreads, 1) void transfer_forward_bf16_kernel(TransferArgs a) {
    using G = XbGeom<F>;
    constexpr int D = kXferD, P2 = G::P2, NFT = G::NFT, NPT = G::NPT;
    constexpr int XLD = G::XLD, TLD = G::TLD, PQLD = G::PQLD;
    __shared__ __attribute__((aligned(16))) unsigned char smem[G::total];
    uint16_t *xq = reinterpret_cast<uint16_t *>(smem + G::xq), *xk = reinterpret_cast<uint16_t *>(smem + G::xk),
             *vT = reinterpret_cast<uint16_t *>(smem + G::vT), *wt = reinterpret_cast<uint16_t *>(smem + G::wt),
             *pqh = reinterpret_cast<uint16_t *>(smem + G::pqh), *pql = reinterpret_cast<uint16_t *>(smem + G::pql),
             *pkh = reinterpret_cast<uint16_t *>(smem + G::pkh), *pkl = reinterpret_cast<uint16_t *>(smem + G::pkl),
             *pph = reinterpret_cast<uint16_t *>(smem + G::pph), *ppl = reinterpret_cast<uint16_t *>(smem + G::ppl);
    float *Zs = reinterpret_cast<float *>(smem + G::z), *zp = reinterpret_cast<float *>(smem + G::zp),
          *rs = reinterpret_cast<float *>(smem + G::rs), *rowp = reinterpret_cast<float *>(smem + G::rowp),
          *red = reinterpret_cast<float *>(smem + G::red);

    const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % a.H);
    const int L = a.L;
    const int64_t N = (int64_t)a.nb * L;
    const int64_t npad = (N + 3) & ~int64_t(3);
    const uint16_t *qg = static_cast<const uint16_t *>(a.q) + bh * N * D;
    const uint16_t *kg = static_cast<const uint16_t *>(a.k) + (bh / a.G) * N * D;
    const uint16_t *vg = static_cast<const uint16_t *>(a.v) + (bh / a.G) * N * D;
    // per-(request, head) bases (uniform); offsets inside a sequence are
    // 32-bit: a sequence holds at most 2^31 / d elements (checked on the host)
    const float *tg = a.target + bh * N * D;
    float *outg = a.out ? a.out + bh * N * D : nullptr;
    const float w = 1.f / (1.f + __expf(-a.alpha[h]));
    const float log2w = __log2f(w);
    constexpr float kScaleLog2 = 0.08838834764831845f * 1.4426950408889634f;   // log2(e) / sqrt(128)
    const XferWs ws = xfer_ws((int64_t)a.B * a.H, N, F);
    float *dng = a.ws + ws.dnum + bh * N * D;
    float *ddg = a.ws + ws.dden + bh * npad;
    const int c0 = 16 * wave;
    const int lofs = 4 * lg * D + c0 + li;   // row 4 lg, column c0 + li of a block
    {
        WChunks<uint16_t, D, F> wc;
        load_w<uint16_t, D, F>(static_cast<const uint16_t *>(a.W) + (int64_t)h * D * F, wc);
        store_w<uint16_t, D, F>(wc, wt);
    }
    if (tid < P2) Zs[tid] = 0.f;
    floatx4 S[NPT];
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) S[pt] = floatx4{0.f, 0.f, 0.f, 0.f};
    float loss = 0.f, dw = 0.f;

    // block 0's inputs; later blocks are requested one block ahead
    uint4 cq = load_chunk(qg, L, tid), ck = load_chunk(kg, L, tid), cv = load_chunk_t(vg, L, tid);
    float tv[2][4];   // teacher outputs of rows 16 rt + 4 lg + r, column c0 + li
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * rt + 4 * lg + r;
            tv[rt][r] = row < L ? tg[(16 * rt + r) * D + lofs] : 0.f;
        }

#pragma unroll 1
    for (int n = 0; n < a.nb; ++n) {
        const int t0 = n * L;
        // The thread index, passed through an empty asm so that every address
        // below is formed inside the loop: hoisted out of it, each access site
        // would hold its own address register for the whole sweep instead of
        // sharing a base with its constant offset folded into the instruction.
        int tidv = tid;
        asm volatile("" : "+v"(tidv));
        const int li = tidv & 15, lg = (tidv >> 4) & 3, srow = tidv >> 4, scol = (tidv & 15) * 8;
        const int lofs = 4 * lg * D + c0 + li;
        const bool rok = srow < L, tok = (tidv & 31) < L;   // rows of the chunks inside the block
        *reinterpret_cast<uint4 *>(xq + srow * XLD + scol) = zero_unless(cq, rok);
        *reinterpret_cast<uint4 *>(xk + srow * XLD + scol) = zero_unless(ck, rok);
        {
            const uint4 cvz = zero_unless(cv, tok);
            const uint32_t vw[4] = {cvz.x, cvz.y, cvz.z, cvz.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                vT[((tidv >> 5) * 8 + e) * TLD + (tidv & 31)] = (uint16_t)(vw[e >> 1] >> (16 * (e & 1)));
        }
        if (n + 1 < a.nb) {
            const int t1 = t0 + L;
            cq = load_chunk(qg + t1 * D, L, tid);
            ck = load_chunk(kg + t1 * D, L, tid);
            cv = load_chunk_t(vg + t1 * D, L, tid);
        }
        __syncthreads();

        if (wave < 4) {
            // phi(q), one sign per wave: queries t = 16 rt + li, the features
            // of sign `side` (u^T = W^T q^T, so this lane holds u[16 ft + 4 lg + r])
            const int rt = wave >> 1, side = wave & 1, t = 16 * rt + li;
            const float sg = side ? -1.f : 1.f;
            floatx4 x[NFT];
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) x[ft] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const bf16x8 b = lds_bf16x8(xq + t * XLD + 32 * ks + 8 * lg);
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft)
                    x[ft] = mfma_bf16(lds_bf16x8(wt + wt_off<D>(16 * ft + li, 4 * ks + lg)), b, x[ft]);
                fence();
            }
            float mx = -INFINITY;
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    x[ft][r] *= sg;
                    mx = fmaxf(mx, x[ft][r]);
                }
            mx = xrow_max(mx);
            float sum = 0.f;
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    x[ft][r] = fast_exp(x[ft][r] - mx);   // <= 1
                    sum += x[ft][r];
                }
            sum = xrow_sum(sum);
            const float inv = 1.0f / sum;
            float lpart = 0.f;   // this sign's share of phi(q) . Z
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) {
                const floatx4 z4 = *reinterpret_cast<const floatx4 *>(Zs + side * F + 16 * ft + 4 * lg);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    x[ft][r] *= inv;
                    lpart += x[ft][r] * z4[r];
                }
                // feature 16 pt + 4 lg + r sits at 32 (pt/2) + 8 lg + 4 (pt%2) + r
                const int pt = side * NFT + ft;
                const int pos = t * PQLD + 32 * (pt >> 1) + 8 * lg + 4 * (pt & 1);
                store_split4(pqh + pos, pql + pos, x[ft][0], x[ft][1], x[ft][2], x[ft][3]);
                if ((ft & 1) == 1) fence();
            }
            lpart = xrow_sum(lpart);
            if (lg == 0) rs[t * 4 + (side ? 3 : 0)] = lpart;
            if (side) {
                // scores of queries t against keys 16 jt + 4 lg + r (log2
                // units; transposed, so this lane holds one query's keys)
                floatx4 s[2];
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
                    s[jt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < D / 32; ++ks)
                        s[jt] = mfma_bf16(lds_bf16x8(xk + (16 * jt + li) * XLD + 32 * ks + 8 * lg),
                                          lds_bf16x8(xq + t * XLD + 32 * ks + 8 * lg), s[jt]);
                    fence();
                }
                float M = -INFINITY;
#pragma unroll
                for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        s[jt][r] = 16 * jt + 4 * lg + r < L ? s[jt][r] * kScaleLog2 : -INFINITY;
                        M = fmaxf(M, s[jt][r]);
                    }
                M = xrow_max(M);   // finite: key 0 is always valid
                float smd = 0.f;
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        s[jt][r] = fast_exp2(s[jt][r] - M);
                        smd += s[jt][r];
                    }
                    store_split4(pph + t * TLD + 16 * jt + 4 * lg, ppl + t * TLD + 16 * jt + 4 * lg, s[jt][0],
                                 s[jt][1], s[jt][2], s[jt][3]);
                }
                smd = xrow_sum(smd);
                if (lg == 0) {
                    rs[t * 4 + 1] = M;
                    rs[t * 4 + 2] = smd;
                }
            }
        } else {
            // phi(k), one sign per wave: keys 16 tt + 4 lg + r (u = k W, each
            // key row in one DPP row of 16 lanes); rows past the block get 0
            const int tt = (wave - 4) >> 1, side = wave & 1;
            const float sg = side ? -1.f : 1.f;
            floatx4 x[NFT];
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) x[ft] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const bf16x8 xa = lds_bf16x8(xk + (16 * tt + li) * XLD + 32 * ks + 8 * lg);
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft)
                    x[ft] = mfma_bf16(xa, lds_bf16x8(wt + wt_off<D>(16 * ft + li, 4 * ks + lg)), x[ft]);
                fence();
            }
            float inv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float mx = -INFINITY;
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft) {
                    x[ft][r] *= sg;
                    mx = fmaxf(mx, x[ft][r]);
                }
                mx = row16_max(mx);
                float sum = 0.f;
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft) {
                    x[ft][r] = fast_exp(x[ft][r] - mx);
                    sum += x[ft][r];
                }
                inv[r] = (16 * tt + 4 * lg + r < L ? 1.f : 0.f) / row16_sum(sum);
            }
            // phi(k)^T to LDS; this lane's four-key partial sums of each
            // feature go to zp[4 tt + lg][f] (summed into Z after the barrier)
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) {
#pragma unroll
                for (int r = 0; r < 4; ++r) x[ft][r] *= inv[r];
                const int f = side * F + 16 * ft + li;
                store_split4(pkh + f * TLD + 16 * tt + 4 * lg, pkl + f * TLD + 16 * tt + 4 * lg, x[ft][0], x[ft][1],
                             x[ft][2], x[ft][3]);
                zp[(4 * tt + lg) * P2 + f] = (x[ft][0] + x[ft][1]) + (x[ft][2] + x[ft][3]);
            }
        }
        __syncthreads();

        // Z of blocks 0..n-1 was read above: fold block n in
        if (tid < P2) {
            float z = 0.f;
#pragma unroll
            for (int g = 0; g < 8; ++g) z += zp[g * P2 + tid];
            Zs[tid] += z;
        }
        // block softmax numerator and linear readout for this wave's 16 columns
        const bf16x8 vb = lds_bf16x8(vT + (c0 + li) * TLD + 8 * lg);
        floatx4 smv[2], lin[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            smv[rt] = mfma_bf16(lds_bf16x8(pph + (16 * rt + li) * TLD + 8 * lg), vb, floatx4{0.f, 0.f, 0.f, 0.f});
            smv[rt] = mfma_bf16(lds_bf16x8(ppl + (16 * rt + li) * TLD + 8 * lg), vb, smv[rt]);
            lin[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int m = 0; m < NPT / 2; ++m) {
            bf16x8 sh, sl;
            split_state_pair(S[2 * m], S[2 * m + 1], sh, sl);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int pos = (16 * rt + li) * PQLD + 32 * m + 8 * lg;
                const bf16x8 ah = lds_bf16x8(pqh + pos), al = lds_bf16x8(pql + pos);
                lin[rt] = mfma_bf16(ah, sh, lin[rt]);
                lin[rt] = mfma_bf16(ah, sl, lin[rt]);
                lin[rt] = mfma_bf16(al, sh, lin[rt]);
            }
            if ((m & 1) == 1) fence();
        }
        // output, loss, dnum = g / den, and the row sums g.o and g.smv
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rt + 4 * lg + r;
                // row scalars: phi(q).Z of the two signs, block max, block sum
                const floatx4 st = *reinterpret_cast<const floatx4 *>(rs + row * 4);
                const float lden = st[0] + st[3];
                const float c2 = fmaxf(st[1] + log2w, __log2f(lden));
                const float esm = fast_exp2(st[1] + log2w - c2), elin = fast_exp2(-c2);
                const float rden = __builtin_amdgcn_rcpf(esm * st[2] + elin * lden);
                const float ov = (esm * smv[rt][r] + elin * lin[rt][r]) * rden;
                float g = 0.f;
                if (row < L) {
                    const float e = ov - tv[rt][r];
                    loss += e * e;
                    g = 2.f * e;
                    const int o = (t0 + 16 * rt + r) * D + lofs;
                    if (outg) outg[o] = ov;
                    dng[o] = g * (elin * rden);   // elin / den = 1 / true denominator
                }
                const float go = row16_sum(g * ov), gs = row16_sum(g * smv[rt][r]);
                if (li == 0) {
                    rowp[(wave * kRows + row) * 2 + 0] = go;
                    rowp[(wave * kRows + row) * 2 + 1] = gs;
                }
            }
        if (n + 1 < a.nb) {
            const int t1 = t0 + L;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * rt + 4 * lg + r;
                    tv[rt][r] = row < L ? tg[(t1 + 16 * rt + r) * D + lofs] : 0.f;
                }
        }
        __syncthreads();

        if (wave == 7 && lane < kRows) {
            // per row: g.o and g.smv over the eight waves' columns, dden and
            // the row's share of dL/dw
            const int row = lane;
            float go = 0.f, gs = 0.f;
#pragma unroll
            for (int ww = 0; ww < 8; ++ww) {
                go += rowp[(ww * kRows + row) * 2 + 0];
                gs += rowp[(ww * kRows + row) * 2 + 1];
            }
            if (row < L) {
                const floatx4 st = *reinterpret_cast<const floatx4 *>(rs + row * 4);
                const float lden = st[0] + st[3];
                const float c2 = fmaxf(st[1] + log2w, __log2f(lden));
                const float esm = fast_exp2(st[1] + log2w - c2), elin = fast_exp2(-c2);
                const float den = esm * st[2] + elin * lden;
                ddg[t0 + row] = -go * (elin / den);
                dw += (esm / w) / den * (gs - go * st[2]);
            }
        }
        // commit block n: S[f][c] += sum_t phi(k_t)[f] v_t[c]
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) {
            S[pt] = mfma_bf16(lds_bf16x8(pkh + (16 * pt + li) * TLD + 8 * lg), vb, S[pt]);
            S[pt] = mfma_bf16(lds_bf16x8(pkl + (16 * pt + li) * TLD + 8 * lg), vb, S[pt]);
            if ((pt & 3) == 3) fence();
        }
        __syncthreads();
    }
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

// Eight fp32 values of a 32-row tile per thread (rows >= nrows repeat row
// nrows - 1, zeroed where staged, as for load_chunk).  Row layout: row
// tid/16, columns 8 (tid % 16) ..; column layout (for a transposed tile):
// row tid % 32, columns 8 (tid / 32) ..
template <bool COLS>
__device__ __forceinline__ void load_chunk_f32(const float *__restrict__ rows, int nrows, int tid, float4 &lo4,
                                               float4 &hi4) {
    const int row = COLS ? (tid & 31) : (tid >> 4), c0 = COLS ? (tid >> 5) * 8 : (tid & 15) * 8;
    const int rr = row < nrows ? row : nrows - 1;
    lo4 = *reinterpret_cast<const float4 *>(rows + (rr * kXferD + c0));
    hi4 = *reinterpret_cast<const float4 *>(rows + (rr * kXferD + c0 + 4));
}

// Position of column c (a multiple of 4) of a row stored in the permuted
// order of the state contraction: column 32m + 16h + 4g + r at 32m + 8g + 4h + r.
__device__ __forceinline__ int perm_col4(int c) {
    return (c & ~31) + 8 * ((c >> 2) & 3) + 4 * ((c >> 4) & 1);
}

template <int F, bool KEYS>
struct XsGeom {
    static constexpr int D = kXferD, P2 = 2 * F, NPT = P2 / 16, FW = NPT / 8;
    static constexpr int XLD = ProjGeom<uint16_t, kXferD, F>::XLD, WLD = ProjGeom<uint16_t, kXferD, F>::WLD;
    static constexpr int TLD = kRows + 8, CLD = D + 8, PXLD = P2 + 4;
    static constexpr int UROWS = D + 16;   // U^T rows: d value columns, then the Z / Gz row and 15 zero rows
    static constexpr int wt = 0, xs = wt + F * WLD * 2, ys = xs + kRows * XLD * 2, xT = ys + kRows * XLD * 2,
                         uh = xT + D * TLD * 2, ul = uh + UROWS * TLD * 2,
                         yh = ul + (KEYS ? UROWS * TLD * 2 : 0), yl = yh + P2 * TLD * 2, px = yl + P2 * TLD * 2,
                         dd = px + kRows * PXLD * 4, red = dd + kRows * 4, total = red + 8 * kRows * 4;
    // the contraction operand C (dnum split, or v) is staged over the x / y
    // row tiles once the projections have read them
    static constexpr int cph = xs, cpl = ys;
    static_assert(kRows * CLD * 2 <= kRows * XLD * 2, "C rows must fit a row tile");
    static_assert(xs % 16 == 0 && ys % 16 == 0 && xT % 16 == 0 && uh % 16 == 0 && ul % 16 == 0 && yh % 16 == 0 &&
                      yl % 16 == 0 && px % 16 == 0 && dd % 16 == 0 && red % 16 == 0,
                  "LDS tiles must stay 16-byte aligned");
    static_assert(total <= 160 * 1024, "LDS budget");
};

// 2./3. Gradient sweeps, bf16 inputs.  KEYS = false: x = q, blocks in order,
//   state S (phi(k)^T v, with Z as an extra value column), y = k, U = v,
//   dphi(q) = dnum S^T + dden Z.
// KEYS = true: x = k, blocks in reverse, state G (phi(q)^T dnum, with Gz as
//   an extra column fed by dden), y = q, U = dnum,
//   dphi(k) = v G^T + Gz for the block's keys.
// The state X^T [d + 16][2F] lives in registers split by feature: wave w
// holds features fw0 .. fw0 + 16 FW - 1 (fw0 = 16 FW w) for every value
// column, X[a][b][r] = X^T[16 a + 4(l/16) + r][fw0 + 16 b + l%16]; in that
// layout it is directly the B operand of the contraction over value columns.
// Per block, with a barrier after each step:
//   A  stage x and y rows, x^T, U^T (and dden);
//   B  waves 0-3 phi(x) (one 16-row tile and one sign each, fp32 rows to LDS),
//      waves 4-7 phi(y) (phi(y)^T split to LDS, rows past the block zero);
//   C  stage C over the row tiles, permuted for the state contraction;
//   D  dphi = C X^T (+ the Z / Gz term), then fold the block into X, and each
//      row's p . dphi over the wave's features;
//   E  du = +-p (dphi - p . dphi over the sign's features) into LDS (du^T,
//      over phi(y)^T);
//   F  dW^T += du^T x for the wave's dW tiles (both signs of each feature).
template <int F, bool KEYS>
__global__ __launch_bounds__(kXferThreads, 1) void transfer_sweep_bf16_kernel(TransferArgs a) {
    using G = XsGeom<F, KEYS>;
    constexpr int D = kXferD, P2 = G::P2, NFT = F / 16, FW = G::FW, NA = D / 16 + 1;
    constexpr int XLD = G::XLD, TLD = G::TLD, CLD = G::CLD, PXLD = G::PXLD;
    constexpr int NWT = F == 128 ? 8 : 4;   // dW tiles per wave
    __shared__ __attribute__((aligned(16))) unsigned char smem[G::total];
    uint16_t *wt = reinterpret_cast<uint16_t *>(smem + G::wt), *xs = reinterpret_cast<uint16_t *>(smem + G::xs),
             *ys = reinterpret_cast<uint16_t *>(smem + G::ys), *xT = reinterpret_cast<uint16_t *>(smem + G::xT),
             *uh = reinterpret_cast<uint16_t *>(smem + G::uh), *ul = reinterpret_cast<uint16_t *>(smem + G::ul),
             *yh = reinterpret_cast<uint16_t *>(smem + G::yh), *yl = reinterpret_cast<uint16_t *>(smem + G::yl),
             *cph = reinterpret_cast<uint16_t *>(smem + G::cph), *cpl = reinterpret_cast<uint16_t *>(smem + G::cpl);
    float *px = reinterpret_cast<float *>(smem + G::px), *dd = reinterpret_cast<float *>(smem + G::dd),
          *red = reinterpret_cast<float *>(smem + G::red);

    const int tid = (int)threadIdx.x, wave = tid >> 6;
    const int64_t bh = blockIdx.x;
    const int h = (int)(bh % a.H);
    const int L = a.L;
    const int64_t N = (int64_t)a.nb * L;
    const int64_t npad = (N + 3) & ~int64_t(3);
    const uint16_t *qg = static_cast<const uint16_t *>(a.q) + bh * N * D;
    const uint16_t *kg = static_cast<const uint16_t *>(a.k) + (bh / a.G) * N * D;
    const uint16_t *vg = static_cast<const uint16_t *>(a.v) + (bh / a.G) * N * D;
    const uint16_t *xg = KEYS ? kg : qg;   // the side whose gradient this sweep takes
    const uint16_t *yg = KEYS ? qg : kg;   // the side folded into the state
    const XferWs ws = xfer_ws((int64_t)a.B * a.H, N, F);
    const float *dng = a.ws + ws.dnum + bh * N * D;
    const float *ddg = a.ws + ws.dden + bh * npad;
    const int fw0 = 16 * FW * wave;
    const int wft = F == 128 ? wave : (wave & 3);           // dW feature tile
    const int wkd0 = F == 128 ? 0 : 4 * (wave >> 2);        // first dW value tile

    {
        WChunks<uint16_t, D, F> wc;
        load_w<uint16_t, D, F>(static_cast<const uint16_t *>(a.W) + (int64_t)h * D * F, wc);
        store_w<uint16_t, D, F>(wc, wt);
    }
    // U^T rows d .. d+15: row d is 1 for the block's tokens (queries: Z
    // counts phi(k)) or dden (keys: written per block); the rest stay 0
    for (int e = tid; e < 16 * TLD; e += kXferThreads) {
        const int row = e / TLD, col = e % TLD;
        uh[(D + row) * TLD + col] = (!KEYS && row == 0 && col < L) ? (uint16_t)0x3F80 : (uint16_t)0;
        if (KEYS) ul[(D + row) * TLD + col] = 0;
    }
    floatx4 X[NA][FW];
#pragma unroll
    for (int c = 0; c < NA; ++c)
#pragma unroll
        for (int b = 0; b < FW; ++b) X[c][b] = floatx4{0.f, 0.f, 0.f, 0.f};
    floatx4 dWa[NWT];
#pragma unroll
    for (int m = 0; m < NWT; ++m) dWa[m] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto block_row = [&](int it) { return (KEYS ? a.nb - 1 - it : it) * L; };
    uint4 cx, cy, cxt, cv;
    float4 cd0, cd1;
    float cdd = 0.f;
    auto request = [&](int it) {
        const int t0 = block_row(it);
        cx = load_chunk(xg + t0 * D, L, tid);
        cy = load_chunk(yg + t0 * D, L, tid);
        cxt = load_chunk_t(xg + t0 * D, L, tid);
        cv = KEYS ? load_chunk(vg + t0 * D, L, tid) : load_chunk_t(vg + t0 * D, L, tid);
        load_chunk_f32<KEYS>(dng + t0 * D, L, tid, cd0, cd1);
        if (tid < kRows) cdd = tid < L ? ddg[t0 + tid] : 0.f;
    };
    request(0);

#pragma unroll 1
    for (int it_ = 0; it_ < a.nb; ++it_) {
        // the thread index through an empty asm: addresses are formed inside
        // the loop, sharing bases with their constant offsets folded
        int tidv = tid;
        asm volatile("" : "+v"(tidv));
        const int li = tidv & 15, lg = (tidv >> 4) & 3;
        const int srow = tidv >> 4, scol = (tidv & 15) * 8;     // row-layout chunk
        const int trow = tidv & 31, tcol = (tidv >> 5) * 8;     // column-layout chunk

        // A. stage (rows past the block become zero here)
        const bool rok = srow < L, tok = trow < L;
        *reinterpret_cast<uint4 *>(xs + srow * XLD + scol) = zero_unless(cx, rok);
        *reinterpret_cast<uint4 *>(ys + srow * XLD + scol) = zero_unless(cy, rok);
        {
            const uint4 cxz = zero_unless(cxt, tok);
            const uint32_t w4[4] = {cxz.x, cxz.y, cxz.z, cxz.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) xT[(tcol + e) * TLD + trow] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
        }
        if constexpr (!KEYS) {
            const uint4 cvz = zero_unless(cv, tok);
            const uint32_t w4[4] = {cvz.x, cvz.y, cvz.z, cvz.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) uh[(tcol + e) * TLD + trow] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
            if (tidv < kRows) dd[tidv] = cdd;
        } else {
            // dnum^T split into high parts and residuals, dden as row d
            const float4 c0z = zero_unless(cd0, tok), c1z = zero_unless(cd1, tok);
            const float d8[8] = {c0z.x, c0z.y, c0z.z, c0z.w, c1z.x, c1z.y, c1z.z, c1z.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const __bf16 hi = (__bf16)d8[e];
                const __bf16 lo = (__bf16)(d8[e] - (float)hi);
                uh[(tcol + e) * TLD + trow] = __builtin_bit_cast(uint16_t, hi);
                ul[(tcol + e) * TLD + trow] = __builtin_bit_cast(uint16_t, lo);
            }
            if (tidv < kRows) {
                const __bf16 hi = (__bf16)cdd;
                const __bf16 lo = (__bf16)(cdd - (float)hi);
                uh[D * TLD + tidv] = __builtin_bit_cast(uint16_t, hi);
                ul[D * TLD + tidv] = __builtin_bit_cast(uint16_t, lo);
            }
        }
        // the contraction operand waits in registers until phase C
        const uint4 cvc = zero_unless(cv, rok);
        const float4 cdc0 = zero_unless(cd0, rok), cdc1 = zero_unless(cd1, rok);
        if (it_ + 1 < a.nb) request(it_ + 1);
        __syncthreads();

        // B. feature maps of both sides
        if (wave < 4) {
            // phi(x) rows t = 16 rt + li, one sign per wave (lane holds u[16 ft + 4 lg + r])
            const int rt = wave >> 1, side = wave & 1, t = 16 * rt + li;
            const float sg = side ? -1.f : 1.f;
            floatx4 x[NFT];
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) x[ft] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const bf16x8 b = lds_bf16x8(xs + t * XLD + 32 * ks + 8 * lg);
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft)
                    x[ft] = mfma_bf16(lds_bf16x8(wt + wt_off<D>(16 * ft + li, 4 * ks + lg)), b, x[ft]);
                fence();
            }
            float mx = -INFINITY;
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    x[ft][r] *= sg;
                    mx = fmaxf(mx, x[ft][r]);
                }
            mx = xrow_max(mx);
            float sum = 0.f;
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    x[ft][r] = fast_exp(x[ft][r] - mx);
                    sum += x[ft][r];
                }
            sum = xrow_sum(sum);
            const float inv = 1.0f / sum;
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) {
#pragma unroll
                for (int r = 0; r < 4; ++r) x[ft][r] *= inv;
                *reinterpret_cast<floatx4 *>(px + t * PXLD + side * F + 16 * ft + 4 * lg) = x[ft];
            }
        } else {
            // phi(y) rows 16 tt + 4 lg + r, one sign per wave; rows past the block get 0
            const int tt = (wave - 4) >> 1, side = wave & 1;
            const float sg = side ? -1.f : 1.f;
            floatx4 x[NFT];
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) x[ft] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const bf16x8 xa = lds_bf16x8(ys + (16 * tt + li) * XLD + 32 * ks + 8 * lg);
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft)
                    x[ft] = mfma_bf16(xa, lds_bf16x8(wt + wt_off<D>(16 * ft + li, 4 * ks + lg)), x[ft]);
                fence();
            }
            float inv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float mx = -INFINITY;
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft) {
                    x[ft][r] *= sg;
                    mx = fmaxf(mx, x[ft][r]);
                }
                mx = row16_max(mx);
                float sum = 0.f;
#pragma unroll
                for (int ft = 0; ft < NFT; ++ft) {
                    x[ft][r] = fast_exp(x[ft][r] - mx);
                    sum += x[ft][r];
                }
                inv[r] = (16 * tt + 4 * lg + r < L ? 1.f : 0.f) / row16_sum(sum);
            }
#pragma unroll
            for (int ft = 0; ft < NFT; ++ft) {
#pragma unroll
                for (int r = 0; r < 4; ++r) x[ft][r] *= inv[r];
                const int f = side * F + 16 * ft + li;
                store_split4(yh + f * TLD + 16 * tt + 4 * lg, yl + f * TLD + 16 * tt + 4 * lg, x[ft][0], x[ft][1],
                             x[ft][2], x[ft][3]);
            }
        }
        __syncthreads();

        // C. the contraction operand over the row tiles, columns permuted
        if constexpr (!KEYS) {
            const float d8[8] = {cdc0.x, cdc0.y, cdc0.z, cdc0.w, cdc1.x, cdc1.y, cdc1.z, cdc1.w};
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int pos = srow * CLD + perm_col4(scol + 4 * hh);
                store_split4(cph + pos, cpl + pos, d8[4 * hh], d8[4 * hh + 1], d8[4 * hh + 2], d8[4 * hh + 3]);
            }
        } else {
            *reinterpret_cast<uint2 *>(cph + srow * CLD + perm_col4(scol)) = make_uint2(cvc.x, cvc.y);
            *reinterpret_cast<uint2 *>(cph + srow * CLD + perm_col4(scol + 4)) = make_uint2(cvc.z, cvc.w);
        }
        __syncthreads();

        // D. dphi[i][f] = sum_c C[i][c] X^T[c][f] for this wave's features
        floatx4 dp[2][FW];
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
            for (int b = 0; b < FW; ++b) dp[i2][b] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < D / 32; ++m) {
            bf16x8 sh[FW], sl[FW];
#pragma unroll
            for (int b = 0; b < FW; ++b) split_state_pair(X[2 * m][b], X[2 * m + 1][b], sh[b], sl[b]);
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2) {
                const int pos = (16 * i2 + li) * CLD + 32 * m + 8 * lg;
                const bf16x8 ah = lds_bf16x8(cph + pos);
#pragma unroll
                for (int b = 0; b < FW; ++b) {
                    dp[i2][b] = mfma_bf16(ah, sh[b], dp[i2][b]);
                    dp[i2][b] = mfma_bf16(ah, sl[b], dp[i2][b]);
                }
                if constexpr (!KEYS) {
                    const bf16x8 al = lds_bf16x8(cpl + pos);
#pragma unroll
                    for (int b = 0; b < FW; ++b) dp[i2][b] = mfma_bf16(al, sh[b], dp[i2][b]);
                }
            }
            fence();
        }
        // + Z[f] dden_i (queries) or Gz[f] for the block's keys; Z / Gz sit in
        // the extra value column, lane l%16 of lane group 0
        float zf[FW];
#pragma unroll
        for (int b = 0; b < FW; ++b) zf[b] = __shfl(X[NA - 1][b][0], li, kWave);
        float pv[2][FW][4];   // phi(x) at (row 16 i2 + 4 lg + r, feature fw0 + 16 b + li)
        float part[2][4];
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * i2 + 4 * lg + r;
                const float s = KEYS ? (row < L ? 1.f : 0.f) : dd[row];
                float acc = 0.f;
#pragma unroll
                for (int b = 0; b < FW; ++b) {
                    dp[i2][b][r] += s * zf[b];
                    pv[i2][b][r] = px[row * PXLD + fw0 + 16 * b + li];
                    acc += pv[i2][b][r] * dp[i2][b][r];
                }
                part[i2][r] = acc;
            }
        // fold the block into the state: X^T[c][f] += sum_t U[t][c] Y[t][f]
        {
            bf16x8 bh_[FW], bl_[FW];
#pragma unroll
            for (int b = 0; b < FW; ++b) {
                bh_[b] = lds_bf16x8(yh + (fw0 + 16 * b + li) * TLD + 8 * lg);
                bl_[b] = lds_bf16x8(yl + (fw0 + 16 * b + li) * TLD + 8 * lg);
            }
#pragma unroll
            for (int c = 0; c < NA; ++c) {
                const bf16x8 uah = lds_bf16x8(uh + (16 * c + li) * TLD + 8 * lg);
#pragma unroll
                for (int b = 0; b < FW; ++b) {
                    X[c][b] = mfma_bf16(uah, bh_[b], X[c][b]);
                    X[c][b] = mfma_bf16(uah, bl_[b], X[c][b]);
                }
                if constexpr (KEYS) {
                    const bf16x8 ual = lds_bf16x8(ul + (16 * c + li) * TLD + 8 * lg);
#pragma unroll
                    for (int b = 0; b < FW; ++b) X[c][b] = mfma_bf16(ual, bh_[b], X[c][b]);
                }
                if ((c & 1) == 1) fence();
            }
        }
        // each row's p . dphi over this wave's features
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float tot = row16_sum(part[i2][r]);
                if (li == 0) red[wave * kRows + 16 * i2 + 4 * lg + r] = tot;
            }
        __syncthreads();

        // E. du = +-p (dphi - p . dphi over this sign's features), into du^T
        {
            const int w0 = wave < 4 ? 0 : 4;
            const float sgn = wave < 4 ? 1.f : -1.f;
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2) {
                floatx4 du[FW];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * i2 + 4 * lg + r;
                    const float tot = red[(w0 + 0) * kRows + row] + red[(w0 + 1) * kRows + row] +
                                      red[(w0 + 2) * kRows + row] + red[(w0 + 3) * kRows + row];
#pragma unroll
                    for (int b = 0; b < FW; ++b) du[b][r] = sgn * pv[i2][b][r] * (dp[i2][b][r] - tot);
                }
#pragma unroll
                for (int b = 0; b < FW; ++b) {
                    const int f = fw0 + 16 * b + li;
                    store_split4(yh + f * TLD + 16 * i2 + 4 * lg, yl + f * TLD + 16 * i2 + 4 * lg, du[b][0], du[b][1],
                                 du[b][2], du[b][3]);
                }
            }
        }
        __syncthreads();

        // F. dW^T[f'][kd] += sum_t (du[t][f'] + du[t][F + f']) x[t][kd]
        {
            const int f1 = (16 * wft + li) * TLD + 8 * lg, f2 = (F + 16 * wft + li) * TLD + 8 * lg;
            const bf16x8 a1h = lds_bf16x8(yh + f1), a1l = lds_bf16x8(yl + f1);
            const bf16x8 a2h = lds_bf16x8(yh + f2), a2l = lds_bf16x8(yl + f2);
#pragma unroll
            for (int m = 0; m < NWT; ++m) {
                const bf16x8 xb = lds_bf16x8(xT + (16 * (wkd0 + m) + li) * TLD + 8 * lg);
                dWa[m] = mfma_bf16(a1h, xb, dWa[m]);
                dWa[m] = mfma_bf16(a1l, xb, dWa[m]);
                dWa[m] = mfma_bf16(a2h, xb, dWa[m]);
                dWa[m] = mfma_bf16(a2l, xb, dWa[m]);
                if ((m & 3) == 3) fence();
            }
        }
        __syncthreads();
    }
    // dW parts in the workspace layout [d][F]
    const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
    float *dWg = a.ws + (KEYS ? ws.dWk : ws.dWq) + bh * D * F;
#pragma unroll
    for (int m = 0; m < NWT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) dWg[(int64_t)(16 * (wkd0 + m) + li) * F + 16 * wft + 4 * lg + r] = dWa[m][r];
}

hipError_t launch_transfer_sweeps_bf16(const TransferArgs &a, int F, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)a.B * a.H)), block(kXferThreads);
    hipError_t e = hipErrorInvalidValue;
    if (F == 128) {
        e = launch_kernel(transfer_sweep_bf16_kernel<128, false>, grid, block, a, stream);
        if (e == hipSuccess) e = launch_kernel(transfer_sweep_bf16_kernel<128, true>, grid, block, a, stream);
    } else if (F == 64) {
        e = launch_kernel(transfer_sweep_bf16_kernel<64, false>, grid, block, a, stream);
        if (e == hipSuccess) e = launch_kernel(transfer_sweep_bf16_kernel<64, true>, grid, block, a, stream);
    }
    return e;
}

hipError_t launch_transfer_forward_bf16(const TransferArgs &a, int F, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)a.B * a.H)), block(kXferThreads);
    if (F == 128) return launch_kernel(transfer_forward_bf16_kernel<128>, grid, block, a, stream);
    if (F == 64) return launch_kernel(transfer_forward_bf16_kernel<64>, grid, block, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace hba
