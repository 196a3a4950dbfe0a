// hba_prefix_softmax.hip -- full softmax attention over [prefix cache ; block].
//
// The comparator for block-hybrid attention: the exact softmax attention of
// "Retrofitting Linear Attention into Diffusion Language Models", section 2.2,
// for the active block's queries over every cached prefix token and every
// block token (all visible, scale 1/sqrt d, no gate).  Its cost grows with the
// prefix P, which is what the hybrid step's fixed-size state avoids.
//
// One workgroup (4 waves) per (request, head); the waves take interleaved
// key tiles and keep their own online-softmax state, merged in LDS at the
// end.  The accumulator layout of S^T = K Q^T gives each lane the scores of
// ONE query for a few keys, which is exactly the lane's share of P^T as an
// MFMA operand of O^T += V^T P^T, so P never leaves registers and the running
// max and sum of a query live in the lanes whose output rows they rescale.
//   fp32 inputs: 16-key tiles, both products on fp32 MFMA.
//   bf16 inputs: 32-key tiles, both products on bf16 MFMA (P split into a
//   high part and a residual, V exact), V staged transposed in LDS.
// The next tile's K and V are loaded before the current one is computed.
//
// Few (request, head) pairs (small batches) leave most compute units idle,
// so the keys can also be split: NS workgroups per pair each take a
// contiguous run of key tiles and write a normalised partial output with its
// running max and sum; prefix_combine_kernel then merges the NS partials of
// each query with the usual rescaling (the same algebra that merges waves).
#include <atomic>
#include <mutex>

#include "hba_device.h"
#include "hba_internal.h"

namespace hba {

template <typename T, int D>
struct PrefixOps {
    static constexpr bool kBf16 = sizeof(T) == 2;
    static constexpr int NCT = D / 16;                      // output column tiles
    static constexpr int KREG = kBf16 ? D / 32 : D / 4;     // K operand registers per lane
    static constexpr int VBYTES = NCT * (int)sizeof(T);     // per V row per lane
    static constexpr int VQ = VBYTES / 16 > 0 ? VBYTES / 16 : 1;
    // K operand: bf16 -> D/32 chunks of 8 bf16; fp32 -> D/4 floats
    uint4 kq[kBf16 ? D / 32 : 1];
    float kf[kBf16 ? 1 : D / 4];
    uint4 vq[4][VBYTES >= 16 ? VBYTES / 16 : 1];
    uint2 vh[4];   // used only when a V row slice is 8 bytes (bf16, d = 64)
};

template <typename T, int D>
__device__ __forceinline__ const T *key_row(const PrefixArgs &a, int64_t kvh, int P, int j) {
    // virtual concatenation [prefix cache ; block] of key/value row block kvh;
    // caller clamps j < P + L
    return j < P ? static_cast<const T *>(a.Kc) + (kvh * a.P + j) * D
                 : static_cast<const T *>(a.k) + (kvh * a.L + (j - P)) * D;
}
template <typename T, int D>
__device__ __forceinline__ const T *val_row(const PrefixArgs &a, int64_t kvh, int P, int j) {
    return j < P ? static_cast<const T *>(a.Vc) + (kvh * a.P + j) * D
                 : static_cast<const T *>(a.v) + (kvh * a.L + (j - P)) * D;
}

template <typename T, int D>
__device__ __forceinline__ void load_tile(const PrefixArgs &a, int64_t kvh, int P, int nkeys, int j0,
                                          int li, int lg, PrefixOps<T, D> &op) {
    using O = PrefixOps<T, D>;
    // K row for this lane: key j0 + li (clamped; masked later)
    int jk = j0 + li;
    jk = jk < nkeys ? jk : nkeys - 1;
    const T *kr = key_row<T, D>(a, kvh, P, jk);
    if constexpr (O::kBf16) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) op.kq[s] = *reinterpret_cast<const uint4 *>(kr + 32 * s + 8 * lg);
    } else {
#pragma unroll
        for (int s = 0; s < D / 4; ++s) op.kf[s] = kr[4 * s + lg];
    }
    // V rows for this lane: keys j0 + 4 lg + r, columns NCT*li .. NCT*li + NCT - 1
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        int jv = j0 + 4 * lg + r;
        jv = jv < nkeys ? jv : nkeys - 1;
        const T *vr = val_row<T, D>(a, kvh, P, jv) + O::NCT * li;
        if constexpr (O::VBYTES >= 16) {
#pragma unroll
            for (int q = 0; q < O::VBYTES / 16; ++q) op.vq[r][q] = reinterpret_cast<const uint4 *>(vr)[q];
        } else {
            op.vh[r] = *reinterpret_cast<const uint2 *>(vr);
        }
    }
}

template <typename T, int D>
__device__ __forceinline__ void v_row_f32(const PrefixOps<T, D> &op, int r, float (&o)[D / 16]) {
    using O = PrefixOps<T, D>;
    if constexpr (O::VBYTES >= 16) {
#pragma unroll
        for (int q = 0; q < O::VBYTES / 16; ++q) {
            const uint32_t w[4] = {op.vq[r][q].x, op.vq[r][q].y, op.vq[r][q].z, op.vq[r][q].w};
            if constexpr (O::kBf16) {
#pragma unroll
                for (int e = 0; e < 8; ++e) o[8 * q + e] = bf16_bits_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) o[4 * q + e] = __uint_as_float(w[e]);
            }
        }
    } else {
        const uint32_t w[2] = {op.vh[r].x, op.vh[r].y};
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = bf16_bits_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
    }
}

// Key-tile range [tb, te) of split sp out of ns for a pair with ntiles tiles.
__device__ __forceinline__ void split_range(int ntiles, int ns, int sp, int &tb, int &te) {
    const int per = (ntiles + ns - 1) / ns;
    tb = min(sp * per, ntiles);
    te = min(tb + per, ntiles);
}

// Epilogue shared by the comparator kernels: obuf holds each wave's output
// rows already scaled to the workgroup's common max and divided by its sum
// (row stride OLD floats); add the four waves and store.  Unsplit: the
// result is the output.  Split: it is the split's partial output, stored
// with the split's max M and sum Lt per query (both zero-weight, M = -inf,
// Lt = 0, when the split holds no keys).
template <int D, int OLD, bool SPLIT>
__device__ __forceinline__ void prefix_store(const PrefixArgs &a, int64_t bh, int sp, const float *obuf,
                                             const float (*mbuf)[kRows], const float (*lbuf)[kRows], int tid) {
    const int L = a.L;
    float *og;
    if constexpr (SPLIT) {
        const int64_t p = bh * a.NS + sp;
        og = a.part + p * L * D;
        if (tid < L) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < 4; ++w) M = fmaxf(M, mbuf[w][tid]);
            float Lt = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                Lt += lbuf[w][tid] > 0.f ? lbuf[w][tid] * __builtin_amdgcn_exp2f(mbuf[w][tid] - M) : 0.f;
            float *ml = a.part + (int64_t)a.B * a.H * a.NS * L * D + p * 2 * L;
            ml[tid] = M;
            ml[L + tid] = Lt;
        }
    } else {
        og = a.out + bh * L * D;
    }
#pragma unroll
    for (int it = 0; it < kRows * D / 4 / kThreads; ++it) {
        const int e = tid + it * kThreads;
        const int qi = e / (D / 4), c = 4 * (e % (D / 4));
        if (qi < L) {
            floatx4 v = *reinterpret_cast<const floatx4 *>(obuf + (0 * kRows + qi) * OLD + c);
#pragma unroll
            for (int w = 1; w < 4; ++w) v += *reinterpret_cast<const floatx4 *>(obuf + (w * kRows + qi) * OLD + c);
            if constexpr (SPLIT)
                *reinterpret_cast<floatx4 *>(og + (int64_t)qi * D + c) = v;
            else
                __builtin_nontemporal_store(v, reinterpret_cast<floatx4 *>(og + (int64_t)qi * D + c));
        }
    }
}

// Scale that brings one wave's rows to the workgroup's common max M and
// divides by the workgroup's sum Lt; a split with no keys has Lt = 0 and
// contributes zeros.
__device__ __forceinline__ float wave_scale(float m, float M, float Lt) {
    return Lt > 0.f ? __builtin_amdgcn_exp2f(m - M) / Lt : 0.f;
}

template <typename T, int D, bool SPLIT>
__global__ __launch_bounds__(kThreads) void prefix_kernel(PrefixArgs a) {
    using O = PrefixOps<T, D>;
    constexpr int NCT = O::NCT;
    constexpr int OLD = D + 4;   // merge buffer row stride (floats)
    constexpr float kScaleLog2 = (D == 128 ? 0.08838834764831845f : 0.125f) * 1.4426950408889634f;
    __shared__ __attribute__((aligned(16))) float obuf[4 * kRows * OLD];
    __shared__ float mbuf[4][kRows], lbuf[4][kRows];

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t bh = SPLIT ? (int64_t)blockIdx.x / a.NS : (int64_t)blockIdx.x;
    const int sp = SPLIT ? (int)((int64_t)blockIdx.x - bh * a.NS) : 0;
    const int64_t kvh = bh / a.G;
    const int b = (int)(bh / a.H);
    const int L = a.L;
    int P = a.prefix_len ? a.prefix_len[b] : a.P;
    P = P < 0 ? 0 : (P > a.P ? a.P : P);
    const int nkeys = P + L;
    const int ntiles = (nkeys + 15) / 16;
    int tb = 0, te = ntiles;
    if constexpr (SPLIT) split_range(ntiles, a.NS, sp, tb, te);

    // queries as the B operand of S^T = K Q^T: lane holds query 16 nt + li
    const T *qg = static_cast<const T *>(a.q) + bh * L * D;
    uint4 qq[2][O::kBf16 ? D / 32 : 1];
    float qf[2][O::kBf16 ? 1 : D / 4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int qi = 16 * nt + li;
        const T *qr = qg + (int64_t)(qi < L ? qi : L - 1) * D;
        if constexpr (O::kBf16) {
#pragma unroll
            for (int s = 0; s < D / 32; ++s) {
                const uint4 t = *reinterpret_cast<const uint4 *>(qr + 32 * s + 8 * lg);
                qq[nt][s] = qi < L ? t : make_uint4(0u, 0u, 0u, 0u);
            }
        } else {
#pragma unroll
            for (int s = 0; s < D / 4; ++s) qf[nt][s] = qi < L ? qr[4 * s + lg] : 0.f;
        }
    }

    floatx4 o[NCT][2];
#pragma unroll
    for (int c = 0; c < NCT; ++c) o[c][0] = o[c][1] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

    PrefixOps<T, D> cur, nxt;
    if (tb + wave < te) load_tile<T, D>(a, kvh, P, nkeys, 16 * (tb + wave), li, lg, cur);
#pragma unroll 1
    for (int tile = tb + wave; tile < te; tile += 4) {
        const int j0 = 16 * tile;
        {   // prefetch the wave's next tile (clamped to the last one)
            const int tn = tile + 4 < te ? tile + 4 : te - 1;
            load_tile<T, D>(a, kvh, P, nkeys, 16 * tn, li, lg, nxt);
        }
        floatx4 s[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            s[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
            if constexpr (O::kBf16) {
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks)
                    s[nt] = mfma_bf16(*reinterpret_cast<const bf16x8 *>(&cur.kq[ks]),
                                      *reinterpret_cast<const bf16x8 *>(&qq[nt][ks]), s[nt]);
            } else {
#pragma unroll
                for (int ks = 0; ks < D / 4; ++ks) s[nt] = mfma_f32(cur.kf[ks], qf[nt][ks], s[nt]);
            }
        }
        float p[2][4];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            float x[4];
            float tmax = -INFINITY;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[r] = (j0 + 4 * lg + r) < nkeys ? s[nt][r] * kScaleLog2 : -INFINITY;
                tmax = fmaxf(tmax, x[r]);
            }
            tmax = xrow_max(tmax);
            const float mnew = fmaxf(m[nt], tmax);   // finite: every tile has a valid key
            const float corr = __builtin_amdgcn_exp2f(m[nt] - mnew);
            float rs = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[nt][r] = __builtin_amdgcn_exp2f(x[r] - mnew);
                rs += p[nt][r];
            }
            rs = xrow_sum(rs);
            l[nt] = l[nt] * corr + rs;
            m[nt] = mnew;
#pragma unroll
            for (int c = 0; c < NCT; ++c) o[c][nt] *= corr;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float vv[NCT];
            v_row_f32<T, D>(cur, r, vv);
#pragma unroll
            for (int c = 0; c < NCT; ++c) {
                o[c][0] = mfma_f32(vv[c], p[0][r], o[c][0]);
                o[c][1] = mfma_f32(vv[c], p[1][r], o[c][1]);
            }
        }
        cur = nxt;
    }

    // merge the four waves' partial softmax states
    if (lg == 0) {
        mbuf[wave][li] = m[0];
        mbuf[wave][16 + li] = m[1];
        lbuf[wave][li] = l[0];
        lbuf[wave][16 + li] = l[1];
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int qi = 16 * nt + li;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, mbuf[w][qi]);
        float Lt = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            Lt += lbuf[w][qi] > 0.f ? lbuf[w][qi] * __builtin_amdgcn_exp2f(mbuf[w][qi] - M) : 0.f;
        const float sc = wave_scale(m[nt], M, Lt);
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                obuf[(wave * kRows + qi) * OLD + NCT * (4 * lg + r) + c] = o[c][nt][r] * sc;
    }
    __syncthreads();
    prefix_store<D, OLD, SPLIT>(a, bh, sp, obuf, mbuf, lbuf, tid);
}

// bf16 inputs: both products on bf16 MFMA.  Waves take interleaved 32-key
// tiles.  S^T = K Q^T as above (two 16-key halves), so a lane holds the
// scores of one query for keys 4g..4g+3 and 16+4g..16+4g+3 (g = lane/16).
// Those eight probabilities, in that order, are exactly the lane's B operand
// of O^T += V^T P^T on v_mfma_f32_16x16x32_bf16, split into a bf16 high part
// and a bf16 residual (V is exact in bf16), so P never leaves registers.  The
// A operand needs eight keys of one V column per lane: each wave stages its
// V tile transposed in its own LDS region (8x8 register transposes, keys in
// the same order), read back as one 16-byte load per lane and column tile.
template <int D>
struct PrefixGeomBf16 {
    static constexpr int VTLD = 4 * 8 + 8;                  // V^T row: 4 key groups x 8 keys + pad (bf16)
    static constexpr int vt_bytes = D * VTLD * 2;           // one wave's V^T tile
    static constexpr int OLD = D + 4;                       // merge row stride (floats)
    static constexpr int ob_bytes = 4 * kRows * OLD * 4;    // the four waves' partial outputs
    static constexpr int bytes = (4 * vt_bytes > ob_bytes ? 4 * vt_bytes : ob_bytes);
};

template <int D, bool SPLIT>
__global__ __launch_bounds__(kThreads, 1) void prefix_kernel_bf16(PrefixArgs a) {
    using T = uint16_t;
    using G = PrefixGeomBf16<D>;
    constexpr int KS = D / 32;     // K-steps of S^T = K Q^T
    constexpr int NCT = D / 16;    // 16-column output tiles
    constexpr float kScaleLog2 = (D == 128 ? 0.08838834764831845f : 0.125f) * 1.4426950408889634f;
    __shared__ __attribute__((aligned(16))) char smem[G::bytes];
    __shared__ float mbuf[4][kRows], lbuf[4][kRows];

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t bh = SPLIT ? (int64_t)blockIdx.x / a.NS : (int64_t)blockIdx.x;
    const int sp = SPLIT ? (int)((int64_t)blockIdx.x - bh * a.NS) : 0;
    const int64_t kvh = bh / a.G;
    const int b = (int)(bh / a.H);
    const int L = a.L;
    int P = a.prefix_len ? a.prefix_len[b] : a.P;
    P = P < 0 ? 0 : (P > a.P ? a.P : P);
    const int nkeys = P + L;
    const int ntiles = (nkeys + 31) / 32;
    int tb = 0, te = ntiles;
    if constexpr (SPLIT) split_range(ntiles, a.NS, sp, tb, te);
    const int nt_ = te - tb;   // this workgroup's tiles: tb, tb + 1, ...
    T *vt = reinterpret_cast<T *>(smem + wave * G::vt_bytes);

    // queries as the B operand of S^T = K Q^T: lane holds query 16 nt + li
    const T *qg = static_cast<const T *>(a.q) + bh * L * D;
    bf16x8 qq[2][KS];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int qi = 16 * nt + li;
        const T *qr = qg + (int64_t)(qi < L ? qi : L - 1) * D + 8 * lg;
#pragma unroll
        for (int s_ = 0; s_ < KS; ++s_) qq[nt][s_] = *reinterpret_cast<const bf16x8 *>(qr + 32 * s_);
    }

    // one tile's operands: K rows j0 + 16 h + l%16 (A of S^T), and the V block
    // of rows j0 + 4g + r, j0 + 16 + 4g + r (g = l/16, r < 4), columns 8 (l%16) ..
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    struct Tile {
        u32x4 k[2][KS];
        u32x4 v[8];
    };
    auto load = [&](int j0, Tile &t) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            int jk = j0 + 16 * hh + li;
            jk = jk < nkeys ? jk : nkeys - 1;
            const T *kr = key_row<T, D>(a, kvh, P, jk) + 8 * lg;
#pragma unroll
            for (int s_ = 0; s_ < KS; ++s_) t.k[hh][s_] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kr + 32 * s_));
        }
        if (li < D / 8) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                int jv = j0 + (e < 4 ? 4 * lg + e : 16 + 4 * lg + e - 4);
                jv = jv < nkeys ? jv : nkeys - 1;
                const T *vr = val_row<T, D>(a, kvh, P, jv) + 8 * li;
                t.v[e] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vr));
            }
        }
    };

    floatx4 o[NCT][2];
#pragma unroll
    for (int c = 0; c < NCT; ++c) o[c][0] = o[c][1] = floatx4{0.f, 0.f, 0.f, 0.f};
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};

    // one tile: V^T into the wave's LDS, scores, online softmax, O^T += V^T P^T
    auto process = [&](int tile, const Tile &t) {
        const int j0 = 32 * tile;
            // V^T of this tile into the wave's LDS: row = column, 8 keys per group
            if (li < D / 8) {
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                    uint32_t w[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        w[j] = __builtin_amdgcn_perm(t.v[2 * j + 1][c >> 1], t.v[2 * j][c >> 1], sel);
                    *reinterpret_cast<uint4 *>(vt + (8 * li + c) * G::VTLD + 8 * lg) = make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
            // scores: s[hh][nt][r] = q_(16 nt + l%16) . k_(j0 + 16 hh + 4 (l/16) + r)
            floatx4 sc[2][2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    sc[hh][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s_ = 0; s_ < KS; ++s_)
                        sc[hh][nt] = mfma_bf16(__builtin_bit_cast(bf16x8, t.k[hh][s_]), qq[nt][s_], sc[hh][nt]);
                }
            bf16x8 ph[2], pl[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                float x[8];
                float tmax = -INFINITY;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int key = j0 + (e < 4 ? 4 * lg + e : 16 + 4 * lg + e - 4);
                    x[e] = key < nkeys ? sc[e >> 2][nt][e & 3] * kScaleLog2 : -INFINITY;
                    tmax = fmaxf(tmax, x[e]);
                }
                tmax = xrow_max(tmax);
                const float mnew = fmaxf(m[nt], tmax);   // finite: every tile has a valid key
                const float corr = __builtin_amdgcn_exp2f(m[nt] - mnew);
                float rs = 0.f, pv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pv[e] = __builtin_amdgcn_exp2f(x[e] - mnew);
                    rs += pv[e];
                }
                rs = xrow_sum(rs);
                l[nt] = l[nt] * corr + rs;
                m[nt] = mnew;
#pragma unroll
                for (int c = 0; c < NCT; ++c) o[c][nt] *= corr;
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) split_pk_bf16(pv[2 * j], pv[2 * j + 1], hw[j], lw[j]);
                ph[nt] = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
                pl[nt] = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
            }
            // O^T += V^T P^T: o[c][nt][r] = O[16 nt + l%16][16 c + 4 (l/16) + r]
#pragma unroll
            for (int c = 0; c < NCT; ++c) {
                const bf16x8 va = *reinterpret_cast<const bf16x8 *>(vt + (16 * c + li) * G::VTLD + 8 * lg);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    o[c][nt] = mfma_bf16(va, ph[nt], o[c][nt]);
                    o[c][nt] = mfma_bf16(va, pl[nt], o[c][nt]);
                }
            }
    };
    // two tiles in flight per wave, ping-ponged without copies (a register
    // copy of the prefetched tile would wait for all of its loads)
    Tile t0, t1;
    if (wave < nt_) load(32 * (tb + wave), t0);
#pragma unroll 1
    for (int i = wave; i < nt_; i += 8) {
        load(32 * (tb + (i + 4 < nt_ ? i + 4 : nt_ - 1)), t1);
        process(tb + i, t0);
        if (i + 4 >= nt_) break;
        load(32 * (tb + (i + 8 < nt_ ? i + 8 : nt_ - 1)), t0);
        process(tb + i + 4, t1);
    }

    // merge the four waves' partial softmax states (the V^T tiles are dead)
    if (lg == 0) {
        mbuf[wave][li] = m[0];
        mbuf[wave][16 + li] = m[1];
        lbuf[wave][li] = l[0];
        lbuf[wave][16 + li] = l[1];
    }
    __syncthreads();
    float *obuf = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int qi = 16 * nt + li;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, mbuf[w][qi]);
        float Lt = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            Lt += lbuf[w][qi] > 0.f ? lbuf[w][qi] * __builtin_amdgcn_exp2f(mbuf[w][qi] - M) : 0.f;
        const float sc_ = wave_scale(m[nt], M, Lt);
#pragma unroll
        for (int c = 0; c < NCT; ++c)
            *reinterpret_cast<float4 *>(obuf + (wave * kRows + qi) * G::OLD + 16 * c + 4 * lg) =
                make_float4(o[c][nt][0] * sc_, o[c][nt][1] * sc_, o[c][nt][2] * sc_, o[c][nt][3] * sc_);
    }
    __syncthreads();
    prefix_store<D, G::OLD, SPLIT>(a, bh, sp, obuf, mbuf, lbuf, tid);
}

// Merge of the NS key splits of each (request, head): with split maxima
// M_s and sums Lt_s, query i's output is
//   sum_s Lt_s 2^(M_s - M) o_s / sum_s Lt_s 2^(M_s - M),   M = max_s M_s,
// where o_s is split s's normalised partial output.  Grid: (pair, slice of
// kThreads output float4s); the NS partial loads of a float4 are unrolled so
// they are in flight together.
template <int D>
__global__ __launch_bounds__(kThreads) void prefix_combine_kernel(PrefixArgs a) {
    __shared__ float wgt[kMaxPrefixSplit][kRows];
    const int tid = (int)threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int L = a.L, NS = a.NS;
    const float *po = a.part + bh * NS * L * D;
    const float *ml = a.part + (int64_t)a.B * a.H * NS * L * D + bh * NS * 2 * L;
    if (tid < L) {
        float M = -INFINITY;
        for (int s_ = 0; s_ < NS; ++s_) M = fmaxf(M, ml[s_ * 2 * L + tid]);
        float den = 0.f;
        for (int s_ = 0; s_ < NS; ++s_) {
            const float lt = ml[s_ * 2 * L + L + tid];
            const float w = lt > 0.f ? lt * __builtin_amdgcn_exp2f(ml[s_ * 2 * L + tid] - M) : 0.f;
            wgt[s_][tid] = w;
            den += w;
        }
        const float inv = 1.f / den;   // den > 0: every query sees at least its block's keys
        for (int s_ = 0; s_ < NS; ++s_) wgt[s_][tid] *= inv;
    }
    __syncthreads();
    float *og = a.out + bh * L * D;
    const int e = (int)blockIdx.y * kThreads + tid;
    if (e < L * D / 4) {
        const int qi = e / (D / 4), c = 4 * (e % (D / 4));
        floatx4 v = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int s_ = 0; s_ < NS; ++s_)
            v += wgt[s_][qi] * *reinterpret_cast<const floatx4 *>(po + ((int64_t)s_ * L + qi) * D + c);
        __builtin_nontemporal_store(v, reinterpret_cast<floatx4 *>(og + (int64_t)qi * D + c));
    }
}

template <typename T, int D>
static hipError_t launch_prefix_t(const PrefixArgs &a, hipStream_t stream) {
    const unsigned pairs = (unsigned)(a.B * a.H);
    if (a.NS <= 1) {
        if constexpr (sizeof(T) == 2)
            return launch_kernel(prefix_kernel_bf16<D, false>, dim3(pairs), dim3(kThreads), a, stream);
        else
            return launch_kernel(prefix_kernel<T, D, false>, dim3(pairs), dim3(kThreads), a, stream);
    }
    const dim3 grid((unsigned)((int64_t)pairs * a.NS));
    hipError_t e;
    if constexpr (sizeof(T) == 2)
        e = launch_kernel(prefix_kernel_bf16<D, true>, grid, dim3(kThreads), a, stream);
    else
        e = launch_kernel(prefix_kernel<T, D, true>, grid, dim3(kThreads), a, stream);
    if (e != hipSuccess) return e;
    const unsigned slices = (unsigned)((a.L * D / 4 + kThreads - 1) / kThreads);
    return launch_kernel(prefix_combine_kernel<D>, dim3(pairs, slices), dim3(kThreads), a, stream);
}

// Partials of hba_prefix_softmax_split_noalloc: a fixed array in device
// memory, one copy per device, held until the process ends.  Host code never
// passes `scratch` itself to a kernel (on the host it names a stand-in, not a
// device address); it asks static_scratch() for the device's address, taken
// once per device with hipGetSymbolAddress.
static __device__ __align__(256) float scratch[kStaticScratchBytes / sizeof(float)];

hipError_t static_scratch(float **ptr) {
    static std::atomic<float *> addr[kMaxDevices];
    static std::mutex init;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    float *p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(init);
        p = addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            void *sym = nullptr;
            e = hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!sym) return hipErrorInvalidSymbol;
            p = static_cast<float *>(sym);
            addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_prefix_softmax(const PrefixArgs &a, bool bf16, int d, hipStream_t stream) {
    if (d == 64) return bf16 ? launch_prefix_t<uint16_t, 64>(a, stream) : launch_prefix_t<float, 64>(a, stream);
    if (d == 128) return bf16 ? launch_prefix_t<uint16_t, 128>(a, stream) : launch_prefix_t<float, 128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace hba
