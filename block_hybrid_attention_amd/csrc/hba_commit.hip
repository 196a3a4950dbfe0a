// hba_commit.hip -- fold committed tokens into the recurrent states.
//
// "Retrofitting Linear Attention into Diffusion Language Models", section 3.1
// (state update once a block is committed):
//   S <- S + sum_t phi(k_t) v_t^T,   Z <- Z + sum_t phi(k_t).
//
// The commit is a read-modify-write of the fp32 state (2 x 128 KB at
// F = d = 128) plus a small contraction Phi^T V (K = tokens).  Four kernels:
//   * commit_kernel: fp32 inputs (described here);
//   * commit_kernel_bf16: bf16 inputs, one workgroup per state half (d = 64;
//     d = 128 for one block when the pairs fill at most half of the CUs);
//   * commit_block_kernel_bf16: bf16, d = 128, one block of at most 32
//     tokens, one workgroup per (request, head), above half of the CUs;
//   * commit_chunks_kernel_bf16: bf16, d = 128, several chunks of 32 or 64
//     tokens, pipelined.
// fp32 inputs: one workgroup (4 waves) per (request, head).
//   * The old state is loaded straight into the MFMA accumulators at entry
//     (wave w owns state rows [w 2F/4, (w+1) 2F/4)), so the contraction
//     accumulates onto it and the result is stored once: one read and one
//     write of S, both 512-byte-row coalesced.  To get that, the output column
//     held by MFMA column j of N-tile e is d/16 * j + e, so each lane owns
//     d/16 consecutive columns.
//   * Tokens are processed in chunks of 32: k goes through LDS, u = k W runs
//     on MFMA, phi(k) is formed per token row in fp32 and written over u in
//     place (same row stride), then Phi^T V runs on fp32 MFMA.
//   * Z is accumulated per feature by one thread each.
//   * No atomics: each (request, head) state has exactly one writer, so the
//     update is deterministic.
#include "hba_device.h"
#include "hba_internal.h"

namespace hba {

template <typename T, int D, int F>
struct CommitGeom {
    using P = ProjGeom<T, D, F>;
    static constexpr int PLD = 2 * F + 16;   // phi row stride (floats); u shares it
    static constexpr int k_off = 0;
    static constexpr int w_off = P::x_bytes;
    static constexpr int u_off = w_off + P::w_bytes;
    static constexpr int bytes = u_off + kRows * PLD * 4;
};

// Load NE consecutive input elements (NE = d/16) and widen to fp32.
template <typename T, int NE>
__device__ __forceinline__ void load_cols(const T *__restrict__ p, float (&o)[NE]) {
    constexpr int BYTES = NE * (int)sizeof(T);
    if constexpr (BYTES == 32) {
        const uint4 a = reinterpret_cast<const uint4 *>(p)[0];
        const uint4 b = reinterpret_cast<const uint4 *>(p)[1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = __uint_as_float(w[e]);
    } else if constexpr (BYTES == 16) {
        const uint4 a = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = __uint_as_float(w[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = bf16_bits_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
        }
    } else {  // 4 bf16 = 8 bytes
        const uint2 a = *reinterpret_cast<const uint2 *>(p);
        const uint32_t w[2] = {a.x, a.y};
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = bf16_bits_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
    }
}

template <typename T, int D, int F>
__global__ __launch_bounds__(kThreads) void commit_kernel(CommitArgs a) {
    using G = CommitGeom<T, D, F>;
    constexpr int NE = D / 16;        // N-tiles; a lane owns NE consecutive columns
    constexpr int FW = 2 * F / 4;     // state rows owned by one wave
    constexpr int MT = FW / 16;       // 16-row M-tiles per wave
    constexpr int FM = F / 64;

    __shared__ __attribute__((aligned(16))) char smem[G::bytes];
    T *ks = reinterpret_cast<T *>(smem + G::k_off);
    T *ws = reinterpret_cast<T *>(smem + G::w_off);
    float *us = reinterpret_cast<float *>(smem + G::u_off);   // u, then phi, per row

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int bh = (int)blockIdx.x;
    const int b = bh / a.H, h = bh - b * a.H;
    const int T_ = a.T;
    int nv = a.n_valid ? a.n_valid[b] : T_;
    nv = nv < 0 ? 0 : (nv > T_ ? T_ : nv);
    const int64_t slot = a.slot ? (int64_t)a.slot[b] : (int64_t)b;

    const T *kg = static_cast<const T *>(a.k) + (int64_t)(bh / a.G) * T_ * D;
    const T *vg = static_cast<const T *>(a.v) + (int64_t)(bh / a.G) * T_ * D;
    const T *Wg = static_cast<const T *>(a.W) + (int64_t)h * D * F;
    float *Sg = a.S + (slot * a.H + h) * (int64_t)(2 * F) * D;
    float *Zg = a.Z + (slot * a.H + h) * (int64_t)(2 * F);
    if (nv == 0) return;   // nothing to fold; the state is left untouched

    WChunks<T, D, F> wc;
    load_w<T, D, F>(Wg, wc);

    // old state straight into the accumulators
    const int f_base = wave * FW;
    floatx4 acc[MT][NE];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float *p = Sg + (int64_t)(f_base + 16 * mt + 4 * lg + r) * D + NE * li;
#pragma unroll
            for (int q = 0; q < NE / 4; ++q) {
                const float4 t = reinterpret_cast<const float4 *>(p)[q];
                acc[mt][4 * q + 0][r] = t.x;
                acc[mt][4 * q + 1][r] = t.y;
                acc[mt][4 * q + 2][r] = t.z;
                acc[mt][4 * q + 3][r] = t.w;
            }
        }
    }
    float zacc = tid < 2 * F ? Zg[tid] : 0.f;
    store_w<T, D, F>(wc, ws);

#pragma unroll 1
    for (int t0 = 0; t0 < nv; t0 += kRows) {
        const int nrows = nv - t0 < kRows ? nv - t0 : kRows;
        // B operand: v rows t0 + 4 kk + lg, columns NE*li .. NE*li + NE - 1
        float vop[8][NE];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int j = 4 * kk + lg;
            load_cols<T, NE>(vg + (int64_t)(t0 + (j < nrows ? j : nrows - 1)) * D + NE * li, vop[kk]);
#pragma unroll
            for (int e = 0; e < NE; ++e) vop[kk][e] = j < nrows ? vop[kk][e] : 0.f;
        }
        stage_rows<T, D, F>(kg + (int64_t)t0 * D, D, nrows, ks);
        __syncthreads();
        project_tile<T, D, F, G::PLD>(ks, ws, us);
        __syncthreads();
        // phi(k_t) per token row, written over u in place; rows past the end are 0
#pragma unroll 1
        for (int ii = 0; ii < 8; ++ii) {
            const int i = 8 * wave + ii;
            float *row = us + i * G::PLD;
            if (i < nrows) {
                float pp[FM], pn[FM];
                phi_of_row<F>(row, lane, pp, pn);
#pragma unroll
                for (int m = 0; m < FM; ++m) {
                    row[lane + 64 * m] = pp[m];
                    row[F + lane + 64 * m] = pn[m];
                }
            } else {
#pragma unroll
                for (int m = 0; m < 2 * FM; ++m) row[lane + 64 * m] = 0.f;
            }
        }
        __syncthreads();
        if (tid < 2 * F) {
            float zs = 0.f;
#pragma unroll 8
            for (int i = 0; i < kRows; ++i) zs += us[i * G::PLD + tid];
            zacc += zs;
        }
        // S += Phi^T V : A[f][t] = phi_f(k_t), B[t][col] = v_t[col]
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float av = us[(4 * kk + lg) * G::PLD + f_base + 16 * mt + li];
#pragma unroll
                for (int e = 0; e < NE; ++e) acc[mt][e] = mfma_f32(av, vop[kk][e], acc[mt][e]);
            }
        }
        __syncthreads();   // the next chunk reuses the k tile and u/phi rows
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float *p = Sg + (int64_t)(f_base + 16 * mt + 4 * lg + r) * D + NE * li;
#pragma unroll
            for (int q = 0; q < NE / 4; ++q)
                reinterpret_cast<float4 *>(p)[q] = make_float4(acc[mt][4 * q + 0][r], acc[mt][4 * q + 1][r],
                                                                acc[mt][4 * q + 2][r], acc[mt][4 * q + 3][r]);
        }
    }
    if (tid < 2 * F) Zg[tid] = zacc;
}

// ---------------------------------------------------------------------------
// bf16 inputs: two workgroups per (request, head), one per half of the state
// (rows of softmax(kW) or of softmax(-kW)), four waves each, split-bf16 MFMA.
//   * W, the k tile and v (transposed, so tokens are contiguous for the MFMA
//     B operand) are staged in LDS; the 8x8 transposes run in registers.
//   * Waves 0-1 form u = k W for 16 tokens each (a token row sits in one
//     16-lane DPP row), then this half of phi(k), written in fp32 to LDS; for
//     one-block commits that buffer reuses the LDS of W.
//   * Every wave owns F/4 state rows and adds phi(K)^T V on bf16 MFMA with phi
//     split into a bf16 high part and residual (v is exact in bf16): two
//     products per tile.  N-tile pair p gives lane l the columns 32 p + 2 l
//     and 32 p + 2 l + 1, so each state access of 16 lanes is one contiguous
//     128-byte row segment (measured against 8 consecutive columns per lane,
//     two 16-byte accesses at a 32-byte stride: 128 -> 113 us at B = 128,
//     35.0 -> 31.1 us at B = 32, bitwise the same states).
//   * phi goes to LDS transposed ([feature][token]): the producers write a
//     lane's four tokens of one feature at once, every wave reads a state
//     row's eight tokens as its MFMA operand in two 16-byte loads, and sums
//     them for Z.
template <int D, int F, bool kResidentW>
struct CommitGeomBf16 {
    using P = ProjGeom<uint16_t, D, F>;
    static constexpr int TP = kRows + 8;         // V^T row stride (bf16): tokens + pad
    // phi^T [F features][PTLD] fp32: 10 16-byte chunks per row, so that 16
    // lanes on 16 rows at one chunk each hit distinct banks
    static constexpr int PTLD = kRows + 8;
    static constexpr int k_off = 0;
    static constexpr int v_off = P::x_bytes;
    static constexpr int w_off = v_off + D * TP * 2;
    static constexpr int phi_bytes = F * PTLD * 4;
    static constexpr int phi_off = kResidentW ? w_off + P::w_bytes : w_off;
    static constexpr int wregion = kResidentW ? P::w_bytes + phi_bytes
                                              : (P::w_bytes > phi_bytes ? P::w_bytes : phi_bytes);
    static constexpr int bytes = w_off + wregion;
};

template <int D, int F, bool kResidentW>
__global__ __launch_bounds__(kThreads, 2) void commit_kernel_bf16(CommitArgs a) {
    using T = uint16_t;
    using P = ProjGeom<T, D, F>;
    using G = CommitGeomBf16<D, F, kResidentW>;
    constexpr int NE = D / 16;          // N-tiles, paired: lane owns columns 32 p + 2 l, + 1
    constexpr int FW = F / 4;           // state rows per wave (this half has F rows)
    constexpr int MT = FW / 16;         // M-tiles per wave
    constexpr int NT = F / 16;
    constexpr int WBLK = (D / 8) * (F / 8);       // 8x8 blocks of W
    constexpr int VBLK = (kRows / 8) * (D / 8);   // 8x8 blocks of a v chunk
    constexpr int KCH = kRows * D / 8;            // 16-byte chunks of a k tile
    static_assert(WBLK <= kThreads && VBLK <= kThreads && KCH % kThreads == 0, "staging split");

    __shared__ __attribute__((aligned(16))) char smem[G::bytes];
    T *ks = reinterpret_cast<T *>(smem + G::k_off);
    T *vt = reinterpret_cast<T *>(smem + G::v_off);
    T *ws = reinterpret_cast<T *>(smem + G::w_off);
    float *phs = reinterpret_cast<float *>(smem + G::phi_off);

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    // half 0: softmax(kW) rows, 1: softmax(-kW) rows.  Workgroups are dealt
    // to the 8 XCDs in turn, so in each full group of 16 the two halves of a
    // (request, head) sit 8 apart, on the same XCD: the second reads k and v
    // from that XCD's L2.  A last partial group pairs neighbours.
    int half, bh;
    {
        const int g = (int)blockIdx.x, grp = g >> 4;
        if ((grp + 1) * 8 <= a.B * a.H) {
            half = (g >> 3) & 1;
            bh = grp * 8 + (g & 7);
        } else {
            half = g & 1;
            bh = g >> 1;
        }
    }
    const int b = bh / a.H, h = bh - b * a.H;
    const int T_ = a.T;
    int nv = a.n_valid ? a.n_valid[b] : T_;
    nv = nv < 0 ? 0 : (nv > T_ ? T_ : nv);
    if (nv == 0) return;   // nothing to fold; the state is left untouched
    const int64_t slot = a.slot ? (int64_t)a.slot[b] : (int64_t)b;
    const T *kg = static_cast<const T *>(a.k) + (int64_t)(bh / a.G) * T_ * D;
    const T *vg = static_cast<const T *>(a.v) + (int64_t)(bh / a.G) * T_ * D;
    const T *Wg = static_cast<const T *>(a.W) + (int64_t)h * D * F;
    float *Sg = a.S + ((slot * a.H + h) * (int64_t)(2 * F) + (int64_t)half * F) * D;
    float *Zg = a.Z + (slot * a.H + h) * (int64_t)(2 * F) + half * F;
    const int f_base = wave * FW;

    // staging of one chunk: W blocks (when needed), v blocks and the k tile
    auto stage = [&](int t0, int nrows, bool with_w) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        u32x4 wb[8], vb[8], kb[KCH / kThreads];
        const bool do_w = with_w && tid < WBLK;
        const bool do_v = tid < VBLK;
        if (do_w) {
            const int bf = tid % (F / 8), bi = tid / (F / 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) wb[e] = *reinterpret_cast<const u32x4 *>(Wg + (int64_t)(8 * bi + e) * F + 8 * bf);
        }
        if (do_v) {
            const int bc = tid % (D / 8), bt = tid / (D / 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = 8 * bt + e;
                const u32x4 x = *reinterpret_cast<const u32x4 *>(vg + (int64_t)(t0 + (t < nrows ? t : nrows - 1)) * D + 8 * bc);
                vb[e] = t < nrows ? x : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int it = 0; it < KCH / kThreads; ++it) {
            const int c = tid + it * kThreads;
            const int kr = c / (D / 8), kc = (c % (D / 8)) * 8;
            const u32x4 x = *reinterpret_cast<const u32x4 *>(kg + (int64_t)(t0 + (kr < nrows ? kr : nrows - 1)) * D + kc);
            kb[it] = kr < nrows ? x : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int it = 0; it < KCH / kThreads; ++it) {
            const int c = tid + it * kThreads;
            const int kr = c / (D / 8), kc = (c % (D / 8)) * 8;
            *reinterpret_cast<u32x4 *>(ks + kr * P::XLD + kc) = kb[it];
        }
        // 8x8 transposes in registers: output row c of a block = its column c
        if (do_w) {
            const int bf = tid % (F / 8), bi = tid / (F / 8);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                uint32_t w[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    w[j] = __builtin_amdgcn_perm(wb[2 * j + 1][c >> 1], wb[2 * j][c >> 1], sel);
                *reinterpret_cast<uint4 *>(ws + wt_off<D>(8 * bf + c, bi)) = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
        if (do_v) {
            const int bc = tid % (D / 8), bt = tid / (D / 8);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int col = 8 * bc + c;
                // N-tile 2 (col / 32) + col % 2, lane (col % 32) / 2: lane l holds
                // columns 32 p + 2 l, + 1 of tile pair p (128-byte row segments)
                const int rho = (2 * (col >> 5) + (col & 1)) * 16 + ((col & 31) >> 1);
                const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                uint32_t w[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    w[j] = __builtin_amdgcn_perm(vb[2 * j + 1][c >> 1], vb[2 * j][c >> 1], sel);
                *reinterpret_cast<uint4 *>(vt + rho * G::TP + 8 * bt) = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    };

    // the old state goes straight into the accumulators: row
    // f_base + 16 mt + 4 lg + r of this half, columns 32 q + 2 li (+ 1) of
    // N-tiles 2q (2q + 1).
    // Multi-chunk commits load it at entry; a one-block commit right after
    // its staging barrier.
    floatx4 acc[MT][NE];
    auto load_state = [&]() {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float *p = Sg + (int64_t)(f_base + 16 * mt + 4 * lg + r) * D + 2 * li;
#pragma unroll
                for (int q = 0; q < NE / 2; ++q) {
                    const floatx2 t = __builtin_nontemporal_load(reinterpret_cast<const floatx2 *>(p + 32 * q));
                    acc[mt][2 * q + 0][r] = t[0];
                    acc[mt][2 * q + 1][r] = t[1];
                }
            }
    };
    if constexpr (kResidentW) load_state();
    // Z of rows f_base + 16 mt + l%16, kept (and stored) by lanes l < 16
    float zacc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) zacc[mt] = lg == 0 ? Zg[f_base + 16 * mt + li] : 0.f;

#pragma unroll 1
    for (int t0 = 0; t0 < nv; t0 += kRows) {
        const int nrows = nv - t0 < kRows ? nv - t0 : kRows;
        stage(t0, nrows, !kResidentW || t0 == 0);
        __syncthreads();
        // one-block commit: the state is requested once the staging loads have
        // landed, so it does not queue ahead of them, and its latency overlaps
        // the projection and phi
        if constexpr (!kResidentW) load_state();
        // waves 0-1: u = k W for tokens 16w .. 16w+15 (log2 domain), and the
        // max (or min) and sum of this half's softmax per token
        floatx4 u[NT];
        float mref[4], inv[4];
        if (wave < 2) {
            project_rows16<T, D, F>(ks, ws, 16 * wave, u);
            const float sgn = half ? -1.f : 1.f;   // phi half = softmax(sgn * u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float m0 = -INFINITY;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    u[nt][r] *= sgn * kLog2e;
                    m0 = fmaxf(m0, u[nt][r]);
                }
                mref[r] = row16_max(m0);
                float s0 = 0.f;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    u[nt][r] = fast_exp2(u[nt][r] - mref[r]);   // u becomes the numerators
                    s0 += u[nt][r];
                }
                const bool ok = (16 * wave + 4 * lg + r) < nrows;   // rows past the end: phi = 0
                inv[r] = ok ? 1.0f / row16_sum(s0) : 0.f;
            }
        }
        __syncthreads();   // k tile and W reads done (phi may reuse W's LDS)
        if (wave < 2) {
            // phi^T: a lane's four tokens of feature 16 nt + l%16 in one write
            float *pt = phs + li * G::PTLD + 16 * wave + 4 * lg;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                *reinterpret_cast<float4 *>(pt + 16 * nt * G::PTLD) =
                    make_float4(u[nt][0] * inv[0], u[nt][1] * inv[1], u[nt][2] * inv[2], u[nt][3] * inv[3]);
        }
        __syncthreads();
        // S += phi^T V on bf16 MFMA: A[f][t] = phi_f(k_t) (high + residual),
        // B[t][col] = v_t[col]; the A values also give Z's token sums
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const float *pa = phs + (f_base + 16 * mt + li) * G::PTLD + 8 * lg;
            const float4 x0 = *reinterpret_cast<const float4 *>(pa);
            const float4 x1 = *reinterpret_cast<const float4 *>(pa + 4);
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            bf16x8 ah, al;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const __bf16 hx = (__bf16)xs[t];
                ah[t] = hx;
                al[t] = (__bf16)(xs[t] - (float)hx);
            }
            zacc[mt] += xrow_sum(((xs[0] + xs[1]) + (xs[2] + xs[3])) + ((xs[4] + xs[5]) + (xs[6] + xs[7])));
#pragma unroll
            for (int nt = 0; nt < NE; ++nt) {
                const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(vt + (16 * nt + li) * G::TP + 8 * lg);
                acc[mt][nt] = mfma_bf16(ah, bv, acc[mt][nt]);
                acc[mt][nt] = mfma_bf16(al, bv, acc[mt][nt]);
            }
        }
        __syncthreads();   // the next chunk reuses every staging buffer
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float *p = Sg + (int64_t)(f_base + 16 * mt + 4 * lg + r) * D + 2 * li;
#pragma unroll
            for (int q = 0; q < NE / 2; ++q)
                __builtin_nontemporal_store(floatx2{acc[mt][2 * q + 0][r], acc[mt][2 * q + 1][r]},
                                            reinterpret_cast<floatx2 *>(p + 32 * q));
        }
    if (lg == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) __builtin_nontemporal_store(zacc[mt], Zg + f_base + 16 * mt + li);
    }
}

// ---------------------------------------------------------------------------
// bf16 inputs, d = 128, more than one 32-token chunk (prefill-sized commits):
// the chunks are pipelined.  Two workgroups per (request, head), one per
// state half, with CW producer and CW consumer waves each; a chunk is 16 CW
// tokens.
//   * The producers form phi(K) of chunk j + 1, 16 tokens each, while chunk
//     j is folded in: k rows are loaded straight into MFMA A operands two
//     chunks ahead, W^T (staged through LDS once) is held in registers for
//     the whole call, and phi goes to LDS in fp32, transposed
//     ([feature][token]).
//   * The consumers each own F/CW rows of this state half in the MFMA
//     accumulators for the whole call and add phi(K_j)^T V_j on bf16 MFMA,
//     phi split into a bf16 high part and a residual (v is exact).  They
//     also stage V^T of the next chunk (v rows requested two chunks ahead)
//     and take Z's token sums from the phi values they load as MFMA
//     operands.
//   * phi and V^T are double-buffered; one barrier per chunk.  CW = 2: 64 KB
//     of LDS, two workgroups per CU.  CW = 4: 112 KB, one eight-wave
//     workgroup per CU, for grids that give each CU at most one workgroup
//     (the four-wave form would leave each SIMD a single wave).
// Measured at B = 8, 2048 tokens: the one-chain form above spent 27% of each
// chunk waiting for its k and v rows and 36% with waves 2-3 idle while
// waves 0-1 formed phi; forming phi is the longer of the two roles, so the
// consumers take V^T and Z.
template <int F, int CW>
struct ChunkGeom {
    static constexpr int D = 128;
    static constexpr int CT = 16 * CW;              // tokens per chunk
    // row strides of 6 or 10 16-byte chunks (2 mod 4): the operand reads (16
    // rows at one chunk each) hit distinct banks
    static constexpr int TP = CT + 16;              // V^T row stride (bf16)
    static constexpr int PTLD = CT + 8;             // phi^T row stride (floats)
    static constexpr int vt = 0;                    // [buf][D][TP] bf16, rows in N-tile order
    static constexpr int vt_buf = D * TP * 2;
    static constexpr int ph = vt + 2 * vt_buf;      // phi^T [buf][F features][PTLD] fp32
    static constexpr int ph_buf = F * PTLD * 4;
    static constexpr int loop_bytes = ph + 2 * ph_buf;
    static constexpr int wt_bytes = F * (D + 8) * 2;   // W^T at entry, then the chunk buffers
    static constexpr int bytes = loop_bytes > wt_bytes ? loop_bytes : wt_bytes;
    static_assert(ph % 16 == 0 && TP >= CT + 8, "16-byte aligned buffers, room for a chunk");
    static_assert((TP / 8) % 4 == 2 && (PTLD / 4) % 4 == 2, "conflict-free row strides");
};

template <int F, int CW>
__global__ __launch_bounds__(128 * CW, CW == 2 ? 2 : 1) void commit_chunks_kernel_bf16(CommitArgs a) {
    using T = uint16_t;
    using G = ChunkGeom<F, CW>;
    constexpr int D = G::D;
    constexpr int CT = G::CT;
    constexpr int NT = F / 16;          // feature tiles of this half
    constexpr int KS = D / 32;          // K-steps of the projection
    constexpr int NE = D / 16;          // N-tiles of the state: tile nt, lane l holds column 64 (nt/4) + 4 (l%16) + nt%4
    constexpr int FW = F / CW;          // state rows per consumer wave
    constexpr int MT = FW / 16;
    constexpr int KC = CT / 32;         // K-steps of the contraction per chunk
    constexpr int NP = 64 * CW;         // threads per role
    constexpr int WBLK = (D / 8) * (F / 8);
    static_assert(MT >= 1, "at least one 16-row tile per consumer wave");

    __shared__ __attribute__((aligned(16))) char smem[G::bytes];
    T *wts = reinterpret_cast<T *>(smem);

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    // the two state halves of a (request, head) on one XCD, as in commit_kernel_bf16
    int half, bh;
    {
        const int g = (int)blockIdx.x, grp = g >> 4;
        if ((grp + 1) * 8 <= a.B * a.H) {
            half = (g >> 3) & 1;
            bh = grp * 8 + (g & 7);
        } else {
            half = g & 1;
            bh = g >> 1;
        }
    }
    const int b = bh / a.H, h = bh - b * a.H;
    const int T_ = a.T;
    int nv = a.n_valid ? a.n_valid[b] : T_;
    nv = nv < 0 ? 0 : (nv > T_ ? T_ : nv);
    if (nv == 0) return;   // nothing to fold; the state is left untouched
    const int64_t slot = a.slot ? (int64_t)a.slot[b] : (int64_t)b;
    const T *kg = static_cast<const T *>(a.k) + (int64_t)(bh / a.G) * T_ * D;
    const T *vg = static_cast<const T *>(a.v) + (int64_t)(bh / a.G) * T_ * D;
    const T *Wg = static_cast<const T *>(a.W) + (int64_t)h * D * F;
    float *Sg = a.S + ((slot * a.H + h) * (int64_t)(2 * F) + (int64_t)half * F) * D;
    float *Zg = a.Z + (slot * a.H + h) * (int64_t)(2 * F) + half * F;
    const int nch = (nv + CT - 1) / CT;
    auto vt_of = [&](int buf) { return reinterpret_cast<T *>(smem + G::vt + buf * G::vt_buf); };
    auto ph_of = [&](int buf) { return reinterpret_cast<float *>(smem + G::ph + buf * G::ph_buf); };

    // consumers: the old state straight into the accumulators, at entry
    floatx4 acc[MT][NE];
    const int f_base = (wave - CW) * FW;
    if (wave >= CW) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // four consecutive columns per lane: 256-byte row segments per 16 lanes
                const float *p = Sg + (int64_t)(f_base + 16 * mt + 4 * lg + r) * D + 4 * li;
#pragma unroll
                for (int q = 0; q < NE / 4; ++q) {
                    const floatx4 t = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(p + 64 * q));
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[mt][4 * q + e][r] = t[e];
                }
            }
    }
    // consumers: Z of rows f_base + 16 mt + l%16, kept (and stored) by lanes l < 16
    float zacc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) zacc[mt] = (wave >= CW && lg == 0) ? Zg[f_base + 16 * mt + li] : 0.f;

    if (wave < CW) {
        // W^T into LDS: producer thread tid transposes 8x8 blocks (rows 8 bi..,
        // columns 8 bf..) of W (the consumers' loads are the state's)
        for (int blk = tid; blk < WBLK; blk += NP) {
            const int bf = blk % (F / 8), bi = blk / (F / 8);
            uint4 wb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) wb[e] = *reinterpret_cast<const uint4 *>(Wg + (int64_t)(8 * bi + e) * F + 8 * bf);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                uint32_t w[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    w[j] = __builtin_amdgcn_perm(u4_word(wb[2 * j + 1], c >> 1), u4_word(wb[2 * j], c >> 1), sel);
                *reinterpret_cast<uint4 *>(wts + wt_off<D>(8 * bf + c, bi)) = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
        // ------------------------------------------------------------ producers
        // k row 16 w + l%16 of a chunk, columns 32 ks + 8 (l/16) ..: the MFMA A
        // operand of u = k W.  Two register sets: even chunks in kA, odd in kB,
        // each requested two chunks ahead of its use.
        uint4 kA[KS], kB[KS];
        auto request = [&](int j, uint4 (&kin)[KS]) __attribute__((always_inline)) {
            const int tk = j * CT + 16 * wave + li;
            const T *kr = kg + (int64_t)(tk < nv ? tk : nv - 1) * D + 8 * lg;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kin[ks] = *reinterpret_cast<const uint4 *>(kr + 32 * ks);
        };
        // requests past the last chunk read the last valid row again: every
        // request is unconditional, so the loop's waits count exactly
        request(0, kA);
        request(1, kB);
        __syncthreads();   // W^T staged
        bf16x8 wreg[KS][NT];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                wreg[ks][nt] = *reinterpret_cast<const bf16x8 *>(wts + wt_off<D>(16 * nt + li, 4 * ks + lg));
        __syncthreads();   // W^T read: its LDS becomes the chunk buffers
        // phi of chunk j into buffer j % 2, fp32 [feature][token] (a lane's
        // four tokens of one feature are one 16-byte write); tokens past the
        // chunk's valid ones get 0
        auto produce = [&](int j, const uint4 (&kin)[KS]) __attribute__((always_inline)) {
            const int nrows = nv - j * CT < CT ? nv - j * CT : CT;
            floatx4 u[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) u[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 ak = __builtin_bit_cast(bf16x8, kin[ks]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) u[nt] = mfma_bf16(ak, wreg[ks][nt], u[nt]);
            }
            // u[nt][r] = u[token 16 w + 4 lg + r][feature 16 nt + li]; this half
            // of phi is softmax(sgn u) per token (log2 domain)
            const float sgn2 = half ? -kLog2e : kLog2e;
            float mref[4], inv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float m0 = -INFINITY;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    u[nt][r] *= sgn2;
                    m0 = fmaxf(m0, u[nt][r]);
                }
                mref[r] = row16_max(m0);
                float s0 = 0.f;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    u[nt][r] = fast_exp2(u[nt][r] - mref[r]);   // u becomes the numerators
                    s0 += u[nt][r];
                }
                inv[r] = (16 * wave + 4 * lg + r) < nrows ? 1.0f / row16_sum(s0) : 0.f;
            }
            // this lane's token quad 4 (wave%2) + lg of K-step wave/2, at chunk
            // position q ^ (q/2 % 2) (see consume)
            const int q = 4 * (wave & 1) + lg;
            float *phs = ph_of(j & 1) + li * G::PTLD + 32 * (wave >> 1) + 4 * (q ^ ((q >> 1) & 1));
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                *reinterpret_cast<float4 *>(phs + 16 * nt * G::PTLD) =
                    make_float4(u[nt][0] * inv[0], u[nt][1] * inv[1], u[nt][2] * inv[2], u[nt][3] * inv[3]);
        };
        produce(0, kA);
        request(2, kA);
        // chunk j is handed over at the j-th barrier; pairs of chunks per
        // iteration keep the two register sets static
        int j = 0;
#pragma unroll 1
        for (; j + 2 < nch; j += 2) {
            __syncthreads();   // chunk j handed over; buffer (j + 1) % 2 is free
            produce(j + 1, kB);
            request(j + 3, kB);
            __syncthreads();   // chunk j + 1 handed over
            produce(j + 2, kA);
            request(j + 4, kA);
        }
        __syncthreads();       // chunk j (the last or the one before it)
        if (j + 1 < nch) {
            produce(j + 1, kB);
            __syncthreads();   // the last chunk
        }
    } else {
        // ------------------------------------------------------------ consumers
        // V^T of chunk j into buffer j % 2: consumer thread ct takes tokens
        // 4 tq .. + 3 and columns 8 cb .. + 7 (eight lanes per 128-byte row
        // segment); row rho = 16 nt + l of V^T holds the column that N-tile
        // nt gives lane l, 64 (nt/4) + 4 l + nt%4.  Two register sets, each
        // requested two chunks ahead of its staging.
        const int ct = tid - NP;
        const int tq = (ct & 7) + 8 * (ct >> 7), cb = (ct >> 3) & 15;
        uint4 vA[4], vB[4];
        auto request_v = [&](int j, uint4 (&vin)[4]) __attribute__((always_inline)) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tv = j * CT + 4 * tq + e;
                vin[e] = *reinterpret_cast<const uint4 *>(vg + (int64_t)(tv < nv ? tv : nv - 1) * D + 8 * cb);
            }
        };
        // Column 8 cb + c sits in row 64 (cb/8) + 16 (c%4) + 2 (cb%8) + c/4.
        // The 8-byte writes go out 16 lanes at a time (eight token quads of
        // two neighbouring column blocks); the two blocks' rows are 2 apart,
        // 16 banks at these row strides, so one write covers all 32 banks.
        const int rbase = 64 * (cb >> 3) + 2 * (cb & 7);
        auto stage_v = [&](int j, const uint4 (&vin)[4]) __attribute__((always_inline)) {
            const int nrows = nv - j * CT < CT ? nv - j * CT : CT;
            T *vtb = vt_of(j & 1) + 4 * tq;
            uint4 x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool ok = 4 * tq + e < nrows;   // tokens past the valid ones: v = 0
                x[e] = make_uint4(ok ? vin[e].x : 0u, ok ? vin[e].y : 0u, ok ? vin[e].z : 0u, ok ? vin[e].w : 0u);
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int rho = rbase + 16 * (c & 3) + (c >> 2);
                const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                const uint32_t w0 = __builtin_amdgcn_perm(u4_word(x[1], c >> 1), u4_word(x[0], c >> 1), sel);
                const uint32_t w1 = __builtin_amdgcn_perm(u4_word(x[3], c >> 1), u4_word(x[2], c >> 1), sel);
                *reinterpret_cast<uint2 *>(vtb + rho * G::TP) = make_uint2(w0, w1);
            }
        };
        // S += phi^T V for chunk j, K-step kk over tokens 32 kk ..: A[f][t] =
        // phi_f(k_t) (high + residual), B[t][col] = v_t[col]; the A values
        // also give Z's token sums
        auto consume = [&](int j) __attribute__((always_inline)) {
#pragma unroll
            for (int kk = 0; kk < KC; ++kk) {
                // token quads 2 lg and 2 lg + 1 of K-step kk.  Quad q of a K-step
                // sits at chunk position q ^ (q/2 % 2): with the 2-mod-4 row
                // strides both these reads (lane quads 2 quads apart) and the
                // producers' writes (1 apart) then fall on distinct banks.
                const float *phs = ph_of(j & 1) + (f_base + li) * G::PTLD + 32 * kk;
                const int p0 = 4 * ((2 * lg) ^ (lg & 1)), p1 = 4 * ((2 * lg + 1) ^ (lg & 1));
                const T *vtb = vt_of(j & 1) + 32 * kk + 8 * lg;
                bf16x8 bv[NE];
#pragma unroll
                for (int nt = 0; nt < NE; ++nt) bv[nt] = *reinterpret_cast<const bf16x8 *>(vtb + (16 * nt + li) * G::TP);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const float4 x0 = *reinterpret_cast<const float4 *>(phs + 16 * mt * G::PTLD + p0);
                    const float4 x1 = *reinterpret_cast<const float4 *>(phs + 16 * mt * G::PTLD + p1);
                    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                    bf16x8 ah, al;
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const __bf16 hx = (__bf16)xs[t];
                        ah[t] = hx;
                        al[t] = (__bf16)(xs[t] - (float)hx);
                    }
#pragma unroll
                    for (int nt = 0; nt < NE; ++nt) {
                        acc[mt][nt] = mfma_bf16(ah, bv[nt], acc[mt][nt]);
                        acc[mt][nt] = mfma_bf16(al, bv[nt], acc[mt][nt]);
                    }
                    // tokens 32 kk + 8 (l/16) .. + 7 of row f_base + 16 mt + l%16, then all 32
                    zacc[mt] += xrow_sum(((xs[0] + xs[1]) + (xs[2] + xs[3])) + ((xs[4] + xs[5]) + (xs[6] + xs[7])));
                }
            }
        };
        request_v(0, vA);
        request_v(1, vB);   // past the last chunk: the last valid row again
        __syncthreads();    // W^T staged
        __syncthreads();    // W^T read: V^T of chunk 0 may overwrite it
        stage_v(0, vA);
        request_v(2, vA);
        int j = 0;
#pragma unroll 1
        for (; j + 2 < nch; j += 2) {
            __syncthreads();   // phi and V^T of chunk j are in buffer j % 2
            stage_v(j + 1, vB);
            request_v(j + 3, vB);
            consume(j);
            __syncthreads();   // phi and V^T of chunk j + 1
            stage_v(j + 2, vA);
            request_v(j + 4, vA);
            consume(j + 1);
        }
        __syncthreads();       // chunk j (the last or the one before it)
        const bool two = j + 1 < nch;
        if (two) stage_v(j + 1, vB);
        consume(j);
        if (two) {
            __syncthreads();   // the last chunk
            consume(j + 1);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float *p = Sg + (int64_t)(f_base + 16 * mt + 4 * lg + r) * D + 4 * li;
#pragma unroll
                for (int q = 0; q < NE / 4; ++q)
                    __builtin_nontemporal_store(floatx4{acc[mt][4 * q][r], acc[mt][4 * q + 1][r], acc[mt][4 * q + 2][r],
                                                        acc[mt][4 * q + 3][r]},
                                                reinterpret_cast<floatx4 *>(p + 64 * q));
            }
        if (lg == 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) __builtin_nontemporal_store(zacc[mt], Zg + f_base + 16 * mt + li);
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 inputs, d = 128, one block (at most 32 tokens): one workgroup of four
// waves per (request, head), as the fused step + commit.  Wave w owns state
// columns 64 (w mod 2) .. +63 (four per lane) of the F rows of feature half
// w / 2 and requests that slice before the prologue: each load and store is
// a 256-byte row segment per 16 lanes (a pure read-modify-write of these
// states measured 90.6 us, against 96.7 us with 128-byte segments; this
// kernel 96.1 against 96.9 us at B = 128, H = 16).  Wave w forms phi of sign w / 2 for
// tokens 16 (w mod 2) .. +15 (u = K W, so a lane holds four consecutive
// tokens of one feature) and writes phi(K)^T to LDS as a bf16 high part and
// residual; the stream then adds dS = phi(K)^T V, whose A rows are taken in
// the order that makes dS land in the lanes and registers holding each
// chunk, and stores S + dS in place.  k and v are read once per (request,
// head), and u once per sign.
template <int F>
struct BlockGeom {
    static constexpr int D = 128;
    using P = ProjGeom<uint16_t, D, F>;
    static constexpr int KT = kRows + 8;                  // phi(K)^T row stride (bf16)
    static constexpr int k_off = 0;                       // k rows, then (after the projection) phi(K)^T
    static constexpr int w_off = P::x_bytes;              // W^T
    static constexpr int in_bytes = P::x_bytes + P::w_bytes;
    static constexpr int kt_bytes = 2 * (2 * F) * KT * 2; // hi rows [2F][KT], then lo rows
    static constexpr int r1 = in_bytes > kt_bytes ? in_bytes : kt_bytes;
    static constexpr int zk_off = r1;                     // token sums [2 token tiles][2F]
    static constexpr int bytes = zk_off + 2 * 2 * F * 4;
};

template <int F>
__global__ __launch_bounds__(kThreads, 2) void commit_block_kernel_bf16(CommitArgs a) {
    using T = uint16_t;
    using G = BlockGeom<F>;
    using P = typename G::P;
    constexpr int D = G::D;
    constexpr int NCH = F / 32;   // 32-row chunks of this wave's feature half
    // chunks requested at entry, then after the staging barrier; the rest
    // once phi(K) is formed (with the whole slice in flight through the
    // prologue, the state spilled)
    constexpr int RING = 1;
    constexpr int PRE = NCH / 2 > RING ? NCH / 2 : RING;
    constexpr int NT = F / 16;
    constexpr int KS = D / 32;

    __shared__ __attribute__((aligned(16))) char smem[G::bytes];
    T *ks = reinterpret_cast<T *>(smem + G::k_off);
    T *ws = reinterpret_cast<T *>(smem + G::w_off);
    T *Khi = reinterpret_cast<T *>(smem + G::k_off);
    T *Klo = Khi + 2 * F * G::KT;
    float *zk = reinterpret_cast<float *>(smem + G::zk_off);

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int bh = (int)blockIdx.x;
    const int b = bh / a.H, h = bh - b * a.H;
    const int T_ = a.T;
    int nv = a.n_valid ? a.n_valid[b] : T_;
    nv = nv < 0 ? 0 : (nv > T_ ? T_ : nv);
    if (nv == 0) return;   // nothing to fold; the state is left untouched
    const int64_t slot = a.slot ? (int64_t)a.slot[b] : (int64_t)b;
    const T *kg = static_cast<const T *>(a.k) + (int64_t)(bh / a.G) * T_ * D;
    const T *vg = static_cast<const T *>(a.v) + (int64_t)(bh / a.G) * T_ * D;
    const T *Wg = static_cast<const T *>(a.W) + (int64_t)h * D * F;
    float *Sg = a.S + (slot * a.H + h) * (int64_t)(2 * F) * D;
    float *Zg = a.Z + (slot * a.H + h) * (int64_t)(2 * F);

    // 1. k rows (rows past n_valid read as zero), W and the block values;
    //    then the ring head of the state
    RowChunks<T, D> kc;
    WChunks<T, D, F> wc;
    load_rows<T, D>(kg, D, nv, kc);
    load_w<T, D, F>(Wg, wc);
    const int sh = wave >> 1;                      // feature half of this wave's state rows
    const int c0 = 64 * (wave & 1) + 4 * li;       // its columns c0 .. c0 + 3
    uint2 vw[8];   // tokens 8 lg + t, columns c0 .. c0 + 3 (rows past n_valid repeat row nv - 1; their phi is 0)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int j = 8 * lg + t;
        vw[t] = *reinterpret_cast<const uint2 *>(vg + (j < nv ? j : nv - 1) * D + c0);
    }
    // chunk c holds rows sh F + 32 c + 8 lg + t (t < 8), columns c0 .. c0 + 3
    float sreg[NCH][8][4];
    // 32-bit element offsets from the (uniform) state base: 64-bit lane
    // addresses for every chunk row, formed ahead, took the registers the
    // state needs
    const int lofs = (sh * F + 8 * lg) * D + c0;
    auto load_chunk = [&](int c) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const floatx4 v4 = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(Sg + (lofs + (32 * c + t) * D)));
#pragma unroll
            for (int e = 0; e < 4; ++e) sreg[c][t][e] = v4[e];
        }
    };
#pragma unroll
    for (int c = 0; c < RING; ++c) load_chunk(c);
    store_rows<T, D, F>(kc, ks);
    store_w<T, D, F>(wc, ws);
    __syncthreads();
#pragma unroll
    for (int c = RING; c < PRE; ++c) load_chunk(c);
    __builtin_amdgcn_sched_barrier(0);

    // 2. u = K W for tokens 16 g .. +15: acc[m][r] = u[token 16 g + 4(l/16) + r][feature 16m + l%16]
    const int g = wave & 1, half = wave >> 1;
    floatx4 acc[NT];
#pragma unroll
    for (int m = 0; m < NT; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks_ = 0; ks_ < KS; ++ks_) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8 *>(ks + (16 * g + li) * P::XLD + 32 * ks_ + 8 * lg);
#pragma unroll
        for (int m = 0; m < NT; ++m) {
            const bf16x8 bw = *reinterpret_cast<const bf16x8 *>(ws + wt_off<D>(16 * m + li, 4 * ks_ + lg));
            acc[m] = mfma_bf16(ak, bw, acc[m]);
        }
        // one K-step's operands at a time: with the whole state slice in
        // flight, operands read ahead for every K-step spilled the state
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();   // k and W^T are dead: phi(K)^T takes their LDS

    // 3. this wave's sign of phi(k_t), features half F + 16m + l%16; tokens
    //    past n_valid get phi = 0
    {
        const float sgn2 = half ? -kLog2e : kLog2e;
        const int t0 = 16 * g + 4 * lg;
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
            is[r] = t0 + r < nv ? 1.0f / row16_sum(s0) : 0.f;
        }
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
            zt = xrow_sum(zt);
            if (lg == 0) zk[g * 2 * F + f] = zt;
        }
    }
    __syncthreads();

    // 4. the stream: S + phi(K)^T V, stored in place (the old Z and the
    //    rest of the state are requested first)
    const float zold = Zg[tid % (2 * F)];
#pragma unroll
    for (int c = PRE; c < NCH; ++c) load_chunk(c);
    __builtin_amdgcn_sched_barrier(0);
    // N-tile e: lane l%16 supplies column c0 + e of tokens 8(l/16) ..
    bf16x8 bv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t pk[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w0 = (e >> 1) ? vw[2 * j].y : vw[2 * j].x, w1 = (e >> 1) ? vw[2 * j + 1].y : vw[2 * j + 1].x;
            pk[j] = __builtin_amdgcn_perm(w1, w0, (e & 1) ? 0x07060302u : 0x05040100u);
        }
        bv[e] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        // dS tile mt, row 4(l/16) + r = chunk row 8(l/16) + 4 mt + r: the A
        // operand row of lane l%16 = 4 g' + r' is state row sh F + 32c + 8g' + 4mt + r'
        const int frow = sh * F + 32 * c + 8 * (li >> 2) + (li & 3);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const bf16x8 kh = *reinterpret_cast<const bf16x8 *>(Khi + (frow + 4 * mt) * G::KT + 8 * lg);
            const bf16x8 kl = *reinterpret_cast<const bf16x8 *>(Klo + (frow + 4 * mt) * G::KT + 8 * lg);
            floatx4 ds[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ds[e] = mfma_bf16(kh, bv[e], floatx4{0.f, 0.f, 0.f, 0.f});
                ds[e] = mfma_bf16(kl, bv[e], ds[e]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const floatx4 o4 = {sreg[c][4 * mt + r][0] + ds[0][r], sreg[c][4 * mt + r][1] + ds[1][r],
                                    sreg[c][4 * mt + r][2] + ds[2][r], sreg[c][4 * mt + r][3] + ds[3][r]};
                __builtin_nontemporal_store(o4, reinterpret_cast<floatx4 *>(Sg + (lofs + (32 * c + 4 * mt + r) * D)));
            }
        }
        // one chunk at a time: scheduled across chunks, the dS tiles of all
        // of them were formed ahead of the stores and spilled
        __builtin_amdgcn_sched_barrier(0);
    }
    // 5. Z += sum_t phi(k_t)
    if (tid < 2 * F) __builtin_nontemporal_store(zold + zk[tid] + zk[2 * F + tid], Zg + tid);
}

template <typename T, int D, int F>
static hipError_t launch_commit_t(const CommitArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.B * a.H));
    if constexpr (sizeof(T) == 2) {
        const dim3 grid2((unsigned)(2 * a.B * a.H));   // one workgroup per state half
        if (a.T <= kRows) {   // one block
            if constexpr (D == 128) {
                // at most half a workgroup per CU: one workgroup per state
                // half (9.1-9.2 against 11.4 us at B = 8, H = 16; slower
                // from B = 10 on, 12.5 against 11.5 us)
                const int64_t cus = device_cus();
                if (cus > 0 && 2 * (int64_t)a.B * a.H <= cus)
                    return launch_kernel(commit_kernel_bf16<D, F, false>, grid2, dim3(kThreads), a, stream);
                return launch_kernel(commit_block_kernel_bf16<F>, grid, dim3(kThreads), a, stream);
            }
            return launch_kernel(commit_kernel_bf16<D, F, false>, grid2, dim3(kThreads), a, stream);
        }
        if constexpr (D == 128) {   // several chunks: the pipelined form
            // at most one workgroup per CU: eight waves and 64-token chunks
            const int64_t cus = device_cus();
            if (cus > 0 && 2 * (int64_t)a.B * a.H <= cus)
                return launch_kernel(commit_chunks_kernel_bf16<F, 4>, grid2, dim3(128 * 4), a, stream);
            return launch_kernel(commit_chunks_kernel_bf16<F, 2>, grid2, dim3(kThreads), a, stream);
        }
        return launch_kernel(commit_kernel_bf16<D, F, true>, grid2, dim3(kThreads), a, stream);
    } else {
        return launch_kernel(commit_kernel<T, D, F>, grid, dim3(kThreads), a, stream);
    }
}

hipError_t launch_commit(const CommitArgs &a, bool bf16, int d, int F, hipStream_t stream) {
#define HBA_COMMIT_CASE(DD, FF)                                                            \
    if (d == DD && F == FF)                                                                \
        return bf16 ? launch_commit_t<uint16_t, DD, FF>(a, stream)                         \
                    : launch_commit_t<float, DD, FF>(a, stream);
    HBA_COMMIT_CASE(64, 64)
    HBA_COMMIT_CASE(64, 128)
    HBA_COMMIT_CASE(128, 64)
    HBA_COMMIT_CASE(128, 128)
#undef HBA_COMMIT_CASE
    return hipErrorInvalidValue;
}

}  // namespace hba
