// hba_commit.hip -- fold committed tokens into the recurrent states.
//
// "Retrofitting Linear Attention into Diffusion Language Models", section 3.1
// (state update once a block is committed):
//   S <- S + sum_t phi(k_t) v_t^T,   Z <- Z + sum_t phi(k_t).
//
// One workgroup (4 waves) per (request, head).  The commit is a read-modify-
// write of the fp32 state (2 x 128 KB at F = d = 128) plus a small
// contraction Phi^T V (K = tokens).  Design:
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
//   * Waves 2-3 sum phi over tokens for Z in fp32, one feature per thread.
template <int D, int F, bool kResidentW>
struct CommitGeomBf16 {
    using P = ProjGeom<uint16_t, D, F>;
    static constexpr int TP = kRows + 8;         // V^T row stride (bf16): tokens + pad
    static constexpr int PHLD = F + 2;           // phi-half row stride (floats)
    static constexpr int k_off = 0;
    static constexpr int v_off = P::x_bytes;
    static constexpr int w_off = v_off + D * TP * 2;
    static constexpr int phi_bytes = kRows * PHLD * 4;
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
    const int zf = tid - 128;   // waves 2-3: one feature each for the Z sums
    float zacc = (zf >= 0 && zf < F) ? Zg[zf] : 0.f;

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
                for (int nt = 0; nt < NT; ++nt) s0 += fast_exp2(u[nt][r] - mref[r]);
                const bool ok = (16 * wave + 4 * lg + r) < nrows;   // rows past the end: phi = 0
                inv[r] = ok ? 1.0f / row16_sum(s0) : 0.f;
            }
        }
        __syncthreads();   // k tile and W reads done (phi may reuse W's LDS)
        if (wave < 2) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float *row = phs + (16 * wave + 4 * lg + r) * G::PHLD;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) row[16 * nt + li] = fast_exp2(u[nt][r] - mref[r]) * inv[r];
            }
        }
        __syncthreads();
        if (zf >= 0 && zf < F) {
            float zs = 0.f;
#pragma unroll 8
            for (int i = 0; i < kRows; ++i) zs += phs[i * G::PHLD + zf];
            zacc += zs;
        }
        // S += phi^T V on bf16 MFMA: A[f][t] = phi_f(k_t) (high + residual), B[t][col] = v_t[col]
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            bf16x8 ah, al;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float x = phs[(8 * lg + t) * G::PHLD + f_base + 16 * mt + li];
                const __bf16 hx = (__bf16)x;
                ah[t] = hx;
                al[t] = (__bf16)(x - (float)hx);
            }
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
    if (zf >= 0 && zf < F) __builtin_nontemporal_store(zacc, Zg + zf);
}

template <typename T, int D, int F>
static hipError_t launch_commit_t(const CommitArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.B * a.H));
    if constexpr (sizeof(T) == 2) {
        const dim3 grid2((unsigned)(2 * a.B * a.H));   // one workgroup per state half
        if (a.T <= kRows)   // one block: phi reuses the LDS of W
            return launch_kernel(commit_kernel_bf16<D, F, false>, grid2, dim3(kThreads), a, stream);
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
