// hba_device.h -- device-side building blocks shared by the block-hybrid
// attention kernels (gfx950 / CDNA4, wave64).
//
// Tiles are 32 rows (tokens) by d columns.  Matrix products use the gfx950
// MFMA instructions:
//   v_mfma_f32_16x16x32_bf16  for bf16 x bf16 products (exact in fp32),
//   v_mfma_f32_16x16x4_f32    for fp32 operands.
// Lane layouts (wave64, lane l):
//   16x16x32 bf16: A[i = l%16][k = 8(l/16) .. 8(l/16)+7], B[k = same][j = l%16]
//   16x16x4  f32 : A[i = l%16][k = l/16],                 B[k = l/16][j = l%16]
//   accumulator  : D[i = 4(l/16) + r][j = l%16], r = 0..3 (vector element r)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hba {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kThreads = 256;   // 4 waves per workgroup
constexpr int kRows = 32;       // rows of a token tile (the block size bound)

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_bits_to_f32(x); }

// Two floats -> two bf16 (round to nearest even) packed in one word, one
// v_cvt_pk_bf16_f32; a lands in the low half.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2){a, b}, bf16x2));
}
// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): the residual as a float
__device__ __forceinline__ float bf16_residual(float x) {
    return x - (float)(__bf16)x;
}
// Split two floats into packed bf16 high parts and packed bf16 residuals:
// x = hi + lo + O(2^-17 |x|).
__device__ __forceinline__ void split_pk_bf16(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = cvt_pk_bf16(a, b);
    const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xffff0000u);
    lo = cvt_pk_bf16(a - ha, b - hb);
}

// Exchanges across the 16-lane rows of a wave with the gfx950 permlane
// swaps (one VALU instruction each, no LDS round trip).  With both operands
// equal to v, permlane16_swap leaves lane l holding {v[l], v[l ^ 16]} and
// permlane32_swap {v[l], v[l ^ 32]}, in an order that depends on l.
__device__ __forceinline__ void pair16(float v, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float v, float &a, float &b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
// Reductions over lanes l, l ^ 16, l ^ 32, l ^ 48 (the same position in the
// four rows): first the pair l, l ^ 16, then l, l ^ 32.  Each step combines
// the same two values as a shuffle by 16 then by 32 would (operands only
// swap places), so the results are bitwise those of the shuffle form.
__device__ __forceinline__ float xrow_max(float v) {
    float a, b;
    pair16(v, a, b);
    pair32(fmaxf(a, b), a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float xrow_min(float v) {
    float a, b;
    pair16(v, a, b);
    pair32(fminf(a, b), a, b);
    return fminf(a, b);
}
__device__ __forceinline__ float xrow_sum(float v) {
    float a, b;
    pair16(v, a, b);
    pair32(a + b, a, b);
    return a + b;
}

// Reductions over the 16 lanes of a DPP row (lanes 16g .. 16g+15): rotate by
// 8 and 4 inside the row, then swap within quads; every lane of the row ends
// with the result.  Pure VALU data movement, no LDS traffic.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppRowRor8 = 0x128, kDppRowRor4 = 0x124, kDppQuadSwap2 = 0x4E, kDppQuadSwap1 = 0xB1;

__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<kDppRowRor8>(v));
    v = fmaxf(v, dpp_f<kDppRowRor4>(v));
    v = fmaxf(v, dpp_f<kDppQuadSwap2>(v));
    return fmaxf(v, dpp_f<kDppQuadSwap1>(v));
}
__device__ __forceinline__ float row16_min(float v) {
    v = fminf(v, dpp_f<kDppRowRor8>(v));
    v = fminf(v, dpp_f<kDppRowRor4>(v));
    v = fminf(v, dpp_f<kDppQuadSwap2>(v));
    return fminf(v, dpp_f<kDppQuadSwap1>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<kDppRowRor8>(v);
    v += dpp_f<kDppRowRor4>(v);
    v += dpp_f<kDppQuadSwap2>(v);
    return v + dpp_f<kDppQuadSwap1>(v);
}

// Whole-wave reductions: within each 16-lane row by DPP, then across rows.
__device__ __forceinline__ float wave_max(float v) { return xrow_max(row16_max(v)); }
__device__ __forceinline__ float wave_min(float v) { return xrow_min(row16_min(v)); }
__device__ __forceinline__ float wave_sum(float v) { return xrow_sum(row16_sum(v)); }

__device__ __forceinline__ floatx4 mfma_f32(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_bf16(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// exp(x) through the hardware base-2 exponential.
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// LDS geometry of the projection stage, per input element type.
//   X tile : [32][XLD] rows of x (q, k or x), bf16 or fp32
//   W      : bf16 -> transposed Wt[F][XLD] (row f holds column f of W),
//            fp32 -> as given, W[D][F + 16]
//   u      : [32][F + 4] fp32, u = X W
// Row paddings keep the MFMA operand reads free of LDS bank conflicts.
template <typename T, int D, int F>
struct ProjGeom {
    static constexpr bool kBf16 = sizeof(T) == 2;
    static constexpr int XLD = kBf16 ? D + 8 : D + 4;            // elements
    static constexpr int WROWS = kBf16 ? F : D;
    static constexpr int WLD = kBf16 ? D + 8 : F + 16;           // elements
    static constexpr int ULD = F + 4;                            // floats
    static constexpr int x_bytes = kRows * XLD * (int)sizeof(T);
    static constexpr int w_bytes = WROWS * WLD * (int)sizeof(T);
    static constexpr int u_bytes = kRows * ULD * 4;
};

// Copy `nrows` (1..32) rows of D elements, global row stride `gstride`
// elements, into an LDS tile [32][XLD]; rows >= nrows are zero-filled.
// Branch-free, so loads already in flight are not forced to drain.
template <typename T, int D, int F>
__device__ __forceinline__ void stage_rows(const T *__restrict__ g, int64_t gstride, int nrows,
                                           T *__restrict__ xs) {
    using G = ProjGeom<T, D, F>;
    constexpr int EPC = 16 / (int)sizeof(T);        // elements per 16-byte chunk
    constexpr int CPR = D / EPC;                    // chunks per row
    constexpr int N = kRows * CPR;
    static_assert(N % kThreads == 0, "tile chunks must divide the workgroup");
#pragma unroll
    for (int it = 0; it < N / kThreads; ++it) {
        const int c = (int)threadIdx.x + it * kThreads;
        const int r = c / CPR, col = (c % CPR) * EPC;
        const int rr = r < nrows ? r : nrows - 1;
        const uint4 t = *reinterpret_cast<const uint4 *>(g + (int64_t)rr * gstride + col);
        const bool ok = r < nrows;
        *reinterpret_cast<uint4 *>(xs + r * G::XLD + col) =
            make_uint4(ok ? t.x : 0u, ok ? t.y : 0u, ok ? t.z : 0u, ok ? t.w : 0u);
    }
}

// Two-phase variant used where the global loads should be issued early and
// the LDS writes done later: load into registers, then store.  Requires
// nrows >= 1.
template <typename T, int D>
struct RowChunks {
    static constexpr int EPC = 16 / (int)sizeof(T);
    static constexpr int CPR = D / EPC;
    static constexpr int N = kRows * CPR / kThreads;
    uint4 v[N];
};

template <typename T, int D>
__device__ __forceinline__ void load_rows(const T *__restrict__ g, int64_t gstride, int nrows,
                                          RowChunks<T, D> &rc) {
    constexpr int EPC = RowChunks<T, D>::EPC, CPR = RowChunks<T, D>::CPR;
#pragma unroll
    for (int it = 0; it < RowChunks<T, D>::N; ++it) {
        const int c = (int)threadIdx.x + it * kThreads;
        const int r = c / CPR, col = (c % CPR) * EPC;
        // branch-free: read a valid row (nrows >= 1), then zero rows past the
        // end, so no control flow forces the in-flight loads to drain
        const int rr = r < nrows ? r : nrows - 1;
        uint4 t = *reinterpret_cast<const uint4 *>(g + (int64_t)rr * gstride + col);
        const bool ok = r < nrows;
        rc.v[it] = make_uint4(ok ? t.x : 0u, ok ? t.y : 0u, ok ? t.z : 0u, ok ? t.w : 0u);
    }
}

template <typename T, int D, int F>
__device__ __forceinline__ void store_rows(const RowChunks<T, D> &rc, T *__restrict__ xs) {
    using G = ProjGeom<T, D, F>;
    constexpr int EPC = RowChunks<T, D>::EPC, CPR = RowChunks<T, D>::CPR;
#pragma unroll
    for (int it = 0; it < RowChunks<T, D>::N; ++it) {
        const int c = (int)threadIdx.x + it * kThreads;
        const int r = c / CPR, col = (c % CPR) * EPC;
        *reinterpret_cast<uint4 *>(xs + r * G::XLD + col) = rc.v[it];
    }
}

// W [D][F] of one head (global) -> LDS in the layout ProjGeom describes.
// bf16: each thread owns 8x8 blocks of W; it reads the block's 8 rows
// (16 B each, coalesced across threads), transposes the block in registers
// with byte permutes and writes 8 rows of Wt (16 B each).
// fp32: rows are copied as they are, 16 B per chunk.
template <typename T, int D, int F>
struct WChunks {
    static constexpr bool kBf16 = sizeof(T) == 2;
    static constexpr int EPC = 16 / (int)sizeof(T);
    static constexpr int BLOCKS = kBf16 ? (D / 8) * (F / 8) : 0;
    // bf16: blocks per thread (>= 1 when the thread owns any) ; fp32: chunks
    static constexpr int N = kBf16 ? (BLOCKS + kThreads - 1) / kThreads : D * F / EPC / kThreads;
    uint4 v[kBf16 ? 8 * N : N];
};

template <typename T, int D, int F>
__device__ __forceinline__ void load_w(const T *__restrict__ W, WChunks<T, D, F> &wc) {
    using C = WChunks<T, D, F>;
    if constexpr (C::kBf16) {
#pragma unroll
        for (int it = 0; it < C::N; ++it) {
            int blk = (int)threadIdx.x + it * kThreads;
            blk = blk < C::BLOCKS ? blk : C::BLOCKS - 1;     // spare threads repeat the last block
            const int bf = blk % (F / 8), bi = blk / (F / 8);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                wc.v[8 * it + e] = *reinterpret_cast<const uint4 *>(W + (int64_t)(8 * bi + e) * F + 8 * bf);
        }
    } else {
#pragma unroll
        for (int it = 0; it < C::N; ++it) {
            const int c = (int)threadIdx.x + it * kThreads;
            wc.v[it] = *reinterpret_cast<const uint4 *>(W + (int64_t)c * C::EPC);
        }
    }
}

// bf16 W^T tiles [F][D + 8] in LDS are swizzled: the 16-byte chunk q
// (elements 8q .. 8q+7) of row f sits at chunk q ^ ((f / 16) mod (D / 8)).
// One instruction of the transposing writes of store_w covers rows 8 apart,
// which the 17-chunk row stride alone maps to the same few bank groups; the
// swizzle spreads them (the step kernel's LDS bank-conflict cycles halved).
// The MFMA operand reads (16 consecutive rows, one chunk each) keep their
// pattern.  Element offset of chunk q of row f:
template <int D>
__device__ __forceinline__ int wt_off(int f, int q) {
    return f * (D + 8) + 8 * (q ^ ((f >> 4) & (D / 8 - 1)));
}

__device__ __forceinline__ uint32_t u4_word(const uint4 &v, int j) {
    return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

template <typename T, int D, int F>
__device__ __forceinline__ void store_w(const WChunks<T, D, F> &wc, T *__restrict__ ws) {
    using G = ProjGeom<T, D, F>;
    using C = WChunks<T, D, F>;
    if constexpr (C::kBf16) {
#pragma unroll
        for (int it = 0; it < C::N; ++it) {
            const int blk = (int)threadIdx.x + it * kThreads;
            if (blk < C::BLOCKS) {
                const int bf = blk % (F / 8), bi = blk / (F / 8);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    // column c of the block = row 8 bf + c of Wt: pairs of rows
                    // (2j, 2j+1) give word j, taking the low or high halves
                    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                    uint32_t w[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        w[j] = __builtin_amdgcn_perm(u4_word(wc.v[8 * it + 2 * j + 1], c >> 1),
                                                     u4_word(wc.v[8 * it + 2 * j], c >> 1), sel);
                    *reinterpret_cast<uint4 *>(ws + wt_off<D>(8 * bf + c, bi)) =
                        make_uint4(w[0], w[1], w[2], w[3]);
                }
            }
        }
    } else {
        constexpr int CPR = F / C::EPC;
#pragma unroll
        for (int it = 0; it < C::N; ++it) {
            const int c = (int)threadIdx.x + it * kThreads;
            const int i = c / CPR, f0 = (c % CPR) * C::EPC;
            *reinterpret_cast<uint4 *>(ws + i * G::WLD + f0) = wc.v[it];
        }
    }
}

// u = X W for a 32-row tile: X tile and W staged in LDS; u written to LDS.
// The 2 x (F/16) output tiles of 16x16 are spread over the 4 waves.
template <typename T, int D, int F, int ULD = ProjGeom<T, D, F>::ULD>
__device__ __forceinline__ void project_tile(const T *__restrict__ xs, const T *__restrict__ ws,
                                             float *__restrict__ us) {
    using G = ProjGeom<T, D, F>;
    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    constexpr int TILES = 2 * (F / 16);
    static_assert(TILES % 4 == 0, "tiles must split evenly over 4 waves");
#pragma unroll
    for (int q = 0; q < TILES / 4; ++q) {
        const int tau = wave + 4 * q;
        const int mt = tau & 1, nt = tau >> 1;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (G::kBf16) {
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(xs + (16 * mt + li) * G::XLD + 32 * ks + 8 * lg);
                const bf16x8 b = *reinterpret_cast<const bf16x8 *>(ws + wt_off<D>(16 * nt + li, 4 * ks + lg));
                acc = mfma_bf16(a, b, acc);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < D / 4; ++ks) {
                const float a = xs[(16 * mt + li) * G::XLD + 4 * ks + lg];
                const float b = ws[(4 * ks + lg) * G::WLD + 16 * nt + li];
                acc = mfma_f32(a, b, acc);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) us[(16 * mt + 4 * lg + r) * ULD + 16 * nt + li] = acc[r];
    }
}

// One 16-row tile of u = X W (all F features) for rows row0 .. row0+15 of a
// staged X tile, computed by one wave.  Accumulator layout: u[nt][r] is
// u[row0 + 4(l/16) + r][16 nt + l%16].
// kUnrollK = false keeps one K-step's operands live at a time (less register
// pressure, more LDS latency exposed).
template <typename T, int D, int F, bool kUnrollK = true>
__device__ __forceinline__ void project_rows16(const T *__restrict__ xs, const T *__restrict__ ws,
                                               int row0, floatx4 (&u)[F / 16]) {
    using G = ProjGeom<T, D, F>;
    const int lane = (int)threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int nt = 0; nt < F / 16; ++nt) u[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    if constexpr (G::kBf16) {
#pragma unroll (kUnrollK ? D / 32 : 1)
        for (int ks = 0; ks < D / 32; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(xs + (row0 + li) * G::XLD + 32 * ks + 8 * lg);
#pragma unroll
            for (int nt = 0; nt < F / 16; ++nt) {
                const bf16x8 b = *reinterpret_cast<const bf16x8 *>(ws + wt_off<D>(16 * nt + li, 4 * ks + lg));
                u[nt] = mfma_bf16(a, b, u[nt]);
            }
        }
    } else {
#pragma unroll 4
        for (int ks = 0; ks < D / 4; ++ks) {
            const float a = xs[(row0 + li) * G::XLD + 4 * ks + lg];
#pragma unroll
            for (int nt = 0; nt < F / 16; ++nt) u[nt] = mfma_f32(a, ws[(4 * ks + lg) * G::WLD + 16 * nt + li], u[nt]);
        }
    }
}

// N-tiles nt0 .. nt0+NTW-1 of u = X W for rows row0 .. row0+15 (one wave).
template <typename T, int D, int F, int NTW>
__device__ __forceinline__ void project_rows16_part(const T *__restrict__ xs, const T *__restrict__ ws,
                                                    int row0, int nt0, floatx4 (&u)[NTW]) {
    using G = ProjGeom<T, D, F>;
    const int lane = (int)threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int j = 0; j < NTW; ++j) u[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    if constexpr (G::kBf16) {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(xs + (row0 + li) * G::XLD + 32 * ks + 8 * lg);
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const bf16x8 b =
                    *reinterpret_cast<const bf16x8 *>(ws + wt_off<D>(16 * (nt0 + j) + li, 4 * ks + lg));
                u[j] = mfma_bf16(a, b, u[j]);
            }
        }
    } else {
#pragma unroll 4
        for (int ks = 0; ks < D / 4; ++ks) {
            const float a = xs[(row0 + li) * G::XLD + 4 * ks + lg];
#pragma unroll
            for (int j = 0; j < NTW; ++j)
                u[j] = mfma_f32(a, ws[(4 * ks + lg) * G::WLD + 16 * (nt0 + j) + li], u[j]);
        }
    }
}

// Hedgehog feature map on a 16-row tile held in the accumulator layout of
// project_rows16 ("Retrofitting Linear Attention into Diffusion Language
// Models", section 3.1): phi = [softmax(u), softmax(-u)] per row.  Each row
// lives in one 16-lane DPP row, so the max/min/sum reductions are four DPP
// steps, done for the lane's four rows at once.  On return u holds
// softmax(u) and un holds softmax(-u), in the same layout.
template <int F>
__device__ __forceinline__ void phi_rows16(floatx4 (&u)[F / 16], floatx4 (&un)[F / 16]) {
    constexpr int NT = F / 16;
    float mx[4], mn[4], sp[4], sn[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        mx[r] = u[0][r];
        mn[r] = u[0][r];
#pragma unroll
        for (int nt = 1; nt < NT; ++nt) {
            mx[r] = fmaxf(mx[r], u[nt][r]);
            mn[r] = fminf(mn[r], u[nt][r]);
        }
        mx[r] = row16_max(mx[r]);
        mn[r] = row16_min(mn[r]);
        sp[r] = 0.f;
        sn[r] = 0.f;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = u[nt][r];
            u[nt][r] = fast_exp(x - mx[r]);    // <= 1
            un[nt][r] = fast_exp(mn[r] - x);   // <= 1
            sp[r] += u[nt][r];
            sn[r] += un[nt][r];
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        sp[r] = 1.0f / row16_sum(sp[r]);
        sn[r] = 1.0f / row16_sum(sn[r]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            u[nt][r] *= sp[r];
            un[nt][r] *= sn[r];
        }
}

// Hedgehog feature map of one staged row, computed by one wave
// ("Retrofitting Linear Attention into Diffusion Language Models", section 3.1):
//   phi = [softmax(u), softmax(-u)],  u = x W.
// Lane l ends with phi_pos[m] = phi[l + 64 m] and phi_neg[m] = phi[F + l + 64 m].
template <int F>
__device__ __forceinline__ void phi_of_row(const float *__restrict__ urow, int lane,
                                           float (&phi_pos)[F / 64], float (&phi_neg)[F / 64]) {
    static_assert(F % 64 == 0, "F must be a multiple of 64");
    float u[F / 64];
    float mx = -INFINITY, mn = INFINITY;
#pragma unroll
    for (int m = 0; m < F / 64; ++m) {
        u[m] = urow[lane + 64 * m];
        mx = fmaxf(mx, u[m]);
        mn = fminf(mn, u[m]);
    }
    mx = wave_max(mx);
    mn = wave_min(mn);
    float sp = 0.f, sn = 0.f;
#pragma unroll
    for (int m = 0; m < F / 64; ++m) {
        phi_pos[m] = fast_exp(u[m] - mx);   // <= 1
        phi_neg[m] = fast_exp(mn - u[m]);   // <= 1
        sp += phi_pos[m];
        sn += phi_neg[m];
    }
    sp = wave_sum(sp);
    sn = wave_sum(sn);
    const float ip = 1.0f / sp, in = 1.0f / sn;
#pragma unroll
    for (int m = 0; m < F / 64; ++m) {
        phi_pos[m] *= ip;
        phi_neg[m] *= in;
    }
}

}  // namespace hba
