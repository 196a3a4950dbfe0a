// hba_feature_map.hip -- the Hedgehog feature map as a standalone call.
//
// "Retrofitting Linear Attention into Diffusion Language Models", section 3.1:
//   phi(x) = [softmax(x W), softmax(-x W)] in R^{2F}, W in R^{d x F} per head.
//
// fp32 inputs: one workgroup per (32-row tile, head): the x rows and W go
// through LDS, u = x W runs on fp32 MFMA, and each wave turns 8 rows of u
// into phi with wave-wide max/min/sum reductions, writing 2F contiguous fp32
// per row (the same device code forms phi(k) in the fp32 commit).
#include "hba_device.h"
#include "hba_internal.h"

namespace hba {

template <typename T, int D, int F>
__global__ __launch_bounds__(kThreads) void feature_map_kernel(FeatureMapArgs a) {
    using P = ProjGeom<T, D, F>;
    constexpr int FM = F / 64;
    __shared__ __attribute__((aligned(16))) char smem[P::x_bytes + P::w_bytes + P::u_bytes];
    T *xs = reinterpret_cast<T *>(smem);
    T *ws = reinterpret_cast<T *>(smem + P::x_bytes);
    float *us = reinterpret_cast<float *>(smem + P::x_bytes + P::w_bytes);

    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
    const int h = (int)blockIdx.y;
    const int64_t r0 = (int64_t)blockIdx.x * kRows;
    const int64_t left = a.n - r0;
    const int nrows = left < kRows ? (int)left : kRows;

    const int64_t bz = blockIdx.z;
    const T *xg = static_cast<const T *>(a.x) + bz * a.xs_b + (int64_t)(h / a.G) * a.xs_h + r0 * a.xs_r;
    const T *Wg = static_cast<const T *>(a.W) + (int64_t)h * D * F;
    WChunks<T, D, F> wc;
    load_w<T, D, F>(Wg, wc);
    stage_rows<T, D, F>(xg, a.xs_r, nrows, xs);
    store_w<T, D, F>(wc, ws);
    __syncthreads();
    project_tile<T, D, F>(xs, ws, us);
    __syncthreads();
#pragma unroll 1
    for (int ii = 0; ii < 8; ++ii) {
        const int i = 8 * wave + ii;
        if (i >= nrows) break;
        float pp[FM], pn[FM];
        phi_of_row<F>(us + i * P::ULD, lane, pp, pn);
        float *o = a.phi + bz * a.ps_b + (int64_t)h * a.ps_h + (r0 + i) * a.ps_r;
#pragma unroll
        for (int m = 0; m < FM; ++m) {
            o[lane + 64 * m] = pp[m];
            o[F + lane + 64 * m] = pn[m];
        }
    }
}

// bf16 inputs: one workgroup per (4 row tiles of 32, head), W^T staged in LDS
// once.  Per tile, u^T = W^T x^T runs on bf16 MFMA with the x rows loaded
// straight into the B operand layout (lane: row 16 g + l%16, 8 values of d
// at 32 s + 8 (l/16)), so a lane holds F/4 features of ONE row and its softmax
// reductions are in registers plus two cross-lane steps.  Waves 0-1 form the
// softmax(u) half of rows 0-15 / 16-31, waves 2-3 the softmax(-u) half.  The
// tile of phi goes through LDS so each row (2F floats) is written by whole
// lanes of a wave with 16-byte nontemporal stores.  The next tile's x is
// requested before the current tile is computed.
template <int D, int F>
struct FmGeomBf16 {
    using P = ProjGeom<uint16_t, D, F>;
    static constexpr int PLD = 2 * F + 4;            // phi tile row stride (floats)
    static constexpr int phi_off = P::w_bytes;
    static constexpr int bytes = P::w_bytes + kRows * PLD * 4;
};
// kFmTiles: 32-row tiles per workgroup (W^T is staged once per workgroup)
template <int D, int F, int kFmTiles>
__global__ __launch_bounds__(kThreads, 2) void feature_map_kernel_bf16(FeatureMapArgs a) {
    using T = uint16_t;
    using P = ProjGeom<T, D, F>;
    using G = FmGeomBf16<D, F>;
    constexpr int KS = D / 32;      // K-steps of the projection
    constexpr int NT = F / 16;      // 16-feature tiles of u^T
    constexpr int RV = 2 * F / 4;   // float4 per phi row
    __shared__ __attribute__((aligned(16))) char smem[G::bytes];
    T *ws = reinterpret_cast<T *>(smem);
    float *ph = reinterpret_cast<float *>(smem + G::phi_off);

    const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int qgrp = wave & 1, half = wave >> 1;
    const int h = (int)blockIdx.y;
    const int64_t n = a.n;
    const int64_t tile0 = (int64_t)blockIdx.x * kFmTiles;
    const int64_t bz = blockIdx.z;
    const T *xg = static_cast<const T *>(a.x) + bz * a.xs_b + (int64_t)(h / a.G) * a.xs_h;

    auto load_x = [&](int64_t r0, bf16x8 (&xo)[KS]) {
        int64_t row = r0 + 16 * qgrp + li;
        row = row < n ? row : n - 1;   // rows past the end repeat the last one (not stored)
        const T *p = xg + row * a.xs_r + 8 * lg;
#pragma unroll
        for (int s_ = 0; s_ < KS; ++s_) xo[s_] = *reinterpret_cast<const bf16x8 *>(p + 32 * s_);
    };
    bf16x8 xo[2][KS];
    load_x(tile0 * kRows, xo[0]);
    {
        WChunks<T, D, F> wc;
        load_w<T, D, F>(static_cast<const T *>(a.W) + (int64_t)h * D * F, wc);
        store_w<T, D, F>(wc, ws);
    }
    __syncthreads();

#pragma unroll
    for (int t = 0; t < kFmTiles; ++t) {
        const int64_t r0 = (tile0 + t) * kRows;
        if (r0 >= n) break;   // uniform over the workgroup
        if (t + 1 < kFmTiles) {
            const int64_t rn = r0 + kRows;
            load_x(rn < n ? rn : r0, xo[(t + 1) & 1]);
        }
        // u^T: acc[m][r] = u[row 16 qgrp + l%16][feature 16m + 4(l/16) + r]
        floatx4 acc[NT];
#pragma unroll
        for (int m = 0; m < NT; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s_ = 0; s_ < KS; ++s_)
#pragma unroll
            for (int m = 0; m < NT; ++m) {
                const bf16x8 aw = *reinterpret_cast<const bf16x8 *>(ws + wt_off<D>(16 * m + li, 4 * s_ + lg));
                acc[m] = mfma_bf16(aw, xo[t & 1][s_], acc[m]);
            }
        // this wave's half: softmax over the F features of sgn * u
        const float sgn2 = half ? -kLog2e : kLog2e;
        float mx = -INFINITY;
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[m][r] *= sgn2;
                mx = fmaxf(mx, acc[m][r]);
            }
        mx = xrow_max(mx);
        float sm = 0.f;
#pragma unroll
        for (int m = 0; m < NT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[m][r] = fast_exp2(acc[m][r] - mx);
                sm += acc[m][r];
            }
        sm = xrow_sum(sm);
        const float is = 1.0f / sm;
        float *prow = ph + (16 * qgrp + li) * G::PLD + half * F + 4 * lg;
#pragma unroll
        for (int m = 0; m < NT; ++m)
            *reinterpret_cast<float4 *>(prow + 16 * m) =
                make_float4(acc[m][0] * is, acc[m][1] * is, acc[m][2] * is, acc[m][3] * is);
        __syncthreads();
        // store the tile row by row: 2F contiguous floats per (row, head)
        const int nrows = n - r0 < kRows ? (int)(n - r0) : kRows;
#pragma unroll
        for (int ii = 0; ii < kRows / 4; ++ii) {
            const int i = 4 * ii + wave;
            if (i < nrows) {
                float *o = a.phi + bz * a.ps_b + (int64_t)h * a.ps_h + (r0 + i) * a.ps_r;
#pragma unroll
                for (int e = lane; e < RV; e += kWave)
                    __builtin_nontemporal_store(*reinterpret_cast<const floatx4 *>(ph + i * G::PLD + 4 * e),
                                                reinterpret_cast<floatx4 *>(o) + e);
            }
        }
        __syncthreads();   // the phi tile is rewritten by the next tile
    }
}

template <typename T, int D, int F>
static hipError_t launch_fm_t(const FeatureMapArgs &a, unsigned batches, hipStream_t stream) {
    const int64_t tiles = (a.n + kRows - 1) / kRows;
    if constexpr (sizeof(T) == 2) {
        // the most tiles per workgroup (fewest W stagings) that still launches
        // one full round of two workgroups per CU (measured at 16 heads: 1
        // tile best at 1024 rows, 4 at 4096, 8 at 32768)
        const int64_t cus = device_cus();
        const int64_t round = 2 * (cus > 0 ? cus : 256);
        const int64_t per_tile_groups = tiles * a.H * batches;
        const dim3 blk(kThreads);
        auto groups = [&](int kt) { return (unsigned)((tiles + kt - 1) / kt); };
        if (per_tile_groups >= 8 * round)
            return launch_kernel(feature_map_kernel_bf16<D, F, 8>, dim3(groups(8), (unsigned)a.H, batches), blk, a, stream);
        if (per_tile_groups >= 4 * round)
            return launch_kernel(feature_map_kernel_bf16<D, F, 4>, dim3(groups(4), (unsigned)a.H, batches), blk, a, stream);
        if (per_tile_groups >= 2 * round)
            return launch_kernel(feature_map_kernel_bf16<D, F, 2>, dim3(groups(2), (unsigned)a.H, batches), blk, a, stream);
        return launch_kernel(feature_map_kernel_bf16<D, F, 1>, dim3(groups(1), (unsigned)a.H, batches), blk, a, stream);
    } else {
        return launch_kernel(feature_map_kernel<T, D, F>, dim3((unsigned)tiles, (unsigned)a.H, batches), dim3(kThreads), a, stream);
    }
}

hipError_t launch_feature_map(const FeatureMapArgs &a, bool bf16, int d, int F, hipStream_t stream, int batches) {
    const unsigned nb = (unsigned)batches;
#define HBA_FM_CASE(DD, FF)                                                                \
    if (d == DD && F == FF)                                                                \
        return bf16 ? launch_fm_t<uint16_t, DD, FF>(a, nb, stream) : launch_fm_t<float, DD, FF>(a, nb, stream);
    HBA_FM_CASE(64, 64)
    HBA_FM_CASE(64, 128)
    HBA_FM_CASE(128, 64)
    HBA_FM_CASE(128, 128)
#undef HBA_FM_CASE
    return hipErrorInvalidValue;
}

}  // namespace hba
