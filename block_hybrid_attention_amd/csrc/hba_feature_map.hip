// hba_feature_map.hip -- the Hedgehog feature map as a standalone call.
//
// "Retrofitting Linear Attention into Diffusion Language Models", section 3.1:
//   phi(x) = [softmax(x W), softmax(-x W)] in R^{2F}, W in R^{d x F} per head.
//
// One workgroup per (32-row tile, head): the x rows and W go through LDS,
// u = x W runs on MFMA (bf16 or fp32), and each wave turns 8 rows of u into
// phi with wave-wide max/min/sum reductions, writing 2F contiguous fp32 per
// row.  The same device code forms phi(q) inside the step and phi(k) inside
// the commit.
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

    const T *xg = static_cast<const T *>(a.x) + (r0 * a.H + h) * D;
    const T *Wg = static_cast<const T *>(a.W) + (int64_t)h * D * F;
    WChunks<T, D, F> wc;
    load_w<T, D, F>(Wg, wc);
    stage_rows<T, D, F>(xg, (int64_t)a.H * D, nrows, xs);
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
        float *o = a.phi + ((r0 + i) * a.H + h) * (2 * F);
#pragma unroll
        for (int m = 0; m < FM; ++m) {
            o[lane + 64 * m] = pp[m];
            o[F + lane + 64 * m] = pn[m];
        }
    }
}

template <typename T, int D, int F>
static hipError_t launch_fm_t(const FeatureMapArgs &a, hipStream_t stream) {
    const unsigned tiles = (unsigned)((a.n + kRows - 1) / kRows);
    return launch_kernel(feature_map_kernel<T, D, F>, dim3(tiles, (unsigned)a.H), dim3(kThreads), a, stream);
}

hipError_t launch_feature_map(const FeatureMapArgs &a, bool bf16, int d, int F, hipStream_t stream) {
#define HBA_FM_CASE(DD, FF)                                                                \
    if (d == DD && F == FF)                                                                \
        return bf16 ? launch_fm_t<uint16_t, DD, FF>(a, stream) : launch_fm_t<float, DD, FF>(a, stream);
    HBA_FM_CASE(64, 64)
    HBA_FM_CASE(64, 128)
    HBA_FM_CASE(128, 64)
    HBA_FM_CASE(128, 128)
#undef HBA_FM_CASE
    return hipErrorInvalidValue;
}

}  // namespace hba
