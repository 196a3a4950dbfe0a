// hba_transfer.h -- definitions shared by the stage-1 transfer kernels
// (hba_transfer.hip: fp32 inputs; hba_transfer_bf16.hip: bf16 inputs).
#pragma once
#include "hba_device.h"
#include "hba_internal.h"

namespace hba {

constexpr int kXferThreads = 512;   // eight waves
constexpr int kXferD = 128;

// Scheduling fence inside the long MFMA loops: keeps the compiler from
// hoisting every operand load of a loop at once, which would need more
// registers than the state and the accumulators leave free.
__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// Workspace layout (floats), per (request, head) pair bh of BH:
//   dnum [BH][N][d], dden [BH][Npad], phq, phk [BH][N][2F] (phi(q), phi(k)
//   of every row, written by the feature-map pass of the fp32 path),
//   dWq [BH][d][F], dWk [BH][d][F], scal [BH][4] (loss, dL/dw)
struct XferWs {
    int64_t dnum, dden, phq, phk, dWq, dWk, scal, total;
};
__host__ __device__ inline XferWs xfer_ws(int64_t BH, int64_t N, int F) {
    const int64_t npad = (N + 3) & ~int64_t(3);
    XferWs w;
    w.dnum = 0;
    w.dden = w.dnum + BH * N * kXferD;
    w.phq = w.dden + BH * npad;
    w.phk = w.phq + BH * N * 2 * F;
    w.dWq = w.phk + BH * N * 2 * F;
    w.dWk = w.dWq + BH * kXferD * F;
    w.scal = w.dWk + BH * kXferD * F;
    w.total = w.scal + BH * 4;
    return w;
}

// Forward sweep and the two gradient sweeps for bf16 inputs (hba_transfer_bf16.hip).
hipError_t launch_transfer_forward_bf16(const TransferArgs &a, int F, hipStream_t stream);
hipError_t launch_transfer_sweeps_bf16(const TransferArgs &a, int F, hipStream_t stream);

}  // namespace hba
