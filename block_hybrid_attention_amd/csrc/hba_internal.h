// hba_internal.h -- kernel argument blocks and launchers behind the C ABI.
// Host validation (hba_api.cpp) has already checked every size, pointer and
// alignment the kernels rely on when these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hba.h"

namespace hba {

// Row r of head h in batch b (b < gridDim.z) reads x at
// b xs_b + (h / G) xs_h + r xs_r and writes phi at b ps_b + h ps_h + r ps_r.
// The public call uses x [n][H][d], phi [n][H][2F] (xs_r = H d, xs_h = d,
// ps_r = 2F H, ps_h = 2F, one batch, G = 1).
struct FeatureMapArgs {
    const void *x;
    const void *W;       // [H][d][F]
    float *phi;
    int64_t n;
    int H;
    int64_t xs_r, xs_h, xs_b;   // x strides (elements)
    int64_t ps_r, ps_h, ps_b;   // phi strides (floats)
    int G;                      // query heads per key/value head of x
};

// Key/value inputs are [B][H/G][...][d]: query head h of request b reads
// key/value row block (b H + h) / G = b (H/G) + h / G.  G = 1 is plain
// multi-head attention.
struct StepArgs {
    const void *q;           // [B][H][L][d]
    const void *k, *v;       // [B][H/G][L][d]
    const void *W;           // [H][d][F]
    const float *gate;       // [H] or null
    const float *S;          // [slots][H][2F][d]
    const float *Z;          // [slots][H][2F]
    const int32_t *slot;     // [B] or null
    float *out;              // [B][H][L][d]
    int B, H, L;
    int G;                   // query heads per key/value head
};

struct StepCommitArgs {
    const void *q;           // [B][H][L][d]
    const void *k, *v;       // [B][H/G][L][d]
    const void *W;           // [H][d][F]
    const float *gate;       // [H] or null
    float *S;                // [slots][H][2F][d], updated in place
    float *Z;                // [slots][H][2F], updated in place
    const int32_t *slot;     // [B] or null
    const int32_t *n_valid;  // [B] or null
    float *out;              // [B][H][L][d]
    int B, H, L;
    int G;
};
struct CommitArgs {
    const int32_t *n_valid;  // [B] or null
    const void *k, *v;       // [B][H/G][T][d]
    const void *W;           // [H][d][F]
    float *S;                // [slots][H][2F][d]
    float *Z;                // [slots][H][2F]
    const int32_t *slot;     // [B] or null
    int B, H, T;
    int G;
};

struct PrefixArgs {
    const int32_t *prefix_len;  // [B] or null
    const void *q;              // [B][H][L][d]
    const void *k, *v;          // [B][H/G][L][d]
    const void *Kc, *Vc;        // [B][H/G][P][d]
    float *out;                 // [B][H][L][d]
    int B, H, L, P;
    int G;
    // Split over keys: NS workgroups per (request, head), split s taking a
    // contiguous run of key tiles.  NS == 1 writes out directly; NS > 1
    // writes normalised partial outputs [B*H][NS][L][d] followed by the
    // partial (max, sum) pairs [B*H][NS][2][L] to part, merged afterwards.
    float *part;
    int NS;
};

// Stage-1 attention transfer over sequences of nb blocks of L tokens
// (N = nb L per (request, head)); head_dim 128.
struct TransferArgs {
    const void *q;           // [B][H][N][d]
    const void *k, *v;       // [B][H/G][N][d]
    const void *W;           // [H][d][F]
    const float *alpha;      // [H]
    const float *target;     // [B][H][N][d]
    float *out;              // [B][H][N][d] or null
    float *loss;             // [1]
    float *dW;               // [H][d][F]
    float *dalpha;           // [H]
    float *ws;               // workspace, transfer_workspace_floats(B H, N, F) floats
    int B, H, G, L, nb;
};
int64_t transfer_workspace_floats(int64_t BH, int64_t N, int F);
hipError_t launch_transfer(const TransferArgs &a, bool dtype_bf16, int F, hipStream_t stream);

// Largest key split of the comparator.
constexpr int kMaxPrefixSplit = 64;

// The comparator's library-held scratch (hba_prefix_softmax_split_noalloc):
// its size, and the address of the current device's copy.
constexpr int64_t kStaticScratchBytes = HBA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
hipError_t static_scratch(float **ptr);

// Compute units of the current device (0 if the runtime cannot say).
int device_cus();

// Enqueue kernel `k` with a single by-value argument block on `stream`; the
// returned status is this launch's own.
template <typename Args>
inline hipError_t launch_kernel(void (*k)(Args), dim3 grid, dim3 block, const Args &a,
                                hipStream_t stream) {
    void *args[] = {const_cast<Args *>(&a)};
    return hipLaunchKernel(reinterpret_cast<const void *>(k), grid, block, args, 0, stream);
}

// Each launcher enqueues one kernel on `stream`; dtype_bf16 selects the
// element type of the inputs.  Returns the launch status.
hipError_t launch_feature_map(const FeatureMapArgs &a, bool dtype_bf16, int d, int F, hipStream_t stream,
                              int batches = 1);
hipError_t launch_step(const StepArgs &a, bool dtype_bf16, int d, int F, hipStream_t stream);
hipError_t launch_commit(const CommitArgs &a, bool dtype_bf16, int d, int F, hipStream_t stream);
hipError_t launch_step_commit(const StepCommitArgs &a, bool dtype_bf16, int d, int F, hipStream_t stream);
hipError_t launch_prefix_softmax(const PrefixArgs &a, bool dtype_bf16, int d, hipStream_t stream);

}  // namespace hba
