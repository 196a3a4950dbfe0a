// hba_api.cpp -- the C ABI declared in include/hba.h: host-side validation
// and dispatch to the gfx950 kernels.  Nothing here allocates device memory
// or synchronises; every call only enqueues kernels on the caller's stream:
// one for the step, the commit, the fused step + commit on its bf16 d = 128
// path and the unsplit comparator; two for the split comparator (the split
// kernel and the merge) and for the fused call's other shapes (step, then
// commit); up to six for the stage-1 transfer.
#include "hba.h"

#include <hip/hip_runtime.h>

#include <atomic>

#include "hba_internal.h"

namespace hba {

int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
        cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace hba

namespace {

constexpr int64_t kMaxGrid = 0x7fffffff;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

hba_status check_common(const hba_shape *s, bool need_block, bool need_feat) {
    if (!s) return HBA_ERR_NULL;
    if (s->in_dtype != HBA_F32 && s->in_dtype != HBA_BF16) return HBA_ERR_DTYPE;
    if (s->batch < 0 || s->heads <= 0) return HBA_ERR_SHAPE;
    if (s->head_dim != 64 && s->head_dim != 128) return HBA_ERR_UNSUPPORTED;
    if (need_feat && s->feat != 64 && s->feat != 128) return HBA_ERR_UNSUPPORTED;
    if (need_block && (s->block < 1 || s->block > 32)) {
        return s->block < 1 ? HBA_ERR_SHAPE : HBA_ERR_UNSUPPORTED;
    }
    if ((int64_t)s->batch * s->heads > kMaxGrid) return HBA_ERR_SHAPE;
    return HBA_OK;
}

// Query heads per key/value head, or 0 when kv_heads is negative or does not
// divide heads.
int kv_group(const hba_shape *s) {
    const int hkv = s->kv_heads == 0 ? s->heads : s->kv_heads;
    if (hkv < 0 || hkv > s->heads || s->heads % hkv) return 0;
    return s->heads / hkv;
}

hba_status from_hip(hipError_t e) { return e == hipSuccess ? HBA_OK : HBA_ERR_HIP; }

}  // namespace

extern "C" {

const char *hba_status_string(hba_status st) {
    switch (st) {
        case HBA_OK: return "ok";
        case HBA_ERR_NULL: return "a required pointer is NULL";
        case HBA_ERR_SHAPE: return "a size is out of range";
        case HBA_ERR_UNSUPPORTED: return "unsupported (head_dim, feat, block) combination";
        case HBA_ERR_DTYPE: return "in_dtype is not HBA_F32 or HBA_BF16";
        case HBA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case HBA_ERR_CAPACITY: return "batch exceeds n_slots with no slot map";
        case HBA_ERR_HIP: return "the HIP runtime refused the launch";
    }
    return "unknown status";
}

int32_t hba_abi_version(void) { return 6; }

hba_status hba_feature_map(const hba_shape *shape, int64_t n_rows, const void *x, const void *W,
                           float *phi, void *stream) {
    hba_status st = check_common(shape, false, true);
    if (st != HBA_OK) return st;
    if (n_rows < 0 || n_rows >= ((int64_t)1 << 31)) return HBA_ERR_SHAPE;
    if ((n_rows + 31) / 32 > kMaxGrid || shape->heads > 65535) return HBA_ERR_SHAPE;
    if (n_rows == 0) return HBA_OK;
    if (!x || !W || !phi) return HBA_ERR_NULL;
    if (!aligned16(x) || !aligned16(W) || !aligned16(phi)) return HBA_ERR_ALIGN;
    const int64_t H = shape->heads, d = shape->head_dim, P2 = 2 * shape->feat;
    hba::FeatureMapArgs a{x, W, phi, n_rows, shape->heads, H * d, d, 0, H * P2, P2, 0, 1};
    return from_hip(hba::launch_feature_map(a, shape->in_dtype == HBA_BF16, shape->head_dim,
                                            shape->feat, static_cast<hipStream_t>(stream)));
}

hba_status hba_step(const hba_shape *shape, const void *q, const void *k, const void *v,
                    const void *W, const float *gate, const float *S_pool, const float *Z_pool,
                    const int32_t *slot, float *out, void *stream) {
    hba_status st = check_common(shape, true, true);
    if (st != HBA_OK) return st;
    const int G = kv_group(shape);
    if (shape->n_slots < 0 || G == 0) return HBA_ERR_SHAPE;
    if (shape->batch == 0) return HBA_OK;
    if (!q || !k || !v || !W || !S_pool || !Z_pool || !out) return HBA_ERR_NULL;
    if (!slot && shape->batch > shape->n_slots) return HBA_ERR_CAPACITY;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(W) || !aligned16(S_pool) ||
        !aligned16(Z_pool) || !aligned16(out) || (gate && !aligned4(gate)) || (slot && !aligned4(slot)))
        return HBA_ERR_ALIGN;
    hba::StepArgs a{q, k, v, W, gate, S_pool, Z_pool, slot, out, shape->batch, shape->heads, shape->block, G};
    return from_hip(hba::launch_step(a, shape->in_dtype == HBA_BF16, shape->head_dim, shape->feat,
                                     static_cast<hipStream_t>(stream)));
}

hba_status hba_commit(const hba_shape *shape, int32_t n_tok, const int32_t *n_valid, const void *k,
                      const void *v, const void *W, float *S_pool, float *Z_pool, const int32_t *slot,
                      void *stream) {
    hba_status st = check_common(shape, false, true);
    if (st != HBA_OK) return st;
    const int G = kv_group(shape);
    if (n_tok < 0 || shape->n_slots < 0 || G == 0) return HBA_ERR_SHAPE;
    if (shape->batch == 0 || n_tok == 0) return HBA_OK;
    if (!k || !v || !W || !S_pool || !Z_pool) return HBA_ERR_NULL;
    if (!slot && shape->batch > shape->n_slots) return HBA_ERR_CAPACITY;
    if (!aligned16(k) || !aligned16(v) || !aligned16(W) || !aligned16(S_pool) || !aligned16(Z_pool) ||
        (n_valid && !aligned4(n_valid)) || (slot && !aligned4(slot)))
        return HBA_ERR_ALIGN;
    hba::CommitArgs a{n_valid, k, v, W, S_pool, Z_pool, slot, shape->batch, shape->heads, n_tok, G};
    return from_hip(hba::launch_commit(a, shape->in_dtype == HBA_BF16, shape->head_dim, shape->feat,
                                       static_cast<hipStream_t>(stream)));
}

hba_status hba_step_commit(const hba_shape *shape, const int32_t *n_valid, const void *q, const void *k,
                           const void *v, const void *W, const float *gate, float *S_pool, float *Z_pool,
                           const int32_t *slot, float *out, void *stream) {
    hba_status st = check_common(shape, true, true);
    if (st != HBA_OK) return st;
    const int G = kv_group(shape);
    if (shape->n_slots < 0 || G == 0) return HBA_ERR_SHAPE;
    if (shape->batch == 0) return HBA_OK;
    if (!q || !k || !v || !W || !S_pool || !Z_pool || !out) return HBA_ERR_NULL;
    if (!slot && shape->batch > shape->n_slots) return HBA_ERR_CAPACITY;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(W) || !aligned16(S_pool) ||
        !aligned16(Z_pool) || !aligned16(out) || (gate && !aligned4(gate)) || (slot && !aligned4(slot)) ||
        (n_valid && !aligned4(n_valid)))
        return HBA_ERR_ALIGN;
    hba::StepCommitArgs a{q, k, v, W, gate, S_pool, Z_pool, slot, n_valid, out, shape->batch, shape->heads,
                          shape->block, G};
    return from_hip(hba::launch_step_commit(a, shape->in_dtype == HBA_BF16, shape->head_dim, shape->feat,
                                            static_cast<hipStream_t>(stream)));
}

hba_status hba_prefix_softmax(const hba_shape *shape, int32_t max_prefix, const int32_t *prefix_len,
                              const void *q, const void *k, const void *v, const void *Kc,
                              const void *Vc, float *out, void *stream) {
    return hba_prefix_softmax_split(shape, max_prefix, 1, prefix_len, q, k, v, Kc, Vc, nullptr, 0, out, stream);
}

int32_t hba_prefix_softmax_auto_split(const hba_shape *shape, int32_t max_prefix) {
    if (check_common(shape, true, false) != HBA_OK || max_prefix < 0) return 1;
    // one workgroup per compute unit is resident at a time, so aim for one
    // round of workgroups over the device, with at least 256 keys per split
    const int64_t pairs = (int64_t)shape->batch * shape->heads;
    const int cus = hba::device_cus();
    if (pairs <= 0 || cus <= 0) return 1;
    const int64_t want = ((int64_t)cus + pairs - 1) / pairs;
    const int64_t by_len = ((int64_t)max_prefix + shape->block) / 256;
    int64_t ns = want < by_len ? want : by_len;
    if (ns > hba::kMaxPrefixSplit) ns = hba::kMaxPrefixSplit;
    return ns < 1 ? 1 : (int32_t)ns;
}

int64_t hba_prefix_softmax_workspace_bytes(const hba_shape *shape, int32_t n_split) {
    if (check_common(shape, true, false) != HBA_OK || n_split < 1 || n_split > hba::kMaxPrefixSplit) return -1;
    if (n_split == 1) return 0;
    return 4 * (int64_t)shape->batch * shape->heads * n_split * shape->block * (shape->head_dim + 2);
}

namespace {

// Host checks of the comparator's arguments apart from the workspace.
hba_status check_prefix(const hba_shape *shape, int32_t max_prefix, int32_t n_split, const int32_t *prefix_len,
                        const void *q, const void *k, const void *v, const void *Kc, const void *Vc,
                        const float *out) {
    hba_status st = check_common(shape, true, false);
    if (st != HBA_OK) return st;
    const int G = kv_group(shape);
    if (max_prefix < 0 || (int64_t)max_prefix + shape->block > 0x7fffffff || G == 0) return HBA_ERR_SHAPE;
    if (n_split < 1 || n_split > hba::kMaxPrefixSplit) return HBA_ERR_SHAPE;
    if ((int64_t)shape->batch * shape->heads * n_split > kMaxGrid) return HBA_ERR_SHAPE;
    if (shape->batch == 0) return HBA_OK;
    if (!q || !k || !v || !out) return HBA_ERR_NULL;
    if (max_prefix > 0 && (!Kc || !Vc)) return HBA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (max_prefix > 0 && (!aligned16(Kc) || !aligned16(Vc))) || (prefix_len && !aligned4(prefix_len)))
        return HBA_ERR_ALIGN;
    return HBA_OK;
}

hba_status launch_prefix(const hba_shape *shape, int32_t max_prefix, int32_t n_split, const int32_t *prefix_len,
                         const void *q, const void *k, const void *v, const void *Kc, const void *Vc,
                         float *workspace, float *out, void *stream) {
    hba::PrefixArgs a{prefix_len, q, k, v, Kc, Vc, out, shape->batch, shape->heads, shape->block, max_prefix,
                      kv_group(shape), n_split > 1 ? workspace : nullptr, n_split};
    return from_hip(hba::launch_prefix_softmax(a, shape->in_dtype == HBA_BF16, shape->head_dim,
                                               static_cast<hipStream_t>(stream)));
}

}  // namespace

hba_status hba_prefix_softmax_split(const hba_shape *shape, int32_t max_prefix, int32_t n_split,
                                    const int32_t *prefix_len, const void *q, const void *k, const void *v,
                                    const void *Kc, const void *Vc, float *workspace, int64_t workspace_bytes,
                                    float *out, void *stream) {
    hba_status st = check_prefix(shape, max_prefix, n_split, prefix_len, q, k, v, Kc, Vc, out);
    if (st != HBA_OK || shape->batch == 0) return st;
    if (n_split > 1 && !workspace) return HBA_ERR_NULL;
    if (n_split > 1 && workspace_bytes < hba_prefix_softmax_workspace_bytes(shape, n_split)) return HBA_ERR_CAPACITY;
    if (n_split > 1 && !aligned16(workspace)) return HBA_ERR_ALIGN;
    return launch_prefix(shape, max_prefix, n_split, prefix_len, q, k, v, Kc, Vc, workspace, out, stream);
}

hba_status hba_prefix_softmax_split_noalloc(const hba_shape *shape, int32_t max_prefix, int32_t n_split,
                                            const int32_t *prefix_len, const void *q, const void *k,
                                            const void *v, const void *Kc, const void *Vc, float *out,
                                            void *stream) {
    hba_status st = check_prefix(shape, max_prefix, n_split, prefix_len, q, k, v, Kc, Vc, out);
    if (st != HBA_OK || shape->batch == 0) return st;
    if (hba_prefix_softmax_workspace_bytes(shape, n_split) > hba::kStaticScratchBytes) return HBA_ERR_CAPACITY;
    float *ws = nullptr;
    if (n_split > 1 && hba::static_scratch(&ws) != hipSuccess) return HBA_ERR_HIP;
    return launch_prefix(shape, max_prefix, n_split, prefix_len, q, k, v, Kc, Vc, ws, out, stream);
}

int64_t hba_transfer_workspace_bytes(const hba_shape *shape, int32_t n_blocks) {
    if (check_common(shape, true, true) != HBA_OK || shape->head_dim != 128 || n_blocks < 0) return -1;
    const int64_t N = (int64_t)n_blocks * shape->block;
    return 4 * hba::transfer_workspace_floats((int64_t)shape->batch * shape->heads, N, shape->feat);
}

hba_status hba_transfer(const hba_shape *shape, int32_t n_blocks, const void *q, const void *k, const void *v,
                        const void *W, const float *alpha, const float *target, float *out, float *loss,
                        float *dW, float *dalpha, float *workspace, int64_t workspace_bytes, void *stream) {
    hba_status st = check_common(shape, true, true);
    if (st != HBA_OK) return st;
    if (shape->head_dim != 128) return HBA_ERR_UNSUPPORTED;
    const int G = kv_group(shape);
    if (n_blocks < 0 || G == 0) return HBA_ERR_SHAPE;
    const int64_t N = (int64_t)n_blocks * shape->block;
    // one sequence (N x 128 elements per request and head) is indexed in 32 bits
    if (N * 128 > 0x7fffffff || (int64_t)shape->batch * shape->heads * N > ((int64_t)1 << 40)) return HBA_ERR_SHAPE;
    if (shape->batch > 65535) return HBA_ERR_SHAPE;   // the feature-map pass runs one grid layer per request
    if (!W || !alpha || !loss || !dW || !dalpha || !workspace) return HBA_ERR_NULL;
    const bool work = shape->batch > 0 && n_blocks > 0;
    if (work && (!q || !k || !v || !target)) return HBA_ERR_NULL;
    if (workspace_bytes < hba_transfer_workspace_bytes(shape, n_blocks)) return HBA_ERR_CAPACITY;
    if (!aligned16(W) || !aligned4(alpha) || !aligned4(loss) || !aligned16(dW) || !aligned4(dalpha) ||
        !aligned16(workspace) || (out && !aligned16(out)) ||
        (work && (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(target))))
        return HBA_ERR_ALIGN;
    hba::TransferArgs a{q,   k,  v,      W,         alpha,        target,       out,         loss,
                        dW,  dalpha, workspace, shape->batch, shape->heads, G, shape->block, n_blocks};
    return from_hip(hba::launch_transfer(a, shape->in_dtype == HBA_BF16, shape->feat,
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"
