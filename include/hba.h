/*
 * hba.h -- C ABI of the block-hybrid attention library (libhba.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The method is block-hybrid attention from "Retrofitting Linear Attention
 * into Diffusion Language Models" (arXiv 2608.06628), section 3.1: during
 * blockwise semi-autoregressive diffusion decoding, each query of the active
 * block attends with exact bidirectional softmax to the block's own tokens
 * and reads all previously committed blocks through fixed-size per-head
 * linear-attention states built with the Hedgehog feature map; both parts
 * share one normaliser.  Committing a finished block folds its keys and
 * values into the states.
 *
 * Conventions shared by every call
 *   - Pure C.  Every buffer is caller-owned device memory (pointers from
 *     hipMalloc or a framework allocator); the library allocates nothing and
 *     keeps no global state, so calls are thread-safe.  The one exception is
 *     hba_prefix_softmax_split_noalloc, which uses a fixed scratch array the
 *     library holds per device (see there).
 *   - Calls enqueue kernels on `stream` (a hipStream_t passed as void*; NULL
 *     is the default stream) and return without synchronising.  A fault on
 *     the device surfaces at the caller's next synchronisation.
 *   - Host-checkable problems return a status and launch nothing: NULL
 *     pointers, non-positive or too-large sizes, unsupported (d, F, L, dtype),
 *     pointers not aligned to 16 bytes, kv_heads that is negative or does not
 *     divide heads.  A launch failure returns
 *     HBA_ERR_HIP.
 *   - Values that live on the device (slot indices, per-request lengths, gate
 *     values) cannot be checked without a synchronisation, so their ranges are
 *     preconditions stated per call; violating one is undefined behaviour.
 *   - All arrays are dense and row-major (C order) with the shapes given.
 *     Offsets are computed in 64 bits, so a state pool may exceed 2^31
 *     elements.
 *   - Supported shapes: head_dim d in {64, 128}; feat F in {64, 128} (the
 *     feature map has 2F entries); block L in [1, 32]; heads H >= 1.
 *   - Key/value head groups.  W, the gate, S and Z belong to query heads
 *     (section 3.1 learns W and the gate per query head; section 3.3 stores
 *     the state per query head beside the paged KV cache).  Keys and values
 *     may have fewer heads, Hkv = kv_heads, with H a multiple of Hkv:
 *     query head h then reads key/value head h / (H / Hkv), so consecutive
 *     groups of H / Hkv query heads share one (grouped-query attention).
 *     kv_heads = 0 or kv_heads = heads is plain multi-head attention.  The
 *     pages do not spell out the grouping; this is the common convention.
 *   - in_dtype selects the element type of q, k, v, x, W, Kc and Vc:
 *     HBA_F32 (float) or HBA_BF16 (bfloat16 stored as uint16).  States S, Z,
 *     feature-map output and attention outputs are always fp32; every
 *     accumulation is fp32.
 */
#ifndef HBA_H
#define HBA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HBA_F32 = 0,
    HBA_BF16 = 1
} hba_dtype;

typedef enum {
    HBA_OK = 0,
    HBA_ERR_NULL = 1,         /* a required pointer is NULL */
    HBA_ERR_SHAPE = 2,        /* a size is negative, zero where not allowed, or too large */
    HBA_ERR_UNSUPPORTED = 3,  /* (d, F, L) outside the supported set */
    HBA_ERR_DTYPE = 4,        /* in_dtype is not an hba_dtype */
    HBA_ERR_ALIGN = 5,        /* a pointer is not 16-byte aligned */
    HBA_ERR_CAPACITY = 6,     /* batch > n_slots while slot == NULL */
    HBA_ERR_HIP = 7           /* the HIP runtime refused a launch */
} hba_status;

/* Problem shape shared by the calls.  Fields a call does not use are
 * ignored by it (each call lists the fields it reads). */
typedef struct {
    int32_t batch;     /* B: requests in this call */
    int32_t heads;     /* H: query heads (one state and one W per head) */
    int32_t block;     /* L: tokens in the active block, 1..32 */
    int32_t head_dim;  /* d: 64 or 128 */
    int32_t feat;      /* F: 64 or 128; phi(x) has 2F entries */
    int32_t in_dtype;  /* hba_dtype of q, k, v, x, W, Kc, Vc */
    int64_t n_slots;   /* slots in the S/Z pool (hba_step, hba_commit) */
    int32_t kv_heads;  /* Hkv: key/value heads, dividing H; 0 means H */
} hba_shape;

/* Hedgehog feature map (section 3.1):
 *   phi(x) = [softmax(x W), softmax(-x W)] in R^{2F}, W in R^{d x F} per head,
 * each softmax taken over the F features.
 * Reads: heads, head_dim, feat, in_dtype.
 *   x    [n_rows][H][d]   in_dtype
 *   W    [H][d][F]        in_dtype
 *   phi  [n_rows][H][2F]  fp32 output; phi[..][0:F] = softmax(xW),
 *                         phi[..][F:2F] = softmax(-xW)
 * n_rows = 0 is a no-op; n_rows must be < 2^31. */
hba_status hba_feature_map(const hba_shape *shape, int64_t n_rows, const void *x,
                           const void *W, float *phi, void *stream);

/* One denoising step of block-hybrid attention (section 3.1), for every
 * request b < B, head h < H and query i < L of the active block:
 *   a_j     = exp(q_i . k_j / sqrt(d))            for all j < L (no mask)
 *   sm_num  = sum_j a_j v_j,  sm_den = sum_j a_j
 *   lin_num = phi(q_i)^T S,   lin_den = phi(q_i)^T Z   (S, Z of the request)
 *   out_i   = (w sm_num + lin_num) / (w sm_den + lin_den),  w = gate[h]
 * The kernels apply one exponent shift per query to both branches, which
 * leaves the ratio unchanged and keeps every term finite.
 * Reads: batch, heads, block, head_dim, feat, in_dtype, n_slots, kv_heads.
 *   q        [B][H][L][d]        in_dtype, the active block's queries
 *   k, v     [B][Hkv][L][d]      in_dtype, the active block's keys/values
 *   W        [H][d][F]           in_dtype
 *   gate     [H] fp32 or NULL    w = sigma(alpha) per head; NULL means w = 1.
 *                                Precondition: 0 < w < inf.
 *   S_pool   [n_slots][H][2F][d] fp32, S = sum_t phi(k_t) v_t^T (read only)
 *   Z_pool   [n_slots][H][2F]    fp32, Z = sum_t phi(k_t)      (read only)
 *   slot     [B] int32 or NULL   pool slot of request b; NULL means slot b
 *                                (then B <= n_slots is checked).
 *                                Precondition: 0 <= slot[b] < n_slots.
 *   out      [B][H][L][d]        fp32 output
 * An empty state (S = 0, Z = 0) gives exact softmax within the block. */
hba_status hba_step(const hba_shape *shape, const void *q, const void *k, const void *v,
                    const void *W, const float *gate, const float *S_pool,
                    const float *Z_pool, const int32_t *slot, float *out, void *stream);

/* Commit tokens into the recurrent states (section 3.1, state update):
 *   S += sum_t phi(k_t) v_t^T,   Z += sum_t phi(k_t)
 * over the first n_valid[b] of the n_tok tokens passed for request b.
 * Any n_tok >= 0 is accepted: a block, several blocks, or a whole prefix in
 * one call; by associativity the result does not depend on the chunking.
 * Reads: batch, heads, head_dim, feat, in_dtype, n_slots, kv_heads (block is
 * ignored).  The state of query head h absorbs key/value head h / (H / Hkv)
 * mapped through that query head's own W.
 *   n_valid  [B] int32 or NULL   tokens to fold per request; NULL means n_tok.
 *                                Precondition: 0 <= n_valid[b] <= n_tok.
 *   k, v     [B][Hkv][n_tok][d]  in_dtype
 *   W        [H][d][F]           in_dtype
 *   S_pool   [n_slots][H][2F][d] fp32, updated in place
 *   Z_pool   [n_slots][H][2F]    fp32, updated in place
 *   slot     [B] int32 or NULL   as for hba_step.  Precondition: slots are
 *                                distinct within one call (each request owns
 *                                its state; no atomics are used).
 * The update is deterministic: the same inputs give bitwise-equal states. */
hba_status hba_commit(const hba_shape *shape, int32_t n_tok, const int32_t *n_valid,
                      const void *k, const void *v, const void *W, float *S_pool,
                      float *Z_pool, const int32_t *slot, void *stream);

/* The last denoising step of a block fused with the commit of that block
 * (section 3.1; section 3.3 describes one launch per hybrid layer with its
 * causal state update).  Equivalent to hba_step(...) on the state as it is,
 * followed by hba_commit(n_tok = block, n_valid, k, v, ...): out is computed
 * from the old S and Z, then
 *   S += sum_t phi(k_t) v_t^T,   Z += sum_t phi(k_t)   (t < n_valid[b])
 * with the block's own keys and values.  For bf16 inputs with head_dim 128
 * it is one kernel that reads S once and writes it once; other shapes run
 * the step kernel and then the commit kernel.
 * Reads: batch, heads, block, head_dim, feat, in_dtype, n_slots, kv_heads.
 *   n_valid  [B] int32 or NULL   tokens of the block to fold; NULL means the
 *                                whole block.  Precondition: 0 <= n_valid[b] <= block.
 *   q, k, v, W, gate, slot, out  as for hba_step
 *   S_pool, Z_pool               as for hba_commit, updated in place.
 *                                Precondition: slots distinct within one call.
 * Errors: as for hba_step and hba_commit; nothing is launched on an error. */
hba_status hba_step_commit(const hba_shape *shape, const int32_t *n_valid, const void *q,
                           const void *k, const void *v, const void *W, const float *gate,
                           float *S_pool, float *Z_pool, const int32_t *slot, float *out,
                           void *stream);

/* Comparator: full softmax attention (section 2.2) of the active block's
 * queries over the request's cached prefix followed by the block itself,
 * scale 1/sqrt(d), every key visible, no gate -- the prefix attention that
 * block-hybrid attention replaces with a fixed-size state.
 * Reads: batch, heads, block, head_dim, in_dtype, kv_heads (feat and n_slots
 * ignored).
 *   prefix_len [B] int32 or NULL  cached tokens used by request b; NULL means
 *                                 max_prefix.  Precondition:
 *                                 0 <= prefix_len[b] <= max_prefix.
 *   q          [B][H][L][d]       in_dtype, the active block's queries
 *   k, v       [B][Hkv][L][d]     in_dtype, the active block's keys/values
 *   Kc, Vc     [B][Hkv][max_prefix][d] in_dtype, the prefix cache; may be NULL
 *                                 only when max_prefix == 0
 *   out        [B][H][L][d]       fp32 output */
hba_status hba_prefix_softmax(const hba_shape *shape, int32_t max_prefix,
                              const int32_t *prefix_len, const void *q, const void *k,
                              const void *v, const void *Kc, const void *Vc, float *out,
                              void *stream);

/* The comparator with its keys split over several workgroups per (request,
 * head), for batches too small to fill the GPU with one workgroup per pair
 * (the small-batch columns of Appendix A, Table 3).  Same result as
 * hba_prefix_softmax up to rounding: split s of a pair takes a contiguous
 * run of its P + L keys, writes its softmax-normalised partial output with
 * its running max and sum to the workspace, and a second kernel merges the
 * n_split partials of each query by rescaling them to their common max.
 * Reads: as hba_prefix_softmax.
 *   n_split          1..64 key splits per pair; 1 runs hba_prefix_softmax and
 *                    ignores the workspace.  hba_prefix_softmax_auto_split
 *                    gives a choice for the current device.
 *   workspace        device scratch of workspace_bytes >= the value of
 *                    hba_prefix_softmax_workspace_bytes(shape, n_split)
 *                    (4 B H n_split L (d + 2) bytes), 16-byte aligned, owned
 *                    by the caller; its contents on entry do not matter and
 *                    are undefined on return.  Calls in flight at the same
 *                    time need separate workspaces.
 *   other arguments  as hba_prefix_softmax.
 * Errors: as hba_prefix_softmax; HBA_ERR_SHAPE for n_split outside 1..64,
 * HBA_ERR_NULL for a NULL workspace with n_split > 1, HBA_ERR_CAPACITY for
 * a workspace smaller than required. */
hba_status hba_prefix_softmax_split(const hba_shape *shape, int32_t max_prefix, int32_t n_split,
                                    const int32_t *prefix_len, const void *q, const void *k,
                                    const void *v, const void *Kc, const void *Vc, float *workspace,
                                    int64_t workspace_bytes, float *out, void *stream);

/* Key splits for hba_prefix_softmax_split on the current device: enough
 * workgroups for one per compute unit, at least 256 keys per split, at most
 * 64; 1 when one workgroup per pair already fills the device or the shape is
 * invalid.  Reads: batch, heads, block, head_dim, in_dtype. */
int32_t hba_prefix_softmax_auto_split(const hba_shape *shape, int32_t max_prefix);

/* Workspace bytes hba_prefix_softmax_split needs: 0 for n_split = 1,
 * 4 B H n_split L (d + 2) otherwise, -1 for an invalid shape or n_split. */
int64_t hba_prefix_softmax_workspace_bytes(const hba_shape *shape, int32_t n_split);

/* Bytes of the library-held scratch behind hba_prefix_softmax_split_noalloc
 * (16 MiB per device). */
#define HBA_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)

/* hba_prefix_softmax_split without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The split partials go to a
 * fixed array of HBA_NOALLOC_SCRATCH_BYTES in device memory that the library
 * holds, one copy per device, until the process ends; its address is looked
 * up once per device, on the first call made with that device current.  A
 * call uses the array of the device current when it is made, which must be
 * the device of `stream` and of the buffers.  The call allocates nothing.  Same kernels and the same results as
 * hba_prefix_softmax_split with a caller workspace.
 *   Every call on one device shares that device's array, and the array keeps
 *   the last call's partials: calls that overlap on one device (concurrent
 *   streams, or host threads) race and give undefined results.  Calls
 *   ordered on one stream are safe.  Nothing in the array needs to start at
 *   zero.
 * Arguments: as hba_prefix_softmax_split, without workspace and
 * workspace_bytes.
 * Errors: as hba_prefix_softmax_split; HBA_ERR_CAPACITY when
 * hba_prefix_softmax_workspace_bytes(shape, n_split) exceeds
 * HBA_NOALLOC_SCRATCH_BYTES (nothing is launched); HBA_ERR_HIP when the
 * array's address cannot be obtained. */
hba_status hba_prefix_softmax_split_noalloc(const hba_shape *shape, int32_t max_prefix, int32_t n_split,
                                            const int32_t *prefix_len, const void *q, const void *k,
                                            const void *v, const void *Kc, const void *Vc, float *out,
                                            void *stream);

/* Stage-1 attention transfer (section 3.2): for the hybrid layer of section
 * 3.1 run over whole training sequences of N = n_blocks * block tokens per
 * (request, head) -- the queries of block n see exact softmax over block n
 * and the states S, Z of blocks 0..n-1 through the shared normaliser, gate
 * w = sigma(alpha[h]) -- the summed squared error against the frozen
 * softmax teacher's output and its gradient with respect to the layer's own
 * parameters:
 *   loss      = sum over b, h, tokens, columns of (out - target)^2
 *   dW[h]     = d loss / d W[h],   dalpha[h] = d loss / d alpha[h]
 * q, k, v and target are inputs (the backbone is frozen); the gradient flows
 * through the shared normaliser, phi(q), the states and phi(k).
 * fp32 inputs run on fp32 matrix cores.  For bf16 inputs the products of
 * two bf16 values are exact and every fp32 operand is split into a bf16 high
 * part and a bf16 residual on the bf16 matrix cores; accumulation is fp32
 * for both.  head_dim 128 only.
 * Reads: batch, heads, block, head_dim, feat, in_dtype, kv_heads.
 *   q, target  [B][H][N][128]      q in_dtype, target fp32
 *   k, v       [B][Hkv][N][128]    in_dtype
 *   W          [H][128][F]         in_dtype
 *   alpha      [H] fp32            the gate parameter, w = sigma(alpha)
 *   out        [B][H][N][128] fp32 the layer's output, or NULL
 *   loss       [1] fp32            overwritten
 *   dW         [H][128][F] fp32    overwritten
 *   dalpha     [H] fp32            overwritten
 *   workspace  caller-owned device scratch of at least
 *              hba_transfer_workspace_bytes(shape, n_blocks) bytes,
 *              16-byte aligned; contents on entry do not matter.  Calls in
 *              flight at the same time need separate workspaces.
 * The per-(request, head) parts are summed over requests in request order:
 * the same inputs give bitwise-equal results.  batch = 0 or n_blocks = 0
 * writes zeros.
 * Errors: HBA_ERR_UNSUPPORTED for head_dim != 128; HBA_ERR_CAPACITY for a
 * workspace that is too small; HBA_ERR_SHAPE for batch > 65535 or
 * N * 128 >= 2^31; otherwise as hba_step. */
hba_status hba_transfer(const hba_shape *shape, int32_t n_blocks, const void *q, const void *k,
                        const void *v, const void *W, const float *alpha, const float *target, float *out,
                        float *loss, float *dW, float *dalpha, float *workspace, int64_t workspace_bytes,
                        void *stream);

/* Workspace bytes of hba_transfer (4 B H (N (d + 1 + 4F) + 2 d F + 4), N
 * rounded up to a multiple of 4 in the second term),
 * -1 for an unsupported shape. */
int64_t hba_transfer_workspace_bytes(const hba_shape *shape, int32_t n_blocks);

/* Static description of a status code (never NULL). */
const char *hba_status_string(hba_status status);

/* Library ABI version, currently 6 (2 added hba_step_commit, 3 added
 * hba_shape.kv_heads, 4 added the split comparator, 5 hba_transfer,
 * 6 hba_prefix_softmax_split_noalloc). */
int32_t hba_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HBA_H */
