/*
 * far.h -- C ABI of the fused "sum of partials + residual add + RMSNorm (+ fp8 quant)"
 * epilogue for AMD Instinct MI355X (gfx950).
 *
 * What the operation is (the pages' titles and sections):
 *   - Page "vllm.models.common.ops.fused_allreduce_rms_norm", function
 *     fused_allreduce_rms_norm: returns (normed_output, new_residual), equal to
 *     norm(all_reduce(hidden_states), residual), where hidden_states is one rank's
 *     partial output of a row-parallel linear layer. On one GPU the all-reduce is the
 *     sum of P partial tensors already resident in device memory. The same source
 *     accumulates wider than the storage type (fp32_acc=True), takes eps from the
 *     norm's variance_epsilon and a weight_bias added to gamma (0 for plain RMSNorm,
 *     1 for Gemma-style norms).
 *   - Page "vllm.compilation.fusion": kFp8StaticTensorSym and kFp8DynamicTokenSym,
 *     FusedAddRMSNormStaticQuantPattern (outputs: result, residual) and
 *     FusedAddRMSNormDynamicQuantPattern (outputs: result, residual, scale): the
 *     normalised row is optionally quantised to fp8, symmetric, with one static
 *     per-tensor scale or one dynamic scale per token.
 *   - Page "PR #45307 report", call_trtllm_fused_allreduce_norm: inputs with more than
 *     two dimensions are viewed as [tokens, hidden] (all leading dims are tokens). This
 *     ABI takes the flattened [T, H] view; the Python binding flattens.
 *
 * Per token row t (s exact: summed in binary64 on the device, which holds the sum of
 * up to nine bf16/fp16 values exactly unless their exponents lie ~40 binades apart;
 * x, y in fp32):
 *   s[h]            = sum_p partials[p][t][h] + residual[t][h]
 *   residual_out    = RNE_dtype(s)                       (written; one rounding)
 *   x               = residual_out (the rounded values)
 *   r               = 1 / sqrt(sum_h x[h]^2 / H + eps)
 *   y[h]            = x[h] * r * (weight_bias + gamma[h])
 *   norm_out        = RNE_dtype(y)                       (when requested)
 *   static quant    : quant_out = E4M3(y / scale[0])
 *   dynamic quant   : scale_out[t] = max_h |y[h]| / 448 (1.0 for an all-zero row),
 *                     quant_out = E4M3(xw[h] * (448 / max_h |xw[h]|)) with
 *                     xw = x * (weight_bias + gamma): the same ratio as y / scale_out[t]
 *                     before the scale is rounded to fp32 (r cancels, so the codes need
 *                     no second pass), hence within one e4m3 step of
 *                     E4M3(y / scale_out[t]) and exactly 448 in magnitude at the row's
 *                     largest element (rows holding NaN or inf are converted element by
 *                     element as E4M3(y / scale_out[t])); the per-group mode does the
 *                     same over each FAR_FP8_GROUP consecutive elements of a row (a
 *                     per-group kernel is named on page "vllm.distributed.
 *                     device_communicators.aiter_custom_all_reduce",
 *                     build_supports_per_group_quant, without its group shape), the
 *                     per-tensor mode over the whole [T, H] tensor (page
 *                     "vllm.compilation.fusion", kFp8DynamicTensorSym)
 * E4M3 is OCP fp8 e4m3fn: NaN -> 0x7F (sign kept), clamp to [-448, 448], round to
 * nearest even. All tensors are row-major and contiguous.
 *
 * Execution: every call is asynchronous on `stream`, allocates nothing, needs no
 * workspace (except the per-tensor mode, whose workspace the caller passes), keeps no
 * pointer, and performs no host-device synchronisation, so it may be captured in a HIP
 * graph. The launch configuration depends only on (T, H, P,
 * dtype, quant) and on whether every tensor is element-aligned.
 *
 * Errors: all arguments are validated before anything is launched. On a validation
 * error the call returns a status other than FAR_OK and launches nothing. It never
 * silently does nothing: an unsupported shape is an error, not a no-op. FAR_ERR_HIP
 * means the runtime refused a launch; in the per-tensor mode (three kernels in stream
 * order) that can happen after the first kernel was queued, so the outputs may then
 * hold partial results.
 *
 * Logging: with the environment variable FAR_LOG set (to anything but "" or "0") when
 * the library is first called, every call that launches prints one line on stderr with
 * its shape, mode and launch plan.
 */
#ifndef FAR_H_
#define FAR_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t (a pointer to the runtime's stream object). NULL is
 * the device's default (null) stream. */
typedef struct ihipStream_t *far_stream_t;

#define FAR_MAX_PARTIALS 8
#define FAR_MAX_WAVES_PER_ROW 16   /* vector variant: wavefronts per token row */
#define FAR_MAX_PACKS_PER_LANE 5   /* vector variant: 16-byte packs per lane */

/* The enumerations below name values of plain 32-bit integer types (far_dtype_t,
 * far_quant_t, far_status_t, far_variant_t), so any int a caller passes is a defined
 * input, which the library checks and rejects with a status when it is not one of them. */
enum far_dtype_e {
    FAR_DTYPE_BF16 = 0, /* bfloat16 partials, residual, gamma, residual_out, norm_out */
    FAR_DTYPE_FP16 = 1  /* IEEE binary16 for the same tensors */
};
typedef int32_t far_dtype_t;

enum far_quant_e {
    FAR_QUANT_NONE = 0,              /* outputs: norm_out, residual_out */
    FAR_QUANT_FP8_STATIC_TENSOR = 1, /* outputs: quant_out, residual_out [, norm_out] */
    FAR_QUANT_FP8_DYNAMIC_TOKEN = 2, /* outputs: quant_out, scale_out [T], residual_out [, norm_out] */
    FAR_QUANT_FP8_DYNAMIC_GROUP = 3, /* outputs: quant_out, scale_out [T, ceil(H / FAR_FP8_GROUP)],
                                        residual_out [, norm_out] */
    FAR_QUANT_FP8_DYNAMIC_TENSOR = 4 /* outputs: quant_out, scale_out [1], residual_out [, norm_out];
                                        needs a workspace (far_workspace_bytes) */
};
typedef int32_t far_quant_t;

/* Elements per group along H for FAR_QUANT_FP8_DYNAMIC_GROUP (the last group of a row
 * is shorter when H is not a multiple). */
#define FAR_FP8_GROUP 128

enum far_status_e {
    FAR_OK = 0,
    FAR_ERR_NULL_POINTER = 1,     /* a required pointer is NULL */
    FAR_ERR_BAD_SHAPE = 2,        /* num_tokens < 0, hidden < 1 or hidden > 2^30 */
    FAR_ERR_BAD_DTYPE = 3,        /* dtype not a far_dtype_t */
    FAR_ERR_BAD_NUM_PARTIALS = 4, /* num_partials outside [1, FAR_MAX_PARTIALS] */
    FAR_ERR_BAD_QUANT_ARGS = 5,   /* quant_mode unknown, or scale/quant_out/scale_out
                                     given or missing against the mode */
    FAR_ERR_BAD_ALIAS = 6,        /* an output overlaps an input or another output in a
                                     way other than the allowed in-place forms */
    FAR_ERR_HIP = 7,              /* the HIP runtime refused the launch */
    FAR_ERR_BAD_PLAN = 8,         /* an explicit plan does not fit the shape or limits */
    FAR_ERR_WORKSPACE = 9,        /* the mode needs a workspace and none (or too small a
                                     one) was given */
    FAR_ERR_SCRATCH_LIMIT = 10    /* far_fused_add_rmsnorm_noalloc: the call needs more
                                     scratch than the library holds per GPU */
};
typedef int32_t far_status_t;

/* Bytes of device scratch far_fused_add_rmsnorm_noalloc holds per GPU (2 MiB). */
#define FAR_NOALLOC_SCRATCH_BYTES (2 * 1024 * 1024)

enum far_variant_e {
    FAR_VARIANT_EMPTY = 0,  /* T == 0: nothing to launch */
    FAR_VARIANT_VECTOR = 1, /* 16-byte packs, rows held in registers (a row's partial
                               last pack, H % 8 elements, moved by its lane with
                               4-, 2- and 1-byte accesses) */
    FAR_VARIANT_GENERIC = 2 /* element loop, any H and alignment, three passes per row */
};
typedef int32_t far_variant_t;

/* Launch plan. The vector variant assigns each token row to a team of
 * `waves_per_row` wavefronts (64 lanes each); lane l of the team holds the 16-byte
 * packs l, l + 64*waves_per_row, ... (at most `packs_per_lane` of them), so each wave
 * instruction reads 1 KiB of contiguous row. A workgroup holds `rows_per_block` teams.
 * The generic variant uses one workgroup of `block_threads` lanes per row. */
typedef struct {
    int32_t variant;        /* far_variant_t */
    int32_t waves_per_row;  /* 1..FAR_MAX_WAVES_PER_ROW */
    int32_t rows_per_block; /* >= 1 */
    int32_t packs_per_lane; /* 1..FAR_MAX_PACKS_PER_LANE (vector variant) */
    int32_t block_threads;  /* rows_per_block * waves_per_row * 64 <= 1024 */
    int32_t reserved;
    int64_t grid_blocks;    /* workgroups: at most ceil(T / rows_per_block) and at most
                               2^20 (a dispatch holds fewer than 2^32 lanes); with
                               fewer, each team (generic: workgroup) loops over rows
                               (grid-stride) */
} far_plan_t;

/*
 * far_fused_add_rmsnorm -- the whole epilogue for T token rows of H elements.
 *
 * partials     host array of `num_partials` device pointers, each [T, H] of dtype.
 *              The array itself is read during the call only.
 * num_partials P, 1..8 (P = 1 is plain fused add + RMSNorm).
 * residual     device [T, H] dtype, or NULL for the form without a residual input
 *              (new residual = sum of the partials; the normalisation of an
 *              all-reduce output with no residual add, and plain RMSNorm + fp8 quant
 *              with P = 1: page "vllm.compilation.fusion", RMSNormStaticQuantPattern /
 *              RMSNormDynamicQuantPattern; page "vllm.compilation.sequence_parallelism",
 *              FirstAllReduceRMSNormPattern, whose all-reduce output becomes the
 *              residual).
 * gamma        device [H] dtype (the norm weight; effective weight weight_bias + gamma).
 * num_tokens   T >= 0 (T == 0 returns FAR_OK and launches nothing).
 * hidden       H, 1..2^30. H <= 8 * 64 * FAR_MAX_WAVES_PER_ROW *
 *              FAR_MAX_PACKS_PER_LANE (= 40960) with element-aligned (2-byte)
 *              tensors takes the vector kernels (any H % 8); anything else (longer
 *              rows, a tensor at an odd byte address) the generic kernel.
 * dtype        storage type of partials, residual, gamma, residual_out, norm_out.
 * eps, weight_bias  host fp32 scalars, used as given (not validated; the arithmetic is
 *              IEEE fp32, so e.g. a negative eps gives r = NaN for a row whose mean
 *              square is below -eps, and that row's outputs are NaN).
 * quant_mode   far_quant_t.
 * scale        device fp32 [1], the static dequantisation scale S (q = E4M3(y / S));
 *              required for FAR_QUANT_FP8_STATIC_TENSOR, NULL otherwise.
 * norm_out     device [T, H] dtype; required for FAR_QUANT_NONE, optional (NULL skips
 *              it) with quantisation.
 * residual_out device [T, H] dtype, or NULL when the new residual is not wanted (page
 *              "vllm.compilation.sequence_parallelism", LastAllReduceRMSNormPattern
 *              keeps only the normalised output). It may be exactly `residual`
 *              (in-place residual update) or exactly one partial's buffer (the new
 *              residual written into the all-reduce input, as page
 *              "vllm.models.common.ops.fused_allreduce_rms_norm" does); otherwise it
 *              must not overlap any tensor. It may never overlap gamma or the static
 *              scale, which every row reads (not even when T == 1 makes gamma the size
 *              of a row tensor): FAR_ERR_BAD_ALIAS.
 * quant_out    device [T, H] bytes of fp8 e4m3fn; required iff quant_mode != NONE.
 * scale_out    device fp32; required iff the mode is dynamic: [T] per token,
 *              [T, ceil(H / FAR_FP8_GROUP)] row-major per group, [1] per tensor. With
 *              T == 0 nothing is written, the per-tensor scale included.
 * stream       the HIP stream the kernel is launched on.
 *
 * norm_out, quant_out and scale_out must not overlap any input or each other.
 * Inputs may overlap each other (they are only read). The per-tensor mode needs a
 * workspace, so it is only available through far_fused_add_rmsnorm_ex; here it
 * returns FAR_ERR_WORKSPACE.
 */
far_status_t far_fused_add_rmsnorm(
    const void *const *partials, int num_partials,
    const void *residual, const void *gamma,
    int64_t num_tokens, int64_t hidden, far_dtype_t dtype,
    float eps, float weight_bias,
    far_quant_t quant_mode, const float *scale,
    void *norm_out, void *residual_out, void *quant_out, float *scale_out,
    far_stream_t stream);

/*
 * far_fused_add_rmsnorm_ex -- as far_fused_add_rmsnorm, with an optional explicit
 * launch plan and a caller-provided workspace.
 *
 * plan         NULL for the automatic plan. Otherwise the library derives
 *              block_threads, takes grid_blocks as given when 1 <= grid_blocks <=
 *              ceil(T / rows_per_block) (0 means that maximum; with fewer, each team
 *              loops over rows), and checks the plan against the shape
 *              (FAR_ERR_BAD_PLAN if the packs do not fit, the block is too large,
 *              grid_blocks < 0, or the vector variant is asked for a tensor at an odd
 *              byte address). The generic variant ignores the
 *              other fields (its workgroup size follows H).
 * workspace    device memory of workspace_bytes bytes, used only by
 *              FAR_QUANT_FP8_DYNAMIC_TENSOR (at least far_workspace_bytes()); it may
 *              be NULL otherwise. Its contents on return are unspecified. It must not
 *              overlap any tensor. Calls that overlap in time must not share it.
 *
 * The per-tensor mode runs three kernels in stream order: the row pass (which also
 * records each row's max |y| and r in the workspace), a one-workgroup reduction to the
 * tensor scale, and an elementwise pass writing the codes.
 */
far_status_t far_fused_add_rmsnorm_ex(
    const void *const *partials, int num_partials,
    const void *residual, const void *gamma,
    int64_t num_tokens, int64_t hidden, far_dtype_t dtype,
    float eps, float weight_bias,
    far_quant_t quant_mode, const float *scale,
    void *norm_out, void *residual_out, void *quant_out, float *scale_out,
    far_stream_t stream, const far_plan_t *plan,
    void *workspace, int64_t workspace_bytes);

/*
 * far_fused_add_rmsnorm_noalloc -- as far_fused_add_rmsnorm, with the same arguments,
 * for callers that cannot allocate device memory: code being captured into a HIP
 * graph, tight serving loops, hosts that forbid allocation. It calls no allocating
 * routine. Every mode is available, the per-tensor dynamic mode included: its
 * workspace (8 * T bytes of per-row max |y| and r) is a scratch array of
 * FAR_NOALLOC_SCRATCH_BYTES bytes that the library keeps in each GPU's memory until the
 * process ends; its address on the current device is looked up (hipGetSymbolAddress)
 * by the first per-tensor call on that device.
 *
 * Limit: the per-tensor mode needs 8 * num_tokens <= FAR_NOALLOC_SCRATCH_BYTES, i.e. at
 * most 262144 tokens; a larger batch returns FAR_ERR_SCRATCH_LIMIT and launches
 * nothing. The other modes use no scratch and have no extra limit.
 * Devices: the scratch is per device, so `stream` must belong to the current device.
 * Concurrency: all calls on one GPU share that GPU's scratch, which keeps whatever the
 * last call left (nothing in it needs to start at zero: the row pass writes every
 * entry the later kernels read). Per-tensor calls that can overlap in time on one GPU
 * (different streams, or host threads without ordering between them) race on it and
 * give wrong results; calls queued on one stream are ordered and safe.
 */
far_status_t far_fused_add_rmsnorm_noalloc(
    const void *const *partials, int num_partials,
    const void *residual, const void *gamma,
    int64_t num_tokens, int64_t hidden, far_dtype_t dtype,
    float eps, float weight_bias,
    far_quant_t quant_mode, const float *scale,
    void *norm_out, void *residual_out, void *quant_out, float *scale_out,
    far_stream_t stream);

/* Workspace bytes a call with these arguments needs (0 for every mode but
 * FAR_QUANT_FP8_DYNAMIC_TENSOR, which needs 8 * num_tokens); -1 for invalid
 * arguments. */
int64_t far_workspace_bytes(int64_t num_tokens, int64_t hidden, far_quant_t quant_mode);

/*
 * far_plan -- the automatic launch plan for a shape, assuming element-aligned tensors
 * (tensors at odd byte addresses take the generic variant at call time). Pure host logic: it
 * touches no device. Token-count aware: few rows (decode) spread each row over many
 * wavefronts, many rows (prefill) give each row a workgroup of the wavefronts that hold it
 * at two 16-byte packs per lane. Page
 * "vllm.distributed.device_communicators.aiter_custom_all_reduce",
 * use_1stage_fused_ar_rms, states the launcher contract this follows: the launch shape
 * is a function of the call's static shape (token count, hidden size as 16-byte packs,
 * dtype), so a captured graph replays it unchanged, and the small-batch (decode)
 * regime is told apart from larger batches by the token count. Unlike that contract,
 * every token count and hidden size gets a plan here (rows beyond its pack limit take
 * the generic variant).
 * Returns FAR_OK and fills *out, or an argument error (out NULL -> FAR_ERR_NULL_POINTER).
 */
far_status_t far_plan(int64_t num_tokens, int64_t hidden, int num_partials,
                      far_dtype_t dtype, far_quant_t quant_mode, far_plan_t *out);

/* Static text naming a status code (never NULL). Every rejected call returns one of
 * these codes: page "vllm.distributed.device_communicators.aiter_custom_all_reduce",
 * supports_dynamic_hidden_dim, records that an older launcher did nothing, without an
 * error, for hidden sizes it did not support; this library reports such cases. */
const char *far_status_string(far_status_t status);

/* ABI version: major * 10000 + minor * 100 + patch. */
int far_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FAR_H_ */
