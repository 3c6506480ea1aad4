/*
 * da2.h - C ABI of the DraftAttention2 hot path on AMD Instinct MI355X (gfx950).
 *
 * The path replaces one attention call of a video diffusion transformer over
 * spatiotemporal latent tokens [DraftAttention2 (arXiv 2609.32628), abstract;
 * DraftAttention (arXiv 2505.14708), abstract]:
 *
 *   da2_plan       host only: validate a configuration, derive the window
 *                  geometry, the per-row block budgets and the workspace layout.
 *   da2_prepare    enqueue the fused operand preparation (pool + reorder +
 *                  fp8/MXFP4 quantize) and the draft map + shared ranking.
 *   da2_attention  enqueue the single block-sparse attention kernel with an
 *                  fp8 phase and an MXFP4 phase that share the online-softmax
 *                  state and the output accumulator; it writes outputs back in
 *                  the original (raster) token order.
 *
 * Conventions
 *  - Every device buffer (q, k, v, out, workspace, labels) is allocated and
 *    owned by the caller. The library allocates no device memory; a plan is
 *    an immutable host object, so calls on different plans (or the same plan
 *    from different threads) are safe. The one exception is
 *    da2_forward_scratch, whose workspace is a static device array of the
 *    library shared by all its calls on a GPU (see there).
 *  - Tensors q, k, v, out are [batch, heads, tokens, head_dim] addressed by
 *    element strides (stride_b, stride_h, stride_n; out may have its own,
 *    out_stride_*), head_dim contiguous.
 *    Tokens are in raster order (frame, row, column) of a frames x grid_h x
 *    grid_w latent grid. q, k, v are bf16; out is bf16 or fp32.
 *  - Rows are read and written as 16-byte vectors: the q, k, v and out
 *    pointers must be 16-byte aligned and the strides (inputs' and out's)
 *    multiples of 8 elements; otherwise da2_prepare / da2_attention return
 *    DA2_ERR_UNSUPPORTED before enqueuing anything.
 *  - Every call that takes a workspace also takes its size in bytes
 *    (workspace_bytes): a buffer smaller than the plan's workspace_bytes, or
 *    not 256-byte aligned, is DA2_ERR_WORKSPACE.
 *  - q, k and v are expected to hold finite values. Non-finite values give
 *    unspecified labels and outputs, but the kernels still access only the
 *    caller's buffers: the ranking sorts a NaN score below every real score,
 *    so its lists stay a permutation of real blocks, and every list entry
 *    that da2_prepare or da2_set_labels writes names a real block (the
 *    attention kernel reads tiles through these lists).
 *  - Argument errors are reported synchronously, before anything is enqueued.
 *    Kernel faults surface at the caller's next synchronisation, as usual in
 *    HIP. No C++ exception crosses this interface.
 *  - The workspace written by da2_prepare stays valid for da2_attention on
 *    the same stream until it is overwritten; q, k, v may be released once
 *    da2_prepare has completed on the stream.
 */
#ifndef DA2_H
#define DA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum da2_status {
    DA2_OK = 0,
    DA2_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, bad budget, ... */
    DA2_ERR_UNSUPPORTED = 2,   /* valid but outside what the kernels implement */
    DA2_ERR_WORKSPACE = 3,     /* workspace too small or not 256-byte aligned */
    DA2_ERR_HIP = 4            /* a HIP runtime call or launch failed */
} da2_status;

enum { DA2_OUT_BF16 = 0, DA2_OUT_FP32 = 1 };

/* da2_config.flags.
 * DA2_FLAG_PACK_EDGES: packed edge windows. The full windows stay one block
 * each (numbered (frame, window row, window column) among themselves, first);
 * the tokens of every partial window follow as one stream, window by window
 * in (frame, window row, window column) order and row-major inside each
 * window, cut into consecutive blocks of win_h * win_w tokens, so only the
 * last block can be short. A stream block may mix windows and frames; its
 * pooled statistics are over its own tokens. The pages fix neither this nor
 * the default (partial windows padded up to whole blocks); packing removes
 * the padded slots from the attention's work. */
enum { DA2_FLAG_PACK_EDGES = 1u };

/* Block labels, one int8 per (query block, key block). */
enum { DA2_SKIP = 0, DA2_LO = 1, DA2_HI = 2 };

/* Tile geometry of the workspace: every block is stored as DA2_TILE slots of
 * DA2_DPAD channels; slots beyond the window and channels beyond head_dim are
 * zero. */
#define DA2_TILE 128
#define DA2_DPAD 128
#define DA2_MAX_BLOCKS 4096
/* Size of the library's own static workspace, used by da2_forward_scratch. */
#define DA2_SCRATCH_BYTES (256ull << 20)

typedef struct da2_config {
    int32_t batch;
    int32_t heads;
    int32_t frames;
    int32_t grid_h;           /* latent rows per frame */
    int32_t grid_w;           /* latent columns per frame */
    int32_t head_dim;         /* 32, 64, 96 or 128 (other positive values: DA2_ERR_UNSUPPORTED) */
    int32_t win_h;            /* pooling window = one block: win_h x win_w tokens */
    int32_t win_w;            /* win_h * win_w <= 128 (larger: DA2_ERR_UNSUPPORTED) */
    double budget_hi;         /* fraction of key blocks per query block in fp8 */
    double budget_lo;         /* fraction in MXFP4 (clamped to 1 - budget_hi) */
    double softmax_scale;     /* tau; 0 selects 1/sqrt(head_dim) */
    int64_t stride_b;         /* element strides shared by q, k, v and out; */
    int64_t stride_h;         /* all three 0 selects the contiguous layout  */
    int64_t stride_n;
    int32_t out_dtype;        /* DA2_OUT_BF16 or DA2_OUT_FP32 */
    uint32_t flags;           /* 0 or DA2_FLAG_PACK_EDGES; other bits are invalid */
    int64_t out_stride_b;     /* element strides of out; all three 0 selects the */
    int64_t out_stride_h;     /* strides of q, k, v (so a fused QKV input can   */
    int64_t out_stride_n;     /* feed an output in another layout, e.g. [B,N,H,d]) */
} da2_config;

typedef struct da2_plan_s da2_plan_t;

/* Workspace sections (byte offsets from the workspace base, each 256-byte
 * aligned). BH = batch * heads, NB = n_blocks, T = DA2_TILE, P = DA2_DPAD.
 *   pool    f64 [4][BH][NB][P]  mean Q, max Q, mean K, max K over the window's tokens
 *   k8      u8  [BH][NB][T][P]  E4M3 codes of K, slot-major
 *   q8      u8  [BH][NB][T][P]  E4M3 codes of Q, slot-major
 *   v8t     u8  [BH][NB][P][T]  E4M3 codes of V, channel-major (transposed tile)
 *   e8      u8  [3][BH][NB]     E8M0 scale of each block for q, k, v
 *   q4, k4  u8  [BH][NB][T][P/2] E2M1 codes, two per byte, low nibble = even channel
 *   sq4,sk4 u8  [BH][NB][T][P/32] E8M0 scale per token per 32 channels
 *   v4t     u8  [BH][NB][P][T/2] E2M1 codes of V, channel-major, low nibble = even slot
 *   sv4t    u8  [BH][NB][P][T/32] E8M0 scale per channel per 32 slots
 *   scores  f64 [2][BH][NB][NB] draft logits; after da2_prepare section 0 holds
 *                               the combined block score C
 *   labels  i8  [BH][NB][NB]   DA2_SKIP / DA2_LO / DA2_HI
 *   hi, lo  i32 [BH][NB][n_hi], [BH][NB][n_lo]  key-block indices: in rank order
 *                               (best first) after da2_prepare, ascending after
 *                               da2_set_labels
 *   status  u32 [4]             [0]: rows whose labels had the wrong counts
 *                               (written by da2_set_labels)
 *   bias    f32 [NB+1][T]       0 for a slot holding a token, -inf for a padded slot;
 *                               row NB is all -inf (a key tile with no tokens)
 */
typedef struct da2_plan_info_s {
    int32_t n_blocks;
    int32_t block_size;
    int32_t n_wy;
    int32_t n_wx;
    int32_t n_hi;
    int32_t n_lo;
    int64_t tokens;
    int64_t slots;            /* n_blocks * block_size */
    double tau;
    uint64_t workspace_bytes;
    uint64_t off_pool, off_k8, off_v8t, off_e8;
    uint64_t off_q4, off_k4, off_v4t, off_sq4, off_sk4, off_sv4t;
    uint64_t off_scores, off_labels, off_hi, off_lo, off_status;
    uint64_t off_q8, off_bias;
    int32_t n_full;           /* full windows (fill a block each); with DA2_FLAG_PACK_EDGES the
                                 first n_full blocks, the rest being the packed stream */
    uint32_t flags;           /* the configuration's flags */
} da2_plan_info_t;

/* Validate cfg and build a plan. Host only: touches no GPU state.
 * Errors: DA2_ERR_INVALID_ARG for a NULL argument, a non-positive size,
 * negative strides (or stride_n < head_dim, or a zero stride_b / stride_h
 * when any stride is given; the same for the out_stride_* triple), budgets outside [0, 1] or not finite, a
 * negative or non-finite softmax_scale, an unknown out_dtype or flag bit,
 * or n_ret = 0; DA2_ERR_UNSUPPORTED for a head_dim or window outside the
 * domains above, more than DA2_MAX_BLOCKS blocks, batch * heads > 65535, or
 * a launch whose work-items along x exceed 32 bits: batch * heads * NB >
 * 8388607 (attention, 512 work-items per (b*h, query block)) or
 * batch * heads * ceil(NB / 32)^2 > 8388607 (draft logits, 2 x 256 per
 * 32 x 32 tile).
 * Geometry [DraftAttention (arXiv 2505.14708), abstract; news article on it,
 * method steps 1 and 4]: each frame is cut into win_h x win_w windows, padded
 * up to whole windows; a window is one block (with DA2_FLAG_PACK_EDGES: the
 * full windows plus ceil(partial-window tokens / (win_h * win_w)) packed
 * blocks). Budget counts per query block
 * [DraftAttention2, abstract, configurable budgets]:
 *   n_hi = floor(budget_hi * NB + 1/2),
 *   n_ret = floor((budget_hi + min(budget_lo, 1 - budget_hi)) * NB + 1/2),
 *   n_lo = n_ret - n_hi; n_ret = 0 is DA2_ERR_INVALID_ARG.
 * On success *out owns a heap object; release it with da2_plan_destroy. */
da2_status da2_plan(const da2_config* cfg, da2_plan_t** out);

/* Free a plan; NULL is accepted. */
void da2_plan_destroy(da2_plan_t* plan);

/* Sizes, budget counts and workspace offsets of a plan. */
da2_status da2_plan_info(const da2_plan_t* plan, da2_plan_info_t* out);

/* da2_prepare, da2_attention and da2_set_labels enqueue kernel launches
 * only (no allocation, memset or copy), so a caller may capture them in a
 * HIP graph; a replay reads and writes the buffers captured, with whatever
 * values they hold at replay time.
 *
 * Enqueue operand preparation and the draft ranking on hip_stream (a
 * hipStream_t; NULL = the null stream). Asynchronous.
 * [DraftAttention2, abstract]: 2D average- and max-pooled Q and K give a
 * low-resolution draft attention map that scores every (query block, key
 * block) pair; one shared ranking per query block labels the top n_hi key
 * blocks fp8, the next n_lo MXFP4 and skips the rest (ties: lower index);
 * operands are prepared once, reordered window-major and quantized to both
 * fp8 E4M3 (one power-of-two scale per block) and MXFP4 (E8M0 per 32
 * elements along the contraction axis).
 * q, k, v: device bf16, layout per cfg. workspace: device, >= workspace_bytes,
 * 256-byte aligned. Writes only the workspace. */
da2_status da2_prepare(const da2_plan_t* plan, const void* q, const void* k, const void* v,
                       void* workspace, size_t workspace_bytes, void* hip_stream);

/* Enqueue the phased block-sparse attention on hip_stream. Asynchronous.
 * [DraftAttention2, abstract]: one kernel runs an fp8 phase over the hi
 * blocks and an MXFP4 phase over the lo blocks, sharing data movement, the
 * softmax statistics and the output accumulator; skipped blocks cost nothing.
 * [DraftAttention, abstract]: outputs return to the original token order.
 * workspace: as left by da2_prepare (or da2_set_labels). out: device, layout
 * per cfg, dtype per cfg.out_dtype; every real token's row is written and
 * nothing else. */
da2_status da2_attention(const da2_plan_t* plan, const void* workspace, size_t workspace_bytes,
                         void* out, void* hip_stream);

/* Test hook, not for production: replace the labels in the workspace with
 * labels_dev (device int8 [BH][NB][NB]) and rebuild the hi/lo lists. A row
 * whose label counts differ from (n_hi, n_lo) is counted in status[0] (the
 * count is reset first) and its lists are left unspecified (every entry a
 * real block, block 0 where the row has too few labels): da2_attention then
 * gives that row unspecified outputs, still reading only the workspace.
 * Asynchronous. */
da2_status da2_set_labels(const da2_plan_t* plan, void* workspace, size_t workspace_bytes,
                          const int8_t* labels_dev, void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the work
 * of da2_prepare followed by da2_attention, with the library's own static
 * workspace of DA2_SCRATCH_BYTES (256 MiB) per GPU instead of a caller's
 * buffer. Same arguments, layouts, results and errors as that pair; a plan
 * whose workspace_bytes exceeds DA2_SCRATCH_BYTES is DA2_ERR_WORKSPACE (for
 * example Wan-480p-sized calls of up to 7 heads fit, Hunyuan-720p-sized of up
 * to 2). Allocates nothing: the static array is a device global of the
 * library's code object, held on each GPU the library runs on until the
 * process ends; its address is looked up once per device (on the device of
 * hip_stream). Every call on one GPU uses the same array, which keeps the
 * last call's contents: calls that may overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller. Asynchronous. */
da2_status da2_forward_scratch(const da2_plan_t* plan, const void* q, const void* k, const void* v, void* out,
                               void* hip_stream);

/* Static, never-NULL description of a status code. */
const char* da2_status_string(da2_status status);

/* The HIP error code behind the last DA2_ERR_HIP returned on the calling
 * thread (0 if none yet), and, when name is not NULL, its static, never-NULL
 * HIP error name in *name. Does not touch the device. */
int da2_last_hip_error(const char** name);

#ifdef __cplusplus
}
#endif

#endif /* DA2_H */
