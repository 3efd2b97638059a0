/*
 * lora_mi355x.h -- C ABI of the multi-LoRA batched low-rank delta on MI355X
 * (gfx950): slot metadata, shrink, expand, and the fused apply.
 *
 * For a batch of T tokens, token t names an adapter slot token_slot[t] in
 * [0, S), or -1 for "no adapter".  The library adds, for every packed output
 * slice s (column window [offset[s], offset[s] + width[s]) of y),
 *
 *     y[t][offset[s] + n] (+)= sum_j u[s][t][j] * B_s[slot][j][n]
 *     u[s][t][j]           =  scale * slot_scale[slot] * sum_k x[t][k] * A_s[slot][k][j]
 *
 * which is y = xW + s*(xA)B of the LoRA forward with the base product xW
 * already in y (page "多 LoRA 服务：分段矩阵乘与适配器调度", section
 * "不合并权重，批量计算"), split into a shrink (x -> rank r, kept in fp32) and
 * an expand (rank r -> output slice) as in page "vLLM 源码完全拆解(十八):多 LoRA
 * 服务", sections "调用链" and "两个低秩 GEMM:shrink、expand 与 fp32 中转缓冲".
 *
 * Conventions shared by every entry point
 *   - Device pointers are HIP device addresses; "host" arrays live in host memory
 *     and are read before the call returns.
 *   - The caller owns every buffer, device and host.  The library never
 *     allocates or frees memory, never synchronises, and keeps no pointer after
 *     a call returns.  All device work is enqueued on `stream` (a hipStream_t
 *     passed as void*, NULL = the null stream), so calls are asynchronous.
 *   - Errors are return codes; nothing is enqueued when a call returns anything
 *     but LORA_OK, except LORA_ERR_HIP, which reports a failed launch.
 *   - Element types: x, A, B and y share one dtype, fp32 or bf16; the rank-r
 *     buffer u is always fp32; scales are fp32.  Accumulation is fp32.  bf16
 *     outputs are rounded once, to nearest even, when y is stored.
 *   - Supported shapes: 1 <= S <= 1023, r_max a multiple of 8 in [8, 128]
 *     (the kernels run at the next of 8, 16, 32, 64, 128 and read ranks past
 *     r_max as zeros; A, B and u keep r_max as their rank extent), d_in and every
 *     slice width a multiple of 8, 1 <= n_slices <= 8, every device pointer
 *     16-byte aligned, ldx and ldy multiples of 8, (r_max + 1) * d_in and
 *     (r_max + 1) * width below 2^28 (one slot's factor matrix is addressed with
 *     32-bit byte offsets).  Row offsets into x, u and y are int64.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lora_status {
    LORA_OK = 0,
    LORA_ERR_INVALID_ARG = 1,       /* null pointer, bad size, misalignment, overlap */
    LORA_ERR_UNSUPPORTED = 2,       /* dtype, r_max, slot count or slice count not built */
    LORA_ERR_WORKSPACE = 3,         /* workspace smaller than the *_workspace_bytes value */
    LORA_ERR_HIP = 4,               /* a HIP launch failed (hipGetLastError) */
    /* Range markers, not statuses: with them every int is a value of the type,
     * so a C caller may pass any int and a C++ definition may read it. */
    LORA_STATUS_RANGE_MIN_ = -2147483647 - 1,
    LORA_STATUS_RANGE_MAX_ = 2147483647
} lora_status;

typedef enum lora_dtype {
    LORA_F32 = 0,
    LORA_BF16 = 1,
    LORA_DTYPE_RANGE_MIN_ = -2147483647 - 1,  /* range markers, as above */
    LORA_DTYPE_RANGE_MAX_ = 2147483647
} lora_dtype;

/* How segments are computed.  BGMV: every segment on the vector (matrix-vector)
 * path; SGMV: every segment on the matrix-core tile path (bf16 only; fp32 falls
 * back to the vector path); AUTO: per segment, by its token count. */
typedef enum lora_mode {
    LORA_MODE_AUTO = 0,
    LORA_MODE_BGMV = 1,
    LORA_MODE_SGMV = 2,
    LORA_MODE_RANGE_MIN_ = -2147483647 - 1,  /* range markers, as above */
    LORA_MODE_RANGE_MAX_ = 2147483647
} lora_mode;

/* Layout of a slice's per-slot factor matrices (lora_weight.layout). */
typedef enum lora_layout {
    /* A_s [d_in][r_max] (row stride r_max), B_s [r_max][width_s] (row stride
     * width_s): the layout of page "多 LoRA 服务：分段矩阵乘与适配器调度",
     * section "不合并权重，批量计算". */
    LORA_LAYOUT_DEFAULT = 0,
    /* A only: A_s [r_max][d_in] (row stride d_in), the rank-major layout of
     * page "vLLM 源码完全拆解(十八):多 LoRA 服务", section "包装层的形态".  A
     * slot's ranks are then whole rows, so with per-slot ranks (d_slot_rank)
     * the ranks past a slot's own are never fetched.  bf16 only, r_max >= 16,
     * mode AUTO or SGMV; every slice of A must use it (else
     * LORA_ERR_UNSUPPORTED / LORA_ERR_INVALID_ARG). */
    LORA_LAYOUT_RANK_ROWS = 1,
    /* B only: B_s [width_s][r_max] (row stride r_max), one row of ranks per
     * output column: the output-major B of the same page and section (B
     * stored d_out x r).  A step of the expand then reads one contiguous
     * block of B.  bf16 only, r_max <= 64, mode AUTO or SGMV; every slice of B
     * must use it (else LORA_ERR_UNSUPPORTED / LORA_ERR_INVALID_ARG).
     * lora_apply runs such calls on the tile kernels (matrix-core expand),
     * never on the decode kernels or the long-segment expand. */
    LORA_LAYOUT_OUT_ROWS = 2
} lora_layout;

/* One packed slice of a stacked factor: slot a's matrix starts at
 * ptr + a * slot_stride elements, laid out as `layout` says. */
typedef struct lora_weight {
    const void *ptr;
    int64_t slot_stride;            /* elements between consecutive slots */
    int32_t layout;                 /* a lora_layout value */
    int32_t reserved;               /* must be 0 */
} lora_weight;

/* Bytes at the start of every lora_apply workspace that hold the per-tile call
 * count words of the decode-shaped apply (below, lora_apply_workspace_init). */
#define LORA_APPLY_SYNC_BYTES 295168
/* Word indices, in that region, of two counters the decode-shaped apply keeps
 * (read them as uint32): waits for peer workgroups' partial results that gave
 * up, and peers met on another accelerator die (XCD).  Each case is handled
 * (the waiting workgroup computes the peer's share itself, with the same
 * result); the counters only report that it happened. */
#define LORA_APPLY_WAITS_GAVE_UP_WORD 73728
#define LORA_APPLY_OTHER_XCD_WORD 73729

/* Slot metadata of one batch (page "vLLM 源码完全拆解(十八):多 LoRA 服务",
 * section "LoRAKernelMeta:先按槽位排序").  lora_prepare_meta fills the struct on
 * the host with device pointers into the caller's workspace and enqueues the
 * kernel that writes the arrays:
 *   sorted[T]       token indices grouped by slot: -1 first, then slots in
 *                   ascending order; original order inside a slot (stable)
 *   sorted_slot[T]  slot of each entry of `sorted` (-1 for no adapter)
 *   seg_slot[S+1]   slot id of each segment in that order, then -1 padding
 *   seg_count[S+1]  tokens per segment, then 0 padding
 *   seg_start[S+2]  0, then running sums of seg_count; T past the last segment
 *   info[8]         num_segments, no_lora (1 when no token has a valid slot,
 *                   also for T = 0), num_bad (tokens whose id lies outside
 *                   [-1, S); they are treated as -1), lora_begin (index in
 *                   `sorted` of the first token with an adapter), num_tiles,
 *                   then 3 zeros
 *   tiles           work tiles: every segment (the -1 one included) cut into
 *                   runs of at most 64 consecutive entries of `sorted`; tile i
 *                   is 68 int32 at tiles + 68 i: slot, rows, first position in
 *                   `sorted`, 0, then the rows token indices (the rest
 *                   unspecified).  Tiles follow the order of `sorted`; there
 *                   are num_tiles <= ceil(T / 64) + S + 1 of them.  The compute
 *                   kernels take their work from this list.
 * Past the tiles the workspace holds per-key counts that lora_prepare_meta
 * uses while it builds the arrays (large batches are counted in parts, by
 * several workgroups); they are not part of the result.
 * The struct stays valid until its workspace is reused; rebuild it whenever
 * token_slot changes.  Pass it by pointer to the compute calls.  They only
 * read it, so any number of calls, on any streams, may use one lora_meta at
 * the same time. */
typedef struct lora_meta {
    int64_t num_tokens;             /* rows of the batch */
    int32_t num_slots;              /* keys: slots, or (slot, local expert) pairs */
    int32_t x_row_div;              /* row i of the batch reads row i / x_row_div of x
                                       (1, or top-k for the MoE gate/up LoRA) */
    int32_t *sorted;
    int32_t *sorted_slot;
    int32_t *seg_slot;
    int32_t *seg_count;
    int32_t *seg_start;
    int32_t *info;
    int32_t *tiles;
} lora_meta;

/* Bytes of device workspace lora_prepare_meta needs for T tokens and S slots. */
lora_status lora_meta_workspace_bytes(int64_t num_tokens, int32_t num_slots,
                                      size_t *bytes);

/* Build the slot metadata of a batch.
 *   d_token_slot  device int32 [T], slot per token (-1 = none)
 *   d_ws          device workspace of at least lora_meta_workspace_bytes bytes,
 *                 16-byte aligned; owned by the caller, overwritten
 *   out           host struct, filled with pointers into d_ws
 * Cites page "vLLM 源码完全拆解(十八):多 LoRA 服务", section
 * "LoRAKernelMeta:先按槽位排序" (stable sort, unique counts, running sum whose
 * first entry is 0) and the worked example of section "一个完整的走查:两步
 * decode 里发生了什么".  T = 0 is valid (no_lora = 1).  Sets x_row_div = 1. */
lora_status lora_prepare_meta(const int32_t *d_token_slot, int64_t num_tokens,
                              int32_t num_slots, void *d_ws, size_t ws_bytes,
                              lora_meta *out, void *stream);

/* Per-slot ranks (argument d_slot_rank of lora_shrink, lora_expand and
 * lora_apply): NULL, or device int32 [S] giving the rank r_a <= r_max that slot
 * a's adapter really has.  The stacked buffers are sized for r_max, and an
 * adapter of smaller rank occupies only its first r_a columns of A and rows of
 * B, the rest being zero (page "vLLM 源码完全拆解(十八):多 LoRA 服务", section
 * "两个 LRU 缓存": a slot's buffers are written only in the adapter's valid
 * range).  With d_slot_rank the kernels read only those ranks, rounded up to a
 * multiple of 8, so a batch that mixes ranks no longer moves every adapter at
 * r_max (page "多 LoRA 服务：分段矩阵乘与适配器调度", section "练习": mixed ranks
 * padded to the largest waste memory traffic).  The result equals the padded
 * one whenever the padding holds zeros; u[s][t][j] is written as 0 for
 * j >= r_a.  Values are clamped to [0, r_max]. */

/* MoE LoRA: metadata over the (token, choice) pairs of a top-k routing step,
 * keyed by (slot, local expert).  Page "vLLM 源码完全拆解(十八):多 LoRA 服务",
 * section "融合计算:add_lora_w13 与 add_lora_w2": the experts' LoRA is applied
 * after the gate/up projection (before the activation) and after the down
 * projection (before the top-k weighted sum), on the tokens regrouped by
 * (adapter, expert); section "MoE 的 LoRA:按专家挂载、融合 kernel 与 EP 切片",
 * its buffer list: the factors are stacked per slot and
 * local expert; section "EP 下只装载本地专家的权重": a rank holds only its
 * local experts.
 * Row p = t * topk + j is token t's j-th choice.  Its key is
 *     slot(t) * E_local + local(topk_ids[t][j])
 * where local(e) = d_expert_map[e] when a map is given (-1: the expert lives
 * on another rank) and e otherwise; the key is -1 when the token has no
 * adapter or the expert is not local.  Ids out of range (a slot outside
 * [-1, S), an expert outside [0, E_global), a mapped id outside [-1, E_local),
 * or without a map an expert >= E_local) count as bad (info[2]) and as -1.
 * The result is an ordinary lora_meta over T * topk rows and S * E_local keys
 * (S * E_local <= 1023), with x_row_div = topk: lora_shrink and lora_apply
 * then read x row t for pair p, the token's hidden state (gate/up LoRA).  For
 * the down-projection LoRA, whose input has one row per pair, use a copy of
 * the struct with x_row_div = 1.  Factor slot index = slot * E_local + expert:
 * for stacks [S][E_local][...] pass slot_stride = one expert's matrix.
 *   d_topk_ids    device int32 [T][topk]
 *   d_token_slot  device int32 [T]
 *   d_expert_map  device int32 [E_global] or NULL */
lora_status lora_moe_meta_workspace_bytes(int64_t num_tokens, int32_t topk,
                                          int32_t num_slots,
                                          int32_t num_local_experts,
                                          size_t *bytes);
lora_status lora_prepare_moe_meta(const int32_t *d_topk_ids, int64_t num_tokens,
                                  int32_t topk, const int32_t *d_token_slot,
                                  int32_t num_slots, int32_t num_experts,
                                  int32_t num_local_experts,
                                  const int32_t *d_expert_map, void *d_ws,
                                  size_t ws_bytes, lora_meta *out, void *stream);

/* Bytes of device workspace lora_shrink needs (split-K partial sums; 0 when
 * the shape needs none).  No initialisation is required; calls that run at the
 * same time need workspaces of their own. */
lora_status lora_shrink_workspace_bytes(int64_t num_tokens, int32_t num_slots,
                                        int64_t d_in, int32_t n_slices,
                                        int32_t r_max, lora_dtype dtype,
                                        lora_mode mode, size_t *bytes);

/* Shrink: u[s][t][j] = scale * slot_scale[slot(t)] * sum_k x[t][k] * A_s[slot(t)][k][j]
 * for every token t with an adapter and every slice s; rows of tokens without
 * an adapter are not written.
 *   meta          metadata from lora_prepare_meta for this batch
 *   d_x           device [T][ldx] of dtype; the first d_in columns are read
 *   A             host array of n_slices descriptors (device pointers)
 *   scale         fp32 multiplier; d_slot_scale: device fp32 [S] or NULL (= 1)
 *   d_slot_rank   device int32 [S] or NULL (= r_max for every slot), see above
 *   d_u           device fp32 [n_slices][T][r_max], contiguous
 *   d_ws          workspace of lora_shrink_workspace_bytes bytes (may be NULL
 *                 when that size is 0)
 * Cites page "vLLM 源码完全拆解(十八):多 LoRA 服务", section "两个低秩 GEMM:
 * shrink、expand 与 fp32 中转缓冲" (the shrink kernel, its scaling argument and
 * the fp32 buffer laid out [slice][token][rank]). */
lora_status lora_shrink(const lora_meta *meta, const void *d_x, int64_t ldx,
                        int64_t d_in, lora_dtype dtype, int32_t n_slices,
                        const lora_weight *A, int32_t r_max, float scale,
                        const float *d_slot_scale, const int32_t *d_slot_rank,
                        float *d_u, lora_mode mode, void *d_ws, size_t ws_bytes,
                        void *stream);

/* Expand: for every token t and slice s, columns [offset[s], offset[s]+width[s])
 * of row t of y become (add_into_y ? y : 0) + sum_j u[s][t][j] * B_s[slot(t)][j][n];
 * a token without an adapter contributes 0 (its row is left as is when
 * add_into_y != 0 and its windows are set to 0 otherwise).  Columns outside
 * every window are never touched.
 *   d_u           device fp32 [n_slices][T][r_max] from lora_shrink
 *   B             host array of n_slices descriptors
 *   width, offset host int64 arrays [n_slices]; windows must not overlap and
 *                 must lie inside [0, ldy)
 *   d_slot_rank   device int32 [S] or NULL; ranks j >= r_a of u and B are not read
 *   d_y           device [T][ldy] of dtype, updated in place
 * Cites page "vLLM 源码完全拆解(十八):多 LoRA 服务", section "两个低秩 GEMM:
 * shrink、expand 与 fp32 中转缓冲" (the expand kernel: per-slice width and start
 * column, ADD_INPUTS) and section "双流:让 LoRA 与基座前向并行" (rows without an
 * adapter and a cleared output). */
lora_status lora_expand(const lora_meta *meta, const float *d_u, int32_t n_slices,
                        const lora_weight *B, const int64_t *width,
                        const int64_t *offset, int32_t r_max,
                        const int32_t *d_slot_rank, void *d_y, int64_t ldy,
                        lora_dtype dtype, int add_into_y, lora_mode mode,
                        void *stream);

/* Bytes of device workspace lora_apply needs for these sizes (a workspace
 * sized for the largest call can serve every smaller one).  Layout: the
 * count words (LORA_APPLY_SYNC_BYTES), the fp32 rank-r buffer, then the
 * partial sums of a shrink that splits d_in or of the decode-shaped kernel.
 * Only the count words need initialising: see lora_apply_workspace_init. */
lora_status lora_apply_workspace_bytes(int64_t num_tokens, int32_t num_slots,
                                       int64_t d_in, int32_t n_slices,
                                       int32_t r_max, lora_dtype dtype,
                                       lora_mode mode, size_t *bytes);

/* Zero the count words of an apply workspace (its first
 * LORA_APPLY_SYNC_BYTES bytes; enqueued on `stream`).  Call it once, before
 * the first lora_apply on a workspace; zero-filled memory needs no call.  The
 * decode-shaped apply (page "多 LoRA 服务：分段矩阵乘与适配器调度", section
 * "不合并权重，批量计算": the fused form for decode batches) spreads each work
 * tile over several workgroups that exchange partial results tagged with the
 * tile, the slice range and the call count, which these words keep.  Every
 * call leaves them consistent for the next call on the same workspace,
 * whatever its shapes.
 * The words must not be written between calls.
 *   d_ws      device workspace, 16-byte aligned
 *   ws_bytes  its size, at least LORA_APPLY_SYNC_BYTES (else LORA_ERR_WORKSPACE) */
lora_status lora_apply_workspace_init(void *d_ws, size_t ws_bytes, void *stream);

/* Shrink then expand on one stream: the whole delta of one layer, added into
 * (or stored to) the slices of y.  Arguments as in lora_shrink and lora_expand;
 * the rank-r buffer lives in d_ws.  Decode-shaped calls (few tokens per slot,
 * small per-token factors, mode AUTO or BGMV, r_max one of 8, 16, 32, 64,
 * default factor layouts) run as one fused kernel that keeps each token's
 * rank-r vector on chip; the others run the shrink and expand kernels.  Cites
 * page "vLLM 源码完全拆解(十八):多 LoRA
 * 服务", section "调用链" (add_lora_linear = shrink into an fp32 buffer, then
 * expand into the output slices).
 *   d_ws      workspace of at least lora_apply_workspace_bytes bytes, 16-byte
 *             aligned, whose count words were initialised once
 *             (lora_apply_workspace_init) and not written since except by
 *             lora_apply.  Calls that run at the same time need workspaces of
 *             their own; calls in stream order may share one. */
lora_status lora_apply(const lora_meta *meta, const void *d_x, int64_t ldx,
                       int64_t d_in, lora_dtype dtype, int32_t n_slices,
                       const lora_weight *A, const lora_weight *B,
                       const int64_t *width, const int64_t *offset,
                       int32_t r_max, float scale, const float *d_slot_scale,
                       const int32_t *d_slot_rank, void *d_y, int64_t ldy,
                       int add_into_y, lora_mode mode, void *d_ws,
                       size_t ws_bytes, void *stream);

/* Size of the device array that lora_apply_noalloc uses as its workspace. */
#define LORA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* lora_apply for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, checks and results as lora_apply,
 * without d_ws and ws_bytes: the workspace is a static device array of the
 * library, LORA_NOALLOC_SCRATCH_BYTES (64 MiB) per device, which each device
 * holds from the library's first use there until the process ends (zero at
 * load, so no lora_apply_workspace_init is needed).  Calls whose
 * lora_apply_workspace_bytes exceed that size return LORA_ERR_WORKSPACE and
 * enqueue nothing.  Allocates nothing: no hipMalloc, no hipFree, no allocating
 * library routine; the first call on a device looks up that device's copy of
 * the array once (hipGetSymbolAddress; LORA_ERR_HIP if that fails).  Every call
 * on a device shares its array: calls in stream order are fine, but calls
 * that overlap on one device (other streams, graphs replayed at the same time)
 * race and give wrong results. */
lora_status lora_apply_noalloc(const lora_meta *meta, const void *d_x, int64_t ldx,
                               int64_t d_in, lora_dtype dtype, int32_t n_slices,
                               const lora_weight *A, const lora_weight *B,
                               const int64_t *width, const int64_t *offset,
                               int32_t r_max, float scale, const float *d_slot_scale,
                               const int32_t *d_slot_rank, void *d_y, int64_t ldy,
                               int add_into_y, lora_mode mode, void *stream);

/* Human-readable name of a status code (static storage). */
const char *lora_status_string(lora_status status);

/* Library version, for the binding's sanity check. */
int32_t lora_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_H */
