/*
 * lora_oracle.c -- plain, slow, fp64 CPU oracle for the multi-LoRA batched
 * low-rank delta (metadata sort, shrink, expand).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path
 * never links, loads or calls it, and this file shares no code, header,
 * table or constant with the HIP kernels.
 *
 * Sources (pages of the open web; cited by title and section):
 *   [V]  "vLLM 源码完全拆解(十八):多 LoRA 服务——adapter 槽位、Punica 低秩核与批内多租户路由"
 *   [H]  "多 LoRA 服务：分段矩阵乘与适配器调度" (AI infra handbook)
 *
 * What is computed:
 *   oracle_prepare_meta   -- [V] section "LoRAKernelMeta:先按槽位排序": tokens
 *                            stably ordered by slot id (-1 = no adapter is the
 *                            smallest key), the distinct slot ids in ascending
 *                            order, their token counts and the running start
 *                            offsets whose first entry is 0.  Worked example in
 *                            [V] section "一个完整的走查:两步 decode 里发生了什么".
 *   oracle_lora_rows      -- [H] section "不合并权重，批量计算": the LoRA forward
 *                            y = xW + s*(xA)B, evaluated token by token with the
 *                            weights of the token's own adapter; A stored
 *                            [d_in][r], B stored [r][d_out] as on that page.  The
 *                            shrink (x -> rank r, scaled) and the expand (rank r ->
 *                            output slice, added into the base output or stored)
 *                            follow [V] sections "调用链" and "两个低秩 GEMM:shrink、
 *                            expand 与 fp32 中转缓冲"; the per-slice output window
 *                            [offset, offset+width) follows the expand kernel
 *                            description there.
 *   oracle_moe_keys       -- [V] sections "融合计算:add_lora_w13 与 add_lora_w2"
 *                            and "EP 下只装载本地专家的权重": the (slot, local
 *                            expert) key of every (token, choice) pair of a
 *                            top-k routing step; the experts' LoRA is then the
 *                            rows above with these keys as slots.
 *   oracle_expand_rows    -- the expand step alone, from a given fp32 rank-r
 *                            buffer laid out [slice][token][rank] ([V] section
 *                            "调用链").
 *
 * Readings taken where the pages are silent (each is also listed with the
 * design notes of the repository):
 *   - a slot id outside [-1, S) is counted as bad and the token is treated as
 *     having no adapter;
 *   - metadata arrays past the last segment are padded with slot -1, count 0
 *     and start offset T;
 *   - with the add flag clear, every slice window of every row is overwritten,
 *     so rows without an adapter receive 0 there (the pages leave such rows
 *     unwritten and have the caller pre-zero the output, [V] section
 *     "双流:让 LoRA 与基座前向并行"; storing 0 gives the same result);
 *   - the scale multiplies the rank-r vector (the scale is an argument of the
 *     shrink in [V]); in fp64 its placement changes only rounding.
 *
 * Every floating-point input is read exactly as stored (fp32, or bf16 widened
 * to fp32) and all arithmetic is fp64 with a plain left-to-right summation
 * over the contraction index.  No blocking, no reordering.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* Read element idx of a buffer holding fp32 or bf16 values, as a double. */
static double elem(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* The slot a token really uses: its id, or -1 when the id is not a valid slot. */
static int32_t effective_slot(int32_t id, int32_t num_slots)
{
    return (id >= -1 && id < num_slots) ? id : -1;
}

/*
 * Metadata of one batch.
 *   token_slot[T]      slot id per token, -1 = no adapter
 *   sorted[T]          token indices grouped by slot: keys -1, 0, 1, ... in that
 *                      order, original index order inside a key (stable)
 *   seg_slot[S+1]      distinct slot ids present, ascending; padded with -1
 *   seg_count[S+1]     tokens per segment; padded with 0
 *   seg_start[S+2]     seg_start[0] = 0, seg_start[i+1] = seg_start[i] + seg_count[i];
 *                      entries past num_segments hold T
 *   *num_segments      number of segments (the -1 segment counts when present)
 *   *no_lora           1 when no token has an adapter (also when T == 0)
 *   *num_bad           number of tokens whose id is outside [-1, S)
 * The definition is applied literally: for each key in ascending order, scan
 * the batch from the first token to the last and append the tokens that carry
 * that key.
 */
int oracle_prepare_meta(const int32_t *token_slot, int64_t T, int32_t S,
                        int32_t *sorted, int32_t *seg_slot, int32_t *seg_count,
                        int32_t *seg_start, int32_t *num_segments,
                        int32_t *no_lora, int32_t *num_bad)
{
    if (T < 0 || S < 0 || (T > 0 && (!token_slot || !sorted)))
        return ORACLE_BAD_ARG;

    int32_t bad = 0, with_adapter = 0;
    for (int64_t t = 0; t < T; ++t) {
        if (effective_slot(token_slot[t], S) != token_slot[t])
            ++bad;
        if (effective_slot(token_slot[t], S) >= 0)
            ++with_adapter;
    }

    for (int32_t i = 0; i < S + 1; ++i) {
        seg_slot[i] = -1;
        seg_count[i] = 0;
    }
    for (int32_t i = 0; i < S + 2; ++i)
        seg_start[i] = (int32_t)T;
    seg_start[0] = 0;

    int64_t pos = 0;
    int32_t nseg = 0;
    for (int32_t key = -1; key < S; ++key) {
        int32_t count = 0;
        for (int64_t t = 0; t < T; ++t) {
            if (effective_slot(token_slot[t], S) == key) {
                sorted[pos++] = (int32_t)t;
                ++count;
            }
        }
        if (count > 0) {
            seg_slot[nseg] = key;
            seg_count[nseg] = count;
            seg_start[nseg + 1] = seg_start[nseg] + count;
            ++nseg;
        }
    }

    *num_segments = nseg;
    *no_lora = (with_adapter == 0) ? 1 : 0;
    *num_bad = bad;
    return ORACLE_OK;
}

/*
 * Output rows of y = y0 + s * (x A[slot]) B[slot], one requested token at a time.
 *
 *   dtype                 ORACLE_F32 or ORACLE_BF16, shared by x, A, B and y0
 *   x [T][ldx]            activations; the first d_in columns are used
 *   token_slot [T], S     slot per token and the number of slots
 *   n_slices              number of packed output slices
 *   A[s]                  slice s factor, [S][d_in][r_max] with a_slot_stride[s]
 *                         elements between slots
 *   B[s]                  slice s factor, [S][r_max][width[s]] with b_slot_stride[s]
 *                         elements between slots
 *   width[s], offset[s]   slice s writes columns [offset[s], offset[s]+width[s])
 *   scale, slot_scale     the rank-r vector of a token on slot a is multiplied by
 *                         scale * slot_scale[a] (slot_scale may be NULL = 1)
 *   y0 [T][ldy]           base output; add != 0 adds into it, add == 0 stores
 *   rows[n_rows]          which tokens to evaluate
 *   y_out [n_rows][ldy]   result rows in fp64 (columns outside every window are y0)
 *   u_out                 optional [n_rows][n_slices][r_max]: the scaled rank-r
 *                         vectors (0 for rows without an adapter)
 */
int oracle_lora_rows(int dtype, const void *x, int64_t ldx, int64_t d_in,
                     const int32_t *token_slot, int32_t S, int32_t n_slices,
                     const void *const *A, const int64_t *a_slot_stride,
                     int32_t r_max, const void *const *B,
                     const int64_t *b_slot_stride, const int64_t *width,
                     const int64_t *offset, double scale,
                     const float *slot_scale, const void *y0, int64_t ldy,
                     int add, const int64_t *rows, int64_t n_rows,
                     double *y_out, double *u_out)
{
    if ((dtype != ORACLE_F32 && dtype != ORACLE_BF16) || n_slices < 1 ||
        r_max < 1 || d_in < 1 || ldx < d_in)
        return ORACLE_BAD_ARG;
    double *u = (double *)malloc(sizeof(double) * (size_t)r_max);
    if (!u)
        return ORACLE_BAD_ARG;

    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t t = rows[i];
        const int32_t slot = effective_slot(token_slot[t], S);
        double *yrow = y_out + i * ldy;
        for (int64_t c = 0; c < ldy; ++c)
            yrow[c] = elem(y0, dtype, t * ldy + c);

        for (int32_t s = 0; s < n_slices; ++s) {
            const int64_t w = width[s], off = offset[s];
            if (slot < 0) {
                for (int32_t j = 0; j < r_max; ++j)
                    u[j] = 0.0;
            } else {
                const double sc =
                    scale * (slot_scale ? (double)slot_scale[slot] : 1.0);
                const int64_t abase = a_slot_stride[s] * slot;
                /* shrink: u_j = sc * sum_k x[t][k] * A[slot][k][j] */
                for (int32_t j = 0; j < r_max; ++j) {
                    double acc = 0.0;
                    for (int64_t k = 0; k < d_in; ++k)
                        acc += elem(x, dtype, t * ldx + k) *
                               elem(A[s], dtype, abase + k * r_max + j);
                    u[j] = sc * acc;
                }
            }
            if (u_out)
                for (int32_t j = 0; j < r_max; ++j)
                    u_out[(i * n_slices + s) * r_max + j] = u[j];

            /* expand: y[t][off+n] = (add ? y0 : 0) + sum_j u_j * B[slot][j][n] */
            const int64_t bbase = slot < 0 ? 0 : b_slot_stride[s] * slot;
            for (int64_t n = 0; n < w; ++n) {
                double acc = 0.0;
                if (slot >= 0)
                    for (int32_t j = 0; j < r_max; ++j)
                        acc += u[j] * elem(B[s], dtype, bbase + (int64_t)j * w + n);
                const double base = add ? yrow[off + n] : 0.0;
                yrow[off + n] = base + acc;
            }
        }
    }
    free(u);
    return ORACLE_OK;
}

/*
 * The expand step alone: y rows from a given fp32 rank-r buffer
 * u[n_slices][ldu][r_max] (token-major inside a slice, original token order).
 * Rows without a valid slot get 0 in every window when add == 0 and keep y0
 * when add != 0.  Other arguments as in oracle_lora_rows.
 */
int oracle_expand_rows(int dtype, const float *u, int64_t ldu,
                       const int32_t *token_slot, int32_t S, int32_t n_slices,
                       int32_t r_max, const void *const *B,
                       const int64_t *b_slot_stride, const int64_t *width,
                       const int64_t *offset, const void *y0, int64_t ldy,
                       int add, const int64_t *rows, int64_t n_rows,
                       double *y_out)
{
    if ((dtype != ORACLE_F32 && dtype != ORACLE_BF16) || n_slices < 1 ||
        r_max < 1)
        return ORACLE_BAD_ARG;
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t t = rows[i];
        const int32_t slot = effective_slot(token_slot[t], S);
        double *yrow = y_out + i * ldy;
        for (int64_t c = 0; c < ldy; ++c)
            yrow[c] = elem(y0, dtype, t * ldy + c);
        for (int32_t s = 0; s < n_slices; ++s) {
            const int64_t w = width[s], off = offset[s];
            const float *ut = u + ((int64_t)s * ldu + t) * r_max;
            const int64_t bbase = slot < 0 ? 0 : b_slot_stride[s] * slot;
            for (int64_t n = 0; n < w; ++n) {
                double acc = 0.0;
                if (slot >= 0)
                    for (int32_t j = 0; j < r_max; ++j)
                        acc += (double)ut[j] *
                               elem(B[s], dtype, bbase + (int64_t)j * w + n);
                const double base = add ? yrow[off + n] : 0.0;
                yrow[off + n] = base + acc;
            }
        }
    }
    return ORACLE_OK;
}

/*
 * oracle_moe_keys -- key of every (token, choice) pair of a top-k MoE routing
 * step, for the experts' LoRA ([V] section "融合计算:add_lora_w13 与
 * add_lora_w2": the LoRA works on the tokens regrouped by adapter and expert;
 * section "MoE 的 LoRA:按专家挂载、融合 kernel 与 EP 切片", its buffer list:
 * factors stacked per slot and local expert; section
 * "EP 下只装载本地专家的权重": a rank holds its local experts only).
 *   pair p = t * topk + j is token t's j-th chosen expert e = topk_ids[p];
 *   its local id is expert_map[e] when a map is given (-1: held by another
 *   rank), e itself otherwise;
 *   key = slot(t) * E_local + local id, or -1 when the token has no adapter
 *   or the expert is not local, or -2 when an id is out of range (a slot
 *   outside [-1, S), an expert outside [0, E_global), a local id outside
 *   [-1, E_local), or without a map an expert >= E_local).
 */
int oracle_moe_keys(const int32_t *topk_ids, int64_t T, int32_t topk,
                    const int32_t *token_slot, int32_t S, int32_t E_global,
                    int32_t E_local, const int32_t *expert_map,
                    int32_t *keys)
{
    if (T < 0 || topk < 1 || S < 1 || E_global < 1 || E_local < 1)
        return ORACLE_BAD_ARG;
    for (int64_t t = 0; t < T; ++t) {
        const int32_t slot = token_slot[t];
        for (int32_t j = 0; j < topk; ++j) {
            const int32_t e = topk_ids[t * topk + j];
            int32_t key;
            if (slot < -1 || slot >= S || e < 0 || e >= E_global) {
                key = -2;
            } else {
                int32_t local;
                if (expert_map)
                    local = expert_map[e];
                else
                    local = e < E_local ? e : -2;
                if (local < -1 || local >= E_local)
                    key = -2;
                else if (slot == -1 || local == -1)
                    key = -1;
                else
                    key = slot * E_local + local;
            }
            keys[t * topk + j] = key;
        }
    }
    return ORACLE_OK;
}
