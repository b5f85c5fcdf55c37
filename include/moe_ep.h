/*
 * moe_ep.h -- MoE token dispatch and combine on one MI355X (gfx950).
 *
 * C ABI. Every tensor argument is a plain DEVICE pointer to row-major,
 * densely packed memory that the caller allocated and owns; sizes are plain
 * integers; the stream is a hipStream_t passed as void* (NULL = the default
 * stream). The library never allocates, frees or synchronises: a call
 * validates its arguments on the host, enqueues its kernels on `stream` and
 * returns. MOE_OK means "validated and enqueued". On any error status no
 * kernel has been launched and no output has been touched. The library keeps
 * no mutable global state, so calls on different streams are independent;
 * calls that share a workspace must be ordered by the caller.
 *
 * Notation: W = ep_world (logical expert-parallel ranks), bs = tokens per
 * rank, N = W*bs, K = topk, epr = experts_per_rank, E = W*epr experts,
 * S = epr*W segments per rank, ROWS = N*K. Token t = s*bs + tok belongs to
 * source rank s. Expert e lives on rank r = e / epr as local expert
 * el = e % epr. The logical ranks' receive windows are back-to-back
 * partitions of one expand_x buffer, rank 0 first.
 *
 * Pages this interface follows:
 *  - "aclnnMoeDistributeDispatchV4" (CANN 9.1.0-beta.3 API reference):
 *    接口功能 and 计算公式 (optional quantisation, then the expert-parallel
 *    all-to-all expandXOut = AllToAllV(X)); the two-phase call (a workspace
 *    query that validates, then the execution); the aclnnStatus return code;
 *    parameter ranges (epWorldSize in [2, 768], moeExpertNum in (0, 1024],
 *    quantMode 0 or 2 on the A2/A3 parts, 0 to 4 on another part); 约束说明:
 *    deterministic by default, dispatch outputs are handed to combine
 *    unchanged and are opaque to the caller, and scalar parameters must match
 *    between dispatch and combine.
 *  - "双平面 MoE Combine 示例" (CANN SHMEM combine_doubleplane README):
 *    功能说明 (expand_x grouped by expert; assist_info_for_combine rows
 *    [src_rank_id, src_token_id, src_topk_id]; ep_recv_count, the cumulative
 *    receive count per (local_expert_id, src_rank_id) segment; the combine
 *    check formula) and 方案设计 (the large-segment predicate).
 */
#ifndef MOE_EP_H
#define MOE_EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (the two-phase API of aclnnMoeDistributeDispatchV4 returns a
 * status and validates in its first phase). */
enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULLPTR = 1,   /* a required pointer is NULL, or a forbidden one is not */
    MOE_ERR_SHAPE = 2,     /* a size is out of range or a product overflows */
    MOE_ERR_DTYPE = 3,     /* unknown token dtype */
    MOE_ERR_QUANT = 4,     /* unknown quant mode, quantisation of int32 data, a shape the
                              static or per-group quantiser does not take, or a static
                              coefficient count other than 1, h or E*h */
    MOE_ERR_WORKSPACE = 5, /* workspace smaller than the queried size */
    MOE_ERR_LAUNCH = 6,    /* the HIP runtime refused a launch (a call reads and clears HIP's
                              last-error state before its launches, so an earlier error that
                              the caller has not collected is not reported as this one) */
    MOE_ERR_SCHEDULE = 7,  /* unknown schedule mode, or the segment schedule (or the
                              segment_is_large output) at W*S above 11264 */
    MOE_ERR_ALIGN = 8,     /* a pointer is not aligned to its element size (16 bytes for
                              the workspace, and for the inputs moe_quant lists under
                              quant modes 1 and 3) */
    MOE_ERR_MASK = 9       /* unknown mask kind, or a mask pointer that does not match it */
};

/* Token element types. */
enum moe_dtype { MOE_INT32 = 0, MOE_FP16 = 1, MOE_BF16 = 2 };

/* Quantisation modes; the numbering follows quantMode of
 * aclnnMoeDistributeDispatchV4 (0 = none, 1 = static, 2 = per-token dynamic,
 * 3 = per-group dynamic, 4 = mx).
 *  MOE_QUANT_STATIC: int8 codes rint(x * c) of the exact product, ties to
 *      even, saturated to [-128, 127] (a NaN product gives -128). c
 *      comes from quant_scales (fp32, caller-owned device memory): one value,
 *      one per column (h values), or one per expert and column (E*h values,
 *      row e for the rows of expert e) -- the three shapes the page's 参数说明
 *      gives the static coefficient input (one coefficient, a smoothing vector
 *      shared by the experts, per-expert coefficients fused with smoothing);
 *      its formula is garbled, and multiplying is the reading taken. No
 *      dynamic_scales. Needs h % 16 == 0, h <= 16384, topk <= 64, 16-byte
 *      aligned x, expand_x and (for h or E*h values) quant_scales, and a
 *      token-major schedule (not MOE_SCHED_SEGMENT; the adaptive one runs
 *      this mode token-major).
 *  MOE_QUANT_DYN_TOKEN: int8 codes rint(x / s), s = max|x| / 127 over the token;
 *      dynamic_scales holds one fp32 scale per row.
 *  MOE_QUANT_DYN_GROUP: OCP FP8 E4M3 ("fn") codes per group of 128 elements of
 *      h (the last group may be shorter): s = max|x| / 448 over the group, code
 *      = E4M3 nearest to RN(x / s) clamped to +-448, ties to even, sign of x
 *      kept; an all-zero group has s = 0 and codes 0. dynamic_scales is fp32
 *      [ROWS, ceil(h/128)]. (The pages list the mode; its output types and group
 *      size are garbled, and these are the readings taken.) Needs h % 16 == 0,
 *      h <= 16384, topk <= 64, 16-byte aligned x and expand_x, and a
 *      token-major schedule (not MOE_SCHED_SEGMENT; the adaptive one runs
 *      this mode token-major).
 *  MOE_QUANT_MX: the OCP Microscaling (MX v1.0) format with E4M3 elements
 *      (MXFP8), per block of 32 elements of h (the last block may be shorter):
 *      shared = floor(log2 max|x|) - 8 over the block, clamped to [-127, 127]
 *      (-127 for an all-zero block); code = E4M3 nearest to x * 2^-shared
 *      clamped to +-448, ties to even, sign of x kept (-0 gives 0x80).
 *      dynamic_scales is uint8 [ROWS, ceil(h/32)], one E8M0 byte shared + 127
 *      per block (the scale 2^(byte - 127)); any alignment. (The page lists mx
 *      quantisation with four output types, no scale input and a garbled
 *      scale shape; E4M3 elements are the reading taken, and the other three
 *      types are not provided.) Inputs must be finite. Same limits as
 *      MOE_QUANT_DYN_GROUP. */
enum moe_quant {
    MOE_QUANT_NONE = 0, MOE_QUANT_STATIC = 1, MOE_QUANT_DYN_TOKEN = 2, MOE_QUANT_DYN_GROUP = 3, MOE_QUANT_MX = 4
};

/* Token masks: xActiveMaskOptional of aclnnMoeDistributeDispatchV4 (参数说明):
 * a 1D mask (BS,) per rank or a 2D mask (BS, K); a token whose K entries are
 * all false is not exchanged. Here the mask covers all W*bs tokens, one byte
 * per entry, nonzero = active (a torch.bool tensor qualifies):
 *  MOE_MASK_NONE:  every pair takes part; the mask pointer must be NULL.
 *  MOE_MASK_TOKEN: uint8 [N]; an inactive token sends none of its K pairs.
 *                  The pages ask each rank's active tokens to come first;
 *                  any pattern is accepted here.
 *  MOE_MASK_PAIR:  uint8 [N, K]; pair (t, k) is sent iff its byte is nonzero.
 * An inactive pair gets no row and no count, and its expert id is ignored (a
 * kernel may load it together with the mask byte; its value never matters).
 * The A active pairs fill expand_x rows 0..A-1 in the usual order, with
 * A = sum over ranks r of ep_recv_count[r][S-1]; later rows of the N*K-row
 * buffers are left untouched. Dispatch and combine take the same mask. */
enum moe_mask { MOE_MASK_NONE = 0, MOE_MASK_TOKEN = 1, MOE_MASK_PAIR = 2 };

/* Special experts: zeroExpertNum / copyExpertNum / constExpertNum of
 * aclnnMoeDistributeDispatchV4 (参数说明), id ranges after the E real experts:
 * zero experts [E, E + zero), copy experts [E + zero, E + zero + copy), const
 * experts [E + zero + copy, E + zero + copy + const). The pages give only the
 * ranges; here a pair routed to a special expert is not exchanged (no row, no
 * count, like an inactive pair), and in the combine, at the pair's place in
 * the k order, a zero expert adds nothing, a copy expert adds ori_x[t] * weight
 * and const expert j adds const_x[j] * weight (a const expert's output is one
 * fixed vector, the same for every token). Pass NULL for none.
 *  ori_x:   DEVICE [N, h], the tokens given to dispatch, in the combine's dtype;
 *           read by moe_combine when copy_expert_num > 0, ignored by dispatch.
 *  const_x: DEVICE [const_expert_num, h] in the combine's dtype, caller-owned;
 *           read by moe_combine when const_expert_num > 0, ignored by dispatch.
 * The counts are >= 0 and E + zero + copy + const < 2^31 (else MOE_ERR_SHAPE). */
typedef struct moe_special_experts {
    int32_t zero_expert_num;
    int32_t copy_expert_num;
    int32_t const_expert_num;
    int32_t reserved;
    const void *ori_x;
    const void *const_x;
} moe_special_experts;

/* How dispatch assigns its payload copies to workgroups. Both modes produce
 * bitwise identical outputs (the combine_doubleplane README requires the same
 * x_out whichever return path a segment takes).
 *  MOE_SCHED_TOKEN:   one workgroup per source token reads the row once and
 *                     writes its K copies; the predicate is not consulted.
 *  MOE_SCHED_SEGMENT: workgroups walk expand_x in destination order; a segment
 *                     selected by the large-segment predicate gets whole
 *                     workgroups of its own (split by rows), the other
 *                     segments are packed together. Each token row is then
 *                     read once per destination row rather than once, so
 *                     this mode is slower (16 ranks x 256 bf16 tokens of
 *                     7168, int8: 132 us per dispatch against 50 us).
 *  MOE_SCHED_ADAPTIVE (the default when schedule is NULL): the token
 *                     schedule for every segment the predicate does not
 *                     select; the token-major pass leaves out the rows of
 *                     the selected segments, and a second pass writes them
 *                     in windows of 8 consecutive expand_x rows, each window
 *                     by a wavefront of its own (each such row reads its
 *                     token once more). A segment holds at most bs rows (ids
 *                     are distinct per token), so when bs*h*elem_bytes < T no
 *                     segment can be selected and this mode runs exactly the
 *                     token schedule; with the README's 2 MiB that holds at
 *                     16 ranks x 256 tokens of 7168 int8. It covers copies
 *                     and per-token int8 (quant_mode 0 and 2); the other
 *                     quant modes take the token schedule. */
enum moe_sched_mode { MOE_SCHED_TOKEN = 0, MOE_SCHED_SEGMENT = 1, MOE_SCHED_ADAPTIVE = 2 };

/* Optional dispatch schedule (host struct; pass NULL for the defaults:
 * MOE_SCHED_ADAPTIVE with the README's 2 MiB).
 *  mode: a moe_sched_mode.
 *  large_segment_bytes: threshold T of the predicate (README 方案设计): a
 *      segment (el, s) of rank r is large iff s != r, it is non-empty, its
 *      payload count*h*elem_bytes is >= T, and count*h*elem_bytes*den > num
 *      with num = (rows r receives from other ranks)*h*elem_bytes and
 *      den = max(W-1, 1)*epr (64-bit integers). elem_bytes is the size of an
 *      expand_x element (1 when quantising). A negative value selects the
 *      README's 2 MiB.
 *  segment_is_large: optional DEVICE output, int32 [W, S] in ep_recv_count's
 *      layout, set to 1 for the selected segments and 0 otherwise. */
typedef struct moe_schedule {
    int32_t mode;
    int32_t reserved;
    int64_t large_segment_bytes;
    int32_t *segment_is_large;
} moe_schedule;

/* Phase one of dispatch: validates the scalars and writes the workspace size
 * (bytes, host pointer) that moe_dispatch needs for them. */
int moe_dispatch_workspace_size(int ep_world, int bs, int experts_per_rank, int h, int topk,
                                int dtype, int quant_mode, size_t *bytes);

/*
 * Dispatch: the expert-parallel all-to-all of aclnnMoeDistributeDispatchV4
 * (计算公式, expandXOut = AllToAllV(X)) with every logical rank's window in
 * one HBM, preceded by optional quantisation (static int8, per-token dynamic
 * int8 or per-group dynamic FP8 E4M3).
 *
 *  x              [N, h] dtype           tokens; rows s*bs..s*bs+bs-1 are rank s's
 *  expert_ids     [N, K] int32           global expert ids in [0, E), distinct per token
 *                                        (inactive pairs' ids are ignored)
 *  expert_scales  [N, K] 4-byte or NULL  only read when expand_scales is given
 *  x_active_mask  uint8 [N] or [N, K]    see moe_mask; NULL with MOE_MASK_NONE
 *  mask_kind      moe_mask
 *  special        host pointer or NULL   see moe_special_experts; ids in the special
 *                                        ranges are legal and produce no row
 *  quant_scales   fp32 [quant_scales_numel]  quant_mode 1 only (NULL and 0 otherwise):
 *                                        1, h or E*h coefficients, see MOE_QUANT_STATIC
 *  expand_x       [ROWS, h]              dtype; int8 when quant_mode is 1 or 2, E4M3 bytes when 3 or 4. Row order:
 *                                        rank r, then local expert, then source rank,
 *                                        then ascending source token
 *  dynamic_scales [ROWS] fp32            per-row token scale max|x|/127 (quant_mode 2),
 *                 [ROWS, ceil(h/128)]    per-group fp32 scales max|x|/448 (quant_mode 3), or
 *                 [ROWS, ceil(h/32)]     uint8 E8M0 block scale bytes (quant_mode 4);
 *                                        required for quant_mode 2, 3 and 4, NULL otherwise
 *  assist_info    [ROWS, 3] int32        (src_rank, src_token, topk_id) of each row
 *  ep_recv_count  [W, S] int32           per rank, inclusive prefix of the row counts of
 *                                        its segments ordered el*W + s
 *  expand_scales  [ROWS] 4-byte or NULL  expert_scales[t, k] moved to row(t, k)
 *  schedule       host pointer or NULL   see moe_schedule
 *  workspace      device scratch of at least the queried size; its contents on
 *                 entry do not matter
 *
 * Ranges: ep_world in [2, 768], experts_per_rank >= 1, E <= 1024,
 * 1 <= topk <= E, bs >= 0 (bs == 0 writes zero counts and nothing else),
 * h >= 1, N*K < 2^31, N < 2^24, N*ceil(h/128) < 2^25, E + special experts < 2^31.
 * Active ids outside [0, E + zero + copy + const) or repeated within a token
 * are a precondition violation: the kernels stay in bounds but the outputs are
 * unspecified. Outputs are bitwise deterministic.
 * Copies of up to 4096 (token, expert) pairs with rows in 16-byte pieces and
 * topk <= 16 run as one kernel, which counts each pair's row in the workgroup
 * that writes it; other calls launch the route kernel first. Both give the same
 * outputs; the workspace is required either way.
 */
int moe_dispatch(const void *x, const int32_t *expert_ids, const void *expert_scales,
                 const uint8_t *x_active_mask, int mask_kind, const moe_special_experts *special,
                 int ep_world, int bs, int experts_per_rank, int h, int topk, int dtype,
                 int quant_mode, const float *quant_scales, int64_t quant_scales_numel,
                 void *expand_x, void *dynamic_scales, int32_t *assist_info,
                 int32_t *ep_recv_count, void *expand_scales, const moe_schedule *schedule,
                 void *workspace, size_t workspace_bytes, void *stream);

/* Scratch of moe_dispatch_noalloc, per GPU (bytes). */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * Dispatch without a workspace argument, for callers that cannot allocate:
 * code under HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc. Same arguments, outputs and validation as moe_dispatch, less the
 * workspace. It allocates nothing: its scratch is a file-scope device array of
 * MOE_NOALLOC_SCRATCH_BYTES (32 MiB) that each GPU the library runs on holds
 * until the process ends; its address on the current device (hipGetDevice) is
 * looked up on the first call there, and `stream` must belong to that device.
 * A shape whose moe_dispatch_workspace_size exceeds the scratch returns
 * MOE_ERR_WORKSPACE before anything is launched (16 ranks x 256 tokens, top-8,
 * needs about 0.3 MiB; the limit lies near 6 million (token, expert) pairs);
 * a failed lookup returns MOE_ERR_LAUNCH. Every call on one GPU shares that
 * GPU's array, which keeps the last call's contents (none of which a call
 * needs to find zeroed): calls that overlap on one GPU, on different streams
 * or host threads, race and must be ordered by the caller.
 */
int moe_dispatch_noalloc(const void *x, const int32_t *expert_ids, const void *expert_scales,
                         const uint8_t *x_active_mask, int mask_kind, const moe_special_experts *special,
                         int ep_world, int bs, int experts_per_rank, int h, int topk, int dtype,
                         int quant_mode, const float *quant_scales, int64_t quant_scales_numel,
                         void *expand_x, void *dynamic_scales, int32_t *assist_info,
                         int32_t *ep_recv_count, void *expand_scales, const moe_schedule *schedule,
                         void *stream);

/* Phase one of combine: validates the scalars and writes the workspace size
 * (N*K int32 slots, rounded up to 256 bytes). */
int moe_combine_workspace_size(int ep_world, int bs, int experts_per_rank, int h, int topk,
                               int dtype, size_t *bytes);

/*
 * Combine (README 功能说明, check formula):
 *   x_out[t] = sum_k expand_x[row(t, k)] * expert_scales[t, k]
 * where row(t, k) is the row dispatch gave to pair (t, k). As in the README's
 * 实现逻辑, every expand_x row is returned to its source: row i goes to slot
 * (src_token, topk_id) of rank src_rank as named by assist_info[i]; on one
 * GPU only the row index travels (into the workspace) and the source's
 * weighted sum gathers the rows through those slots.
 * fp16/bf16: accumulated in fp32, one fused multiply-add per k with k
 * ascending from 0.0f, rounded once to nearest-even; int32: wrapping 32-bit
 * integer arithmetic.
 *
 *  expand_x       [ROWS, h] dtype (fp16, bf16 or int32; the expert outputs)
 *  assist_info    [ROWS, 3]: dispatch's, unchanged
 *  ep_recv_count  [W, S]: dispatch's, unchanged (the slot pass locates rows through
 *                 assist_info; the one-launch combine reads segment starts from here)
 *  expert_ids     [N, K] int32: the ids given to dispatch (checked likewise)
 *  expert_scales  [N, K] fp32 for fp16/bf16, int32 for int32 data
 *  x_active_mask, mask_kind: the dispatch's. The sum then runs over the
 *                 active pairs only (k ascending); a token with none gets 0.
 *  special        the dispatch's (NULL for none); needs ori_x when copy experts
 *                 exist and const_x when const experts exist. With a mask or
 *                 special experts, ep_recv_count is read to find the row total.
 *  x_out          [N, h] dtype
 *  workspace      device scratch of at least the queried size
 * The scalars must equal those given to dispatch. Rows that assist_info does
 * not name leave their slot undefined; the kernels stay in bounds but the
 * affected outputs are unspecified. Up to 1024 pairs per source rank (bs*K),
 * fewer than 2^16 pairs in all, rows in 16-byte pieces and topk <= 16, the
 * combine is one kernel that finds each pair's row from ep_recv_count (its
 * segment's start) and the source's earlier expert ids, instead of a slot pass
 * over assist_info; the outputs are the same.
 */
int moe_combine(const void *expand_x, const int32_t *assist_info, const int32_t *ep_recv_count,
                const int32_t *expert_ids, const void *expert_scales,
                const uint8_t *x_active_mask, int mask_kind, const moe_special_experts *special,
                int ep_world, int bs,
                int experts_per_rank, int h, int topk, int dtype, void *x_out,
                void *workspace, size_t workspace_bytes, void *stream);

/* A static, human-readable name for a status code. */
const char *moe_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EP_H */
