/*
 * ep.h -- C ABI of the one-GPU MoE expert-parallel layout / dispatch / combine library (libep_mi355x.so).
 *
 * The library computes, on one GPU (gfx950, MI355X), the data-parallel share of DeepEP-style expert-parallel
 * dispatch and combine:
 *   ep_get_layout  routing table -> per-expert / per-rank counts, token-in-rank membership, aligned
 *                  per-expert row starts, and the slot of every routed entry (kept in a handle);
 *   ep_dispatch    permute token rows into an expert-major, alignment-padded receive buffer (or, without
 *                  expansion, one token-major row per token), optionally cast to FP8 e4m3 with
 *                  per-128-channel fp32 scales, and pack per-destination send windows for experts owned by
 *                  other ranks;
 *   ep_combine     weighted top-k reduction of expert outputs back to token order in BF16, plus bias
 *                  (ep_combine_tokens for the token-major rows);
 *   ep_dispatch_rows / ep_combine_reduce  the receiver's placement of rows that arrived from other ranks and
 *                  the source's sum of the rows those ranks return (the two ends of the exchange);
 *   ep_layout_dispatch  ep_get_layout + ep_dispatch in one call, one kernel launch for <= 256 tokens.
 *
 * Page names used in the citations:
 *   [DeepEP->MegaMoE]  "从 DeepEP 到 Mega MoE：MoE Runtime 演进的三向验证分析" (backyes.github.io)
 *   [DeepEP-hotdry]    DeepEP expert-parallel communication article (blog.hotdry.top)
 *   [MoE-comm]         "MoE 为什么容易卡在通信上？" (locsic.com)
 *   [flops-record]     inference-research record "deepep-expert-parallel-dispatch-combine" (phantomic12)
 *   [repo-map]         "第 2 章 仓库地图与模块职责" (bowenzhou.top)
 *
 * Conventions for every call:
 *   - Device pointers are plain device addresses (hipMalloc / torch CUDA tensors); host pointers are named.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default stream).  No call allocates device
 *     memory, copies to the host or synchronises: counts stay on the device, as with do_cpu_sync off
 *     ([MoE-comm] §二; [flops-record]: capacity-sized outputs and a device psum for the grouped GEMM).
 *   - Every argument is validated on the host before anything is enqueued.  On a validation error nothing is
 *     enqueued, no output is touched, the call returns EP_ERR_INVALID_ARG and ep_last_error() describes it.
 *     A failed launch returns EP_ERR_HIP; kernels of the same call enqueued before it may have run.
 *   - Memory is owned by the caller.  A buffer or handle must not be freed, resized or reused while an
 *     operation using it is still pending on its stream ([MoE-comm] §二, buffer and handle reuse).
 *   - Row-major layouts throughout.  x, y, out, bias, recv_x and send_x must be 16-byte aligned.
 *
 * Limits: 0 <= num_tokens; 1 <= num_topk <= 32; 1 <= num_experts <= 1024; 1 <= num_ranks <= 64 with
 * num_experts % num_ranks == 0; 0 <= rank < num_ranks; 1 <= expert_alignment <= 65536; the receive capacity
 * must fit in int32, and so must num_tokens * num_ranks (the send-window rows); hidden % 8 == 0,
 * 8 <= hidden <= 32768, and hidden % 128 == 0 for FP8.
 *
 * Handles: every call that takes a handle first looks it up among the live handles (created and not yet freed)
 * and returns EP_ERR_INVALID_ARG for any other pointer without reading through it, so a handle freed twice or
 * used after ep_handle_free is an error, not undefined behaviour.  (A stale pointer that the host allocator has
 * since reused for a new handle refers to that new handle.)  Freeing a handle while another thread is inside a
 * call with it is a caller error, like freeing any buffer an operation still uses ([MoE-comm] §二).
 */
#ifndef EP_MI355X_H
#define EP_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ep_status {
    EP_OK = 0,
    EP_ERR_INVALID_ARG = 1,   /* an argument is out of range, misaligned, NULL where required, or a size is short */
    EP_ERR_UNSUPPORTED = 2,   /* a mode this version does not implement (none at present; reserved)               */
    EP_ERR_HIP = 3            /* a HIP launch failed; the stream state is whatever HIP reports                    */
} ep_status_t;

typedef enum ep_dtype {
    EP_DTYPE_BF16 = 0,        /* bf16 rows, bit copies of x                                                        */
    EP_DTYPE_FP8_E4M3 = 1     /* OCP e4m3fn rows + one fp32 scale per 128 channels                                 */
} ep_dtype_t;

typedef struct ep_handle* ep_handle_t;   /* opaque host object created by ep_get_layout / ep_layout_dispatch */

/* Rows the expert-major receive buffers (recv_x and friends, and y of ep_combine) must have:
 * num_tokens * num_topk + num_local_experts * (expert_alignment - 1), the worst case of padding every local
 * expert up to a multiple of the alignment ([flops-record]: outputs sized to configured capacity; [MoE-comm]
 * §一: equal, fixed capacity).  Host only.  Returns -1 for arguments outside the limits. */
int64_t ep_recv_capacity(int num_tokens, int num_topk, int num_local_experts, int expert_alignment);

/* Library helper (no page defines it; it sizes the caller-owned scratch that replaces DeepEP's internal
 * buffers, [MoE-comm] §一: buffers are sized once from the capacity and reused).  Bytes of device workspace
 * ep_get_layout needs for these sizes.  Host only.  Returns 0 for arguments outside the limits (a valid call
 * always needs more than 0 bytes). */
size_t ep_layout_workspace_bytes(int num_tokens, int num_topk, int num_experts, int num_ranks, int expert_alignment);

/* Library helpers (no page defines them; the C ABI's replacement for the exceptions a Python API raises on a
 * failed pre-launch check, [repo-map] §2.1: the runtime validates arguments before launching).  A static
 * description of a status code, and a thread-local description of the last failure in this thread ("" after a
 * successful call). */
const char* ep_status_string(ep_status_t status);
const char* ep_last_error(void);

/*
 * ep_get_layout -- layout of one rank's routing table ([repo-map] §2.1: layout.cu reduces top-k indices to
 * rank counts, expert counts and token-in-rank membership; [DeepEP->MegaMoE] §2.2: per-expert counts and
 * their prefix sum; §2.4: the prefix sum is the start cursor of each expert's rows).
 *
 *   topk_idx             device, int64 [num_tokens, num_topk]: expert of each routed entry; -1 = unused.
 *                        Entries < -1 or >= num_experts are dropped and counted in num_invalid_topk.
 *                        The handle keeps this pointer: keep the array alive and unchanged while the
 *                        handle is used.
 *   num_experts          global expert count E; expert e belongs to rank e / (E / num_ranks).
 *   num_ranks, rank      EP group size and this rank.
 *   expert_alignment     A: every local expert's segment starts at and spans a multiple of A rows
 *                        ([MoE-comm] §一 expert_alignment; §三 padding).  An empty expert spans 0 rows.
 *   workspace            device scratch of at least ep_layout_workspace_bytes(...) bytes, 256-byte aligned,
 *                        owned by the caller; the handle keeps the slot map in it, so it must outlive every
 *                        dispatch/combine that uses the handle.  No initial contents are required.
 *   num_tokens_per_rank  device int32 [num_ranks] out, nullable: tokens with >= 1 expert on rank r
 *                        (a token counts once per rank).
 *   num_tokens_per_expert device int32 [num_experts] out, nullable: routed entries per expert.
 *   is_token_in_rank     device uint8 [num_tokens, num_ranks] out, nullable: 0/1 membership.
 *   psum_num_recv_tokens_per_expert  device int32 [num_experts / num_ranks + 1] out, nullable: aligned
 *                        exclusive row starts of the local experts, psum[0] = 0; local expert j owns rows
 *                        [psum[j], psum[j+1]) of which the first num_tokens_per_expert[rank*El + j] are valid.
 *   num_invalid_topk     device int32 [1] out, nullable.
 *   handle_out           host out: a new handle (free with ep_handle_free).  Rows of one expert are ordered
 *                        by ascending flat entry index t * num_topk + k.  The handle also ranks, for every
 *                        rank r, the tokens with an expert on r in ascending token order: the row of the
 *                        token in the send window of r (r != rank), or in the token-major receive rows
 *                        (r == rank, dispatch with do_expand = 0).
 */
ep_status_t ep_get_layout(const int64_t* topk_idx, int num_tokens, int num_topk, int num_experts, int num_ranks,
                          int rank, int expert_alignment, void* workspace, size_t workspace_bytes,
                          int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                          int32_t* psum_num_recv_tokens_per_expert, int32_t* num_invalid_topk,
                          ep_handle_t* handle_out, void* stream);

/* Outputs of ep_dispatch.  All device memory owned by the caller; NULL = not requested where allowed.
 * "rows" is recv_capacity.  Expert-major (do_expand = 1) and token-major (do_expand = 0) shapes differ where
 * noted. */
typedef struct ep_dispatch_out {
    void*    recv_x;            /* required: [rows, hidden] e4m3 bytes (FP8) or bf16 (BF16)                     */
    float*   recv_x_scales;     /* FP8: required, [rows, hidden / 128] fp32 scales; BF16: ignored                */
    int32_t* recv_src_idx;      /* nullable: [rows] source token of each row; -1 on padding rows                 */
    float*   recv_topk_weights; /* nullable: expert-major [rows] routing weight of each row, 0 on padding rows;
                                   token-major [num_tokens, num_topk] the token's weights                         */
    int64_t* recv_topk_idx;     /* token-major only, nullable: [num_tokens, num_topk] expert id local to this
                                   rank, -1 where another rank owns the entry's expert; ignored otherwise         */
    int64_t  recv_capacity;     /* rows allocated in the recv arrays: >= ep_recv_capacity(...) (expert-major),
                                   >= num_tokens (token-major)                                                    */
    void*    send_x;            /* num_ranks > 1: required, [num_ranks, num_tokens, hidden] rows (window per rank)*/
    float*   send_x_scales;     /* num_ranks > 1 and FP8: required, [num_ranks, num_tokens, hidden / 128]        */
    int32_t* send_src_idx;      /* nullable: [num_ranks, num_tokens] source token of each window row            */
    int64_t* send_topk_idx;     /* nullable: [num_ranks, num_tokens, num_topk] expert id local to the window's
                                   rank, -1 where that rank does not own the entry's expert                       */
    float*   send_topk_weights; /* nullable: [num_ranks, num_tokens, num_topk] routing weights                   */
} ep_dispatch_out_t;

/*
 * ep_dispatch -- expert-major dispatch of this rank's tokens ([MoE-comm] §一 dispatch arguments;
 * [DeepEP->MegaMoE] §2.2 dispatch kernel: read the token row, store to the send buffer; §2.4 copy epilogue:
 * place rows expert-major; [DeepEP-hotdry] key techniques: FP8 dispatch, BF16 combine).
 *
 *   handle          from ep_get_layout; may be reused for any number of dispatches with new x ("cached" use).
 *   x               device bf16 [num_tokens, hidden], read once per token.
 *   topk_weights    device fp32 [num_tokens, num_topk], nullable (weights of 1); copied into
 *                   recv_topk_weights and send_topk_weights only.
 *   recv_dtype      EP_DTYPE_BF16 or EP_DTYPE_FP8_E4M3.  FP8: per token and 128-channel group,
 *                   a = max(max|x|, 1e-4), scale = a / 448, q = e4m3_rne_saturating(x * (448 / a)).
 *                   x must be finite for FP8: the codes and the scale of a group holding a NaN or an infinity
 *                   are unspecified (no page defines them); the token's other groups and all other rows are
 *                   unaffected.  BF16 rows are bit copies whatever they hold.
 *   do_expand       1: expert-major rows, one per routed entry, at the rows of the layout.
 *                   0: token-major rows ([MoE-comm] §一 dispatch arguments, do_expand): one row per token
 *                   with an expert on this rank, in ascending token order (row j = the j-th such token),
 *                   with recv_src_idx = the token, recv_topk_idx / recv_topk_weights its K entries; no
 *                   padding; rows past num_tokens_per_rank[rank] are untouched.  The expert computation
 *                   then returns one row per token, moved back by ep_combine_tokens.
 *   do_zero_padding expert-major only.  1: padding rows [psum[j] + count_j, psum[j+1]) get zero bytes and
 *                   zero scales; 0: their data bytes and scales are left untouched.  Their recv_src_idx /
 *                   weights are written (-1 / 0) either way.  Rows >= psum[El] are never written.
 *   Send windows (num_ranks > 1): for every other rank r, row j of window r holds the j-th token (ascending)
 *   with an expert on r: the same bytes and scales as the token's local rows.  Rows past the window's count
 *   are untouched; window `rank` is untouched.
 */
ep_status_t ep_dispatch(ep_handle_t handle, const void* x, int hidden, const float* topk_weights,
                        ep_dtype_t recv_dtype, int do_expand, int do_zero_padding, const ep_dispatch_out_t* out,
                        void* stream);

/*
 * ep_layout_dispatch -- ep_get_layout and ep_dispatch in one call: the same arguments, the same outputs and the
 * same handle, bit for bit.  For num_tokens <= 256 (the decode shape) both run in a single kernel launch:
 * workgroup t counts in LDS what token t's rows follow from and dispatches token t, so no workgroup waits for another
 * ([DeepEP->MegaMoE] §4.3: at small batches launch overhead, not bytes, sets the time; [DeepEP-hotdry]
 * 性能基准: the low-latency decode path).  Larger batches run the layout and the dispatch launches back to
 * back.  x is only read, as by ep_dispatch.
 *
 *   Arguments as in ep_get_layout (topk_idx .. num_invalid_topk, handle_out) and ep_dispatch (x .. out).
 *   Every argument of both is validated before anything is enqueued; on an error no handle is created.
 *   The handle is reusable afterwards exactly like one from ep_get_layout.
 */
ep_status_t ep_layout_dispatch(const int64_t* topk_idx, int num_tokens, int num_topk, int num_experts, int num_ranks,
                               int rank, int expert_alignment, void* workspace, size_t workspace_bytes,
                               int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                               uint8_t* is_token_in_rank, int32_t* psum_num_recv_tokens_per_expert,
                               int32_t* num_invalid_topk, const void* x, int hidden, const float* topk_weights,
                               ep_dtype_t recv_dtype, int do_expand, int do_zero_padding,
                               const ep_dispatch_out_t* out, ep_handle_t* handle_out, void* stream);

/*
 * ep_layout_dispatch_noalloc -- ep_layout_dispatch for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, and harnesses that forbid device allocation.  The same arguments without the workspace,
 * the same outputs bit for bit.  It calls no device or host allocator: the layout workspace is a static device
 * array of 4 MiB in this library (one copy per GPU, held until the process ends), and the handle is a static
 * per-GPU object.  Set-up on the first call on a GPU (with that GPU current) looks up that GPU's copy of the
 * array; make that first call outside any graph capture.
 *
 *   Limit: sizes whose workspace (ep_layout_workspace_bytes) exceeds 4 MiB are rejected with
 *   EP_ERR_INVALID_ARG before anything is enqueued (about 100,000 tokens at top-8 with 256 experts and
 *   alignment 128).  Every byte of the array that the kernels read is written earlier in the same call, so no
 *   contents need clearing between calls.
 *   Sharing: every call on a GPU uses that GPU's one array and one handle.  The returned handle is valid for
 *   ep_dispatch / ep_combine / ep_combine_tokens / ep_combine_reduce until the next ep_layout_dispatch_noalloc
 *   on the same GPU, which overwrites both (a handle kept from an earlier call then refers to the new layout).
 *   Calls that overlap on one GPU -- from two host threads, or a new call enqueued on another stream while
 *   kernels of an earlier call or of its handle's dispatch / combine may still run -- race on the array.
 *   ep_handle_free on this handle is a no-op returning EP_OK.
 */
ep_status_t ep_layout_dispatch_noalloc(const int64_t* topk_idx, int num_tokens, int num_topk, int num_experts,
                                       int num_ranks, int rank, int expert_alignment, int32_t* num_tokens_per_rank,
                                       int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                                       int32_t* psum_num_recv_tokens_per_expert, int32_t* num_invalid_topk,
                                       const void* x, int hidden, const float* topk_weights, ep_dtype_t recv_dtype,
                                       int do_expand, int do_zero_padding, const ep_dispatch_out_t* out,
                                       ep_handle_t* handle_out, void* stream);

/*
 * ep_dispatch_rows -- the receiver's copy epilogue ([DeepEP->MegaMoE] §2.4: rows that arrived
 * destination-major are placed expert-major, each at its expert's rows).  Rows already carry their receive
 * format (the bytes and scales of a sender's send window), so nothing is converted.
 *
 *   handle          from ep_get_layout over the received rows' expert ids: topk_idx [N, K] holding ids
 *                   local to this rank (0..E_local-1, e.g. a window's send_topk_idx) or -1, with
 *                   num_experts = E_local and num_ranks = 1.  Rows that were not received are all -1.
 *   rows            device [N, row_bytes] bytes, 16-byte aligned; row_bytes % 16 == 0, <= 65536.
 *   row_scales      device fp32 [N, num_scales] (nullable when num_scales == 0), copied with each row.
 *   topk_weights    device fp32 [N, K], nullable (weights of 1): recv_topk_weights of the placed rows.
 *   do_zero_padding as in ep_dispatch.
 *   out             recv_x [recv_capacity, row_bytes], recv_x_scales [recv_capacity, num_scales] (required iff
 *                   num_scales > 0), recv_src_idx = index of the received row (-1 on padding rows),
 *                   recv_topk_weights; send fields are ignored.
 */
ep_status_t ep_dispatch_rows(ep_handle_t handle, const void* rows, int row_bytes, const float* row_scales,
                             int num_scales, const float* topk_weights, int do_zero_padding,
                             const ep_dispatch_out_t* out, void* stream);

/*
 * ep_combine -- top-k reduction back to token order ([DeepEP->MegaMoE] §2.3 and §2.5: element-wise
 * accumulation of the top-k expert outputs of a token; [MoE-comm] §一: the shared expert's output joins
 * as bias).
 *
 *   y             device bf16 [y_rows, hidden], same row layout as recv_x of the handle's dispatch;
 *                 y_rows must be >= ep_recv_capacity(...).  Padding rows are never read.
 *   topk_weights  device fp32 [num_tokens, num_topk], nullable.  Non-NULL: out = sum_k w[t,k] * y[slot];
 *                 NULL: out = sum_k y[slot] (rows already weighted by the expert computation).
 *   bias          device bf16 [num_tokens, hidden], nullable; added after the expert terms.
 *   out           device bf16 [num_tokens, hidden]; every row is written.  A token with no local slot
 *                 gets its bias row (or zeros).
 *   Accumulation is fp32 in ascending k, then one round-to-nearest-even to bf16.
 */
ep_status_t ep_combine(ep_handle_t handle, const void* y, int hidden, int64_t y_rows, const float* topk_weights,
                       const void* bias, void* out, void* stream);

/*
 * ep_combine_tokens -- combine for the token-major rows of a dispatch with do_expand = 0 ([MoE-comm] §一:
 * without expansion the expert side returns one row per received token, so the combine moves that row back
 * to its token; the shared expert's output joins as bias).
 *
 *   y       device bf16 [y_rows, hidden], row j = the output for the j-th token of this rank (as recv_x);
 *           y_rows >= num_tokens.  Rows past num_tokens_per_rank[rank] are never read.
 *   bias    device bf16 [num_tokens, hidden], nullable.
 *   out     device bf16 [num_tokens, hidden] = y[row of t] + bias in fp32, one RNE rounding; a token with no
 *           expert on this rank gets its bias row (or zeros).  Every row is written.
 */
ep_status_t ep_combine_tokens(ep_handle_t handle, const void* y, int hidden, int64_t y_rows, const void* bias,
                              void* out, void* stream);

/*
 * ep_combine_reduce -- the source rank's reduce epilogue after the combine exchange ([DeepEP->MegaMoE] §2.5:
 * the rows returned by the ranks holding a token's experts are added element-wise; [MoE-comm] §一: the
 * shared-expert output joins as bias).  Rank r returns, in window r, one row per token this rank sent it
 * (its experts' already combined outputs, e.g. ep_combine over the receiver's handle), in the same order as
 * the send window.
 *
 *   handle    the source rank's handle (the one its dispatch used).
 *   partials  device bf16 [num_ranks, num_tokens, hidden]; window rank is not read; nullable when num_ranks == 1.
 *   local     device bf16 [num_tokens, hidden], nullable: this rank's own combine output (without bias).
 *   bias      device bf16 [num_tokens, hidden], nullable.
 *   out       device bf16 [num_tokens, hidden] = local + sum over ranks r != rank holding the token of
 *             partials[r][send_slot(t, r)] + bias, fp32 in that order, one RNE rounding.  Every row is written.
 */
ep_status_t ep_combine_reduce(ep_handle_t handle, const void* partials, int hidden, const void* local,
                              const void* bias, void* out, void* stream);

/* End of a handle's life ([MoE-comm] §二: a handle and the buffers it refers to must outlive every operation
 * that uses them; §一: the handle carries the dispatch's grouping for the combine and backward).  Frees the host
 * object only: never blocks, never touches device memory, so kernels already enqueued with the handle are
 * unaffected (they took their arguments at launch).  NULL is allowed (no-op).  A pointer that is not a live
 * handle (already freed, or never returned by ep_get_layout / ep_layout_dispatch) returns EP_ERR_INVALID_ARG
 * without being read. */
ep_status_t ep_handle_free(ep_handle_t handle);

#ifdef __cplusplus
}
#endif
#endif /* EP_MI355X_H */
