/*
 * ep_oracle.h -- CPU oracle for the one-GPU MoE expert-parallel layout / dispatch / combine path.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check in __graft_entry__.py and
 * the cpu_baseline leg of bench.py may load or call this library.  It shares no code, header, table or
 * helper with the HIP library under combine_get_dispatch_03_amd/; neither side includes or links the other.
 *
 * Everything here is a plain, single-threaded, obviously-correct definition of what the path computes.
 * Page names used in the citations:
 *   [DeepEP->MegaMoE]  "从 DeepEP 到 Mega MoE：MoE Runtime 演进的三向验证分析" (backyes.github.io)
 *   [DeepEP-hotdry]    DeepEP expert-parallel communication article (blog.hotdry.top)
 *   [MoE-comm]         "MoE 为什么容易卡在通信上？" (locsic.com, DeepEP-Ascend walk-through)
 *   [flops-record]     inference-research record "deepep-expert-parallel-dispatch-combine" (phantomic12)
 *   [repo-map]         "第 2 章 仓库地图与模块职责" (bowenzhou.top, DeepEP repo map)
 */
#ifndef EP_ORACLE_H
#define EP_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats ------------------------------------------------------------------------------- */
float    oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_f64_to_bf16(double v);          /* round to nearest, ties to even; overflow -> inf      */
float    oracle_e4m3_decode(uint8_t c);         /* OCP FP8 E4M3 (e4m3fn)                                */
uint8_t  oracle_e4m3_encode(float v);           /* RNE onto the finite e4m3fn set, saturating to +-448  */

/* bulk helpers over arrays (same definitions, looped) */
void oracle_e4m3_encode_array(const float* v, int64_t n, uint8_t* out);
void oracle_f64_to_bf16_array(const double* v, int64_t n, uint16_t* out);

/* ---- layout ------------------------------------------------------------------------------------------ */
int64_t oracle_recv_capacity(int num_tokens, int num_topk, int num_local_experts, int expert_alignment);

/* Returns 0, or -1 on an argument the definition does not cover.  Every output is written in full:
 *   cnt[E]            number of (t,k) entries equal to e
 *   ntok_rank[R]      tokens with at least one expert on rank r (a token counts once per rank)
 *   in_rank[T*R]      0/1 membership of token t in rank r
 *   psum[El+1]        aligned exclusive starts of this rank's local experts; psum[El] = rows used
 *   slot[T*K]         row of entry (t,k) in the expert-major buffer, -1 when the expert is not local
 *   row_src[cap]      source token of each row, -1 for padding rows and for rows past psum[El]
 *   send_slot[T*R]    rank of t among the tokens in rank r (send window row for r != rank; token-major
 *                     receive row for r == rank), else -1
 *   num_invalid[1]    entries < -1 or >= E, which are dropped                                          */
int oracle_layout(const int64_t* topk_idx, int T, int K, int E, int R, int rank, int A,
                  int32_t* cnt, int32_t* ntok_rank, uint8_t* in_rank, int32_t* psum,
                  int32_t* slot, int32_t* row_src, int64_t cap, int32_t* send_slot, int32_t* num_invalid);

/* ---- dispatch ---------------------------------------------------------------------------------------- */
/* Per-token per-128-channel FP8 quantisation of one BF16 row (H % 128 == 0). */
void oracle_quantize_row(const uint16_t* x, int H, uint8_t* q, float* scales);

/* fp8 != 0: recv_x is uint8 [rows,H], recv_scales float [rows,H/128]; else recv_x is uint16 (bf16) [rows,H].
 * do_expand: rows = cap, recv_src [cap], recv_w [cap]; else rows = T, recv_src [T], recv_w [T,K],
 * recv_topk_idx int64 [T,K].  Optional outputs may be NULL.  Send windows (R > 1): send_x [R,T,H],
 * send_scales [R,T,H/128], send_src [R,T], send_topk_idx int64 [R,T,K], send_topk_w [R,T,K].          */
int oracle_dispatch(const uint16_t* x, int T, int H, int K, const float* topk_w, const int64_t* topk_idx,
                    int E, int R, int rank, int A, int fp8, int zero_pad, int do_expand,
                    const int32_t* cnt, const int32_t* psum, const int32_t* slot, const int32_t* send_slot,
                    void* recv_x, float* recv_scales, int32_t* recv_src, float* recv_w, int64_t* recv_topk_idx,
                    void* send_x, float* send_scales, int32_t* send_src, int64_t* send_topk_idx,
                    float* send_topk_w);

/* Expert-major placement of rows that already carry their receive format (the receiver side of the copy
 * epilogue): row_bytes bytes per row plus G fp32 scales (G may be 0).  Layout from oracle_layout over the
 * received rows' local expert ids.  recv_src = index of the received row; recv_w = topk_w[i,k] or 1. */
int oracle_dispatch_rows(const uint8_t* rows, int N, int row_bytes, const float* scales, int G, int K,
                         const float* topk_w, int E_local, int A, int zero_pad, const int32_t* cnt,
                         const int32_t* psum, const int32_t* slot, uint8_t* recv_x, float* recv_scales,
                         int32_t* recv_src, float* recv_w);

/* ---- combine ----------------------------------------------------------------------------------------- */
/* out[t,h] = sum_k w[t,k] * y[slot[t,k],h] (+ bias[t,h]) in double; w == NULL means all weights are 1. */
void oracle_combine(const uint16_t* y, int H, const int32_t* slot, const float* topk_w, int T, int K,
                    const uint16_t* bias, double* out);

/* Source-side sum after the combine exchange: out[t,h] = bias + local + sum over ranks r != rank with
 * send_slot[t,r] >= 0 of partials[r, send_slot[t,r], h], in double.  local and bias may be NULL. */
void oracle_combine_reduce(const uint16_t* partials, int T, int H, int R, int rank, const int32_t* send_slot,
                           const uint16_t* local, const uint16_t* bias, double* out);

#ifdef __cplusplus
}
#endif
#endif
