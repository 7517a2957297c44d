/*
 * ep_oracle.c -- CPU oracle for the one-GPU MoE expert-parallel layout / dispatch / combine path.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, __graft_entry__.smoke() and the cpu_baseline
 * leg of bench.py may load it.  It shares nothing with the HIP library and is built by gcc alone with
 * -O2 -ffp-contract=off (IEEE binary32/binary64 arithmetic, no contraction, no fast-math).
 *
 * It is the plain definition of each step, written as loops in the order the definition states.  Page names
 * used in citations are listed in ep_oracle.h.  Readings of points the pages leave open are marked
 * "reading:" and are the ones listed in the design notes of the repository.
 *
 * Pins (tests/test_oracle_*.py): the e4m3 and bf16 codecs against brute-force nearest-value search and
 * torch's CPU casts; the layout against the padding worked example of [MoE-comm] §三, brute-force counts
 * and numpy's stable argsort; the quantiser against hand-computed codes and its dequantisation bound; the
 * combine against a dense scatter-matrix product and its closed forms.  The pages only say that FP8 rows
 * travel with scale factors; the per-128-channel absmax recipe is a reading, pinned by what any absmax scaling
 * to e4m3's largest finite value must satisfy (the group maximum maps to +-448, every element dequantises to
 * within half an e4m3 step).  The 1e-4 floor for all-zero and tiny groups is the one choice those properties
 * leave open: parity unpinned for that floor.
 */
#include "ep_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ======================================================================================================
 * Number formats
 * ====================================================================================================== */

/* BF16 is the upper half of an IEEE binary32: widening is exact. */
float oracle_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a double to BF16 (8 significant bits, exponent range of binary32), nearest, ties to even.
 * The rounding step is the textbook one: divide by the spacing of representable values in the
 * binade of |v| (a power of two, so exact), round the quotient half-to-even with rint(), scale back. */
uint16_t oracle_f64_to_bf16(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7F80;
    double spacing;
    if (a < ldexp(1.0, -126)) {
        spacing = ldexp(1.0, -133);                 /* subnormal spacing */
    } else {
        int ex;
        frexp(a, &ex);                              /* a = f * 2^ex, f in [0.5, 1) */
        spacing = ldexp(1.0, (ex - 1) - 7);         /* 7 stored fraction bits */
    }
    double r = rint(a / spacing) * spacing;         /* exact: rint result * power of two */
    if (r > ldexp(255.0, 120)) return sign | 0x7F80; /* above the largest finite value -> inf */
    if (r < ldexp(1.0, -126)) return sign | (uint16_t)(r / ldexp(1.0, -133));
    int ex;
    double f = frexp(r, &ex);
    int biased = (ex - 1) + 127;
    int frac = (int)((2.0 * f - 1.0) * 128.0);      /* exact */
    return sign | (uint16_t)((biased << 7) | frac);
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3 fraction bits.  Exponent field 0
 * holds subnormals m * 2^-9; fields 1..15 hold normals 2^(e-7) * (1 + m/8), except field 15 with m = 7,
 * which is NaN.  There are no infinities; the largest finite magnitude is 1.75 * 2^8 = 448. */
float oracle_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return (float)(s ? -mag : mag);
}

/* Round a binary32 value to the nearest e4m3fn value, ties to the even code, saturating magnitudes that
 * round beyond 448 to 448.  The sign of zero is kept (a negative value that rounds to zero gives 0x80).
 * NaN gives 0x7F.  This is the "e4m3, round-to-nearest-even, saturating" cast of the FP8 dispatch
 * ([DeepEP-hotdry], key techniques: FP8 dispatch with BF16 combine). */
uint8_t oracle_e4m3_encode(float v) {
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7E;             /* saturate (also covers +-inf) */
    double spacing;
    if (a < ldexp(1.0, -6)) {
        spacing = ldexp(1.0, -9);                   /* subnormal spacing */
    } else {
        int ex;
        frexp(a, &ex);
        spacing = ldexp(1.0, (ex - 1) - 3);         /* 3 stored fraction bits */
    }
    double r = rint(a / spacing) * spacing;         /* r <= 448 because a < 448 */
    if (r < ldexp(1.0, -6)) return sign | (uint8_t)(r / ldexp(1.0, -9));
    int ex;
    double f = frexp(r, &ex);
    int biased = (ex - 1) + 7;
    int frac = (int)((2.0 * f - 1.0) * 8.0);        /* exact */
    return sign | (uint8_t)((biased << 3) | frac);
}

void oracle_e4m3_encode_array(const float* v, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(v[i]);
}

void oracle_f64_to_bf16_array(const double* v, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16(v[i]);
}

/* ======================================================================================================
 * Layout
 * ====================================================================================================== */

/* Rows an expert-major receive buffer must hold: every routed entry plus, per local expert, at most
 * A - 1 padding rows, since ceil(c / A) * A <= c + A - 1.  Capacity is fixed up front so no host sync
 * is needed ([flops-record], Arithmetic intensity: outputs sized to configured capacity). */
int64_t oracle_recv_capacity(int num_tokens, int num_topk, int num_local_experts, int expert_alignment) {
    return (int64_t)num_tokens * num_topk + (int64_t)num_local_experts * (expert_alignment - 1);
}

/* Counting-sort layout of the routing table.
 *  - per-expert counts, as the dispatch notify warps count tokens per destination expert
 *    ([DeepEP->MegaMoE] §2.2) and as layout.cu's expert count ([repo-map] §2.1);
 *  - per-rank token counts and is_token_in_rank membership ([repo-map] §2.1: rank count, membership);
 *    reading: expert e belongs to rank e / (E/R); a token counts once per rank;
 *  - psum_num_recv_tokens_per_expert: aligned exclusive starts of each local expert's segment, the
 *    cursor the copy epilogue places rows from ([DeepEP->MegaMoE] §2.4) and the valid ranges a grouped
 *    GEMM reads ([flops-record]); segments are padded to multiples of expert_alignment
 *    ([MoE-comm] §一 expert_alignment / do_zero_padding; §三 padding worked example);
 *    reading: an empty expert takes no rows;
 *  - the slot of every entry.  Reading: rows of one expert are in ascending flat index t*K+k (a stable
 *    counting sort; the atomics of the copy epilogue allow any order, this fixes one);
 *  - reading: entries equal to -1 are unused; entries < -1 or >= E are dropped and counted;
 *  - per-rank token rows: the rank of t among the tokens with an expert on r, dense in ascending t (send
 *    windows for other ranks; the token-major receive rows for this rank). */
int oracle_layout(const int64_t* topk_idx, int T, int K, int E, int R, int rank, int A,
                  int32_t* cnt, int32_t* ntok_rank, uint8_t* in_rank, int32_t* psum,
                  int32_t* slot, int32_t* row_src, int64_t cap, int32_t* send_slot, int32_t* num_invalid) {
    if (T < 0 || K < 1 || E < 1 || R < 1 || E % R != 0 || rank < 0 || rank >= R || A < 1) return -1;
    const int epr = E / R;                       /* experts per rank */
    const int lo = rank * epr;                   /* first local expert */

    /* step 1: counts, membership, invalid entries */
    for (int e = 0; e < E; ++e) cnt[e] = 0;
    for (int64_t i = 0; i < (int64_t)T * R; ++i) in_rank[i] = 0;
    int32_t invalid = 0;
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[(int64_t)t * K + k];
            if (e == -1) continue;
            if (e < -1 || e >= E) { invalid++; continue; }
            cnt[e]++;
            in_rank[(int64_t)t * R + e / epr] = 1;
        }
    }
    *num_invalid = invalid;

    /* step 2: tokens per rank */
    for (int r = 0; r < R; ++r) {
        int32_t n = 0;
        for (int t = 0; t < T; ++t) n += in_rank[(int64_t)t * R + r];
        ntok_rank[r] = n;
    }

    /* step 3: aligned exclusive starts of the local experts */
    psum[0] = 0;
    for (int j = 0; j < epr; ++j) {
        int32_t c = cnt[lo + j];
        int32_t padded = ((c + A - 1) / A) * A;
        psum[j + 1] = psum[j] + padded;
    }
    if ((int64_t)psum[epr] > cap) return -1;

    /* step 4: stable slots, walking entries in flat order with one cursor per local expert */
    int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)(epr > 0 ? epr : 1));
    for (int j = 0; j < epr; ++j) cursor[j] = psum[j];
    for (int64_t r = 0; r < cap; ++r) row_src[r] = -1;
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int64_t e = topk_idx[(int64_t)t * K + k];
            int32_t s = -1;
            if (e >= lo && e < lo + epr) {
                s = cursor[e - lo]++;
                row_src[s] = t;
            }
            slot[(int64_t)t * K + k] = s;
        }
    }
    free(cursor);

    /* step 5: per-rank token rows, dense from 0 in ascending token order: for r != rank the row of t in the
     * send window of rank r; for r == rank its row in the token-major receive layout (do_expand off) */
    for (int r = 0; r < R; ++r) {
        int32_t j = 0;
        for (int t = 0; t < T; ++t) {
            int32_t s = -1;
            if (in_rank[(int64_t)t * R + r]) s = j++;
            send_slot[(int64_t)t * R + r] = s;
        }
    }
    return 0;
}

/* ======================================================================================================
 * Dispatch
 * ====================================================================================================== */

/* Quantise one BF16 row to e4m3 with one fp32 scale per 128 channels; the token travels with its scale
 * factors as in the x / x_sf pair of [DeepEP->MegaMoE] §3.1.  Reading (the pages give no recipe):
 *   amax = max |x| over the group (exact), a = max(amax, 1e-4),
 *   scale = a / 448 and inv = 448 / a (each one correctly rounded binary32 division),
 *   q = e4m3(x * inv) with one correctly rounded binary32 multiply.
 * Every operation is IEEE binary32, so a GPU doing the same operations gets the same bits. */
void oracle_quantize_row(const uint16_t* x, int H, uint8_t* q, float* scales) {
    for (int g = 0; g < H / 128; ++g) {
        float amax = 0.0f;
        for (int j = 0; j < 128; ++j) {
            float v = fabsf(oracle_bf16_to_f32(x[g * 128 + j]));
            if (v > amax) amax = v;
        }
        float a = amax > 1e-4f ? amax : 1e-4f;
        float scale = a / 448.0f;
        float inv = 448.0f / a;
        scales[g] = scale;
        for (int j = 0; j < 128; ++j) {
            float prod = oracle_bf16_to_f32(x[g * 128 + j]) * inv;
            q[g * 128 + j] = oracle_e4m3_encode(prod);
        }
    }
}

/* Dispatch of this rank's tokens, following the dispatch and copy-epilogue kernels of [DeepEP->MegaMoE] §2.2
 * and §2.4 and the dispatch arguments of [MoE-comm] §一:
 *  - each token row is read once and, when FP8, quantised once ([DeepEP-hotdry] key techniques);
 *  - do_expand: the row (and its scales) is written to every expert-major slot of the token; recv_src = t
 *    and recv_w = w[t,k] per row (the source-token metadata of the received rows, [DeepEP->MegaMoE] §2.3);
 *    padding rows [psum[j] + cnt, psum[j+1]): with do_zero_padding the data bytes and scales are zero;
 *    reading: without it they are left untouched; their recv_src is -1 and recv_w is 0 either way; rows at
 *    or past psum[El] are never written;
 *  - reading of do_expand off: one row per token with an expert on this rank, in ascending token order
 *    (row send_slot[t, rank]), no padding; recv_src[j] = t, recv_topk_idx[j, k] = the local expert id of
 *    entry k or -1, recv_w[j, k] = w[t, k];
 *  - send windows, R > 1: for r != rank, window r row send_slot[t,r] gets the same bytes and scales, the
 *    source token, the destination-local expert ids (e - r*E/R, or -1 when r does not own e) and the
 *    weights ([DeepEP->MegaMoE] §2.2: store to the send buffer before the transfer). */
int oracle_dispatch(const uint16_t* x, int T, int H, int K, const float* topk_w, const int64_t* topk_idx,
                    int E, int R, int rank, int A, int fp8, int zero_pad, int do_expand,
                    const int32_t* cnt, const int32_t* psum, const int32_t* slot, const int32_t* send_slot,
                    void* recv_x, float* recv_scales, int32_t* recv_src, float* recv_w, int64_t* recv_topk_idx,
                    void* send_x, float* send_scales, int32_t* send_src, int64_t* send_topk_idx,
                    float* send_topk_w) {
    if (T < 0 || H < 1 || K < 1 || E % R != 0 || A < 1) return -1;
    if (fp8 && H % 128 != 0) return -1;
    const int epr = E / R;
    const int lo = rank * epr;
    const int G = fp8 ? H / 128 : 0;                        /* scale groups per row */
    const size_t row_bytes = fp8 ? (size_t)H : (size_t)H * 2;
    uint8_t* rx = (uint8_t*)recv_x;
    uint8_t* sx = (uint8_t*)send_x;
    uint8_t* row = (uint8_t*)malloc(row_bytes);
    float* sc = (float*)malloc(sizeof(float) * (size_t)(G > 0 ? G : 1));

    for (int t = 0; t < T; ++t) {
        /* the token's row in the receive format */
        if (fp8) oracle_quantize_row(x + (size_t)t * H, H, row, sc);
        else memcpy(row, x + (size_t)t * H, row_bytes);

        if (do_expand) {
            /* expert-major copies */
            for (int k = 0; k < K; ++k) {
                int32_t s = slot[(int64_t)t * K + k];
                if (s < 0) continue;
                memcpy(rx + (size_t)s * row_bytes, row, row_bytes);
                if (fp8) memcpy(recv_scales + (size_t)s * G, sc, sizeof(float) * (size_t)G);
                if (recv_src) recv_src[s] = t;
                if (recv_w) recv_w[s] = topk_w ? topk_w[(int64_t)t * K + k] : 1.0f;
            }
        } else {
            /* token-major row */
            int32_t j = send_slot[(int64_t)t * R + rank];
            if (j >= 0) {
                memcpy(rx + (size_t)j * row_bytes, row, row_bytes);
                if (fp8) memcpy(recv_scales + (size_t)j * G, sc, sizeof(float) * (size_t)G);
                if (recv_src) recv_src[j] = t;
                for (int k = 0; k < K; ++k) {
                    int64_t e = topk_idx[(int64_t)t * K + k];
                    int owned = (e >= (int64_t)lo && e < (int64_t)lo + epr);
                    if (recv_topk_idx) recv_topk_idx[(size_t)j * K + k] = owned ? e - lo : -1;
                    if (recv_w) recv_w[(size_t)j * K + k] = topk_w ? topk_w[(int64_t)t * K + k] : 1.0f;
                }
            }
        }

        /* send windows */
        for (int r = 0; r < R; ++r) {
            int32_t j = send_slot[(int64_t)t * R + r];
            if (r == rank || j < 0) continue;
            size_t wrow = (size_t)r * T + j;
            memcpy(sx + wrow * row_bytes, row, row_bytes);
            if (fp8) memcpy(send_scales + wrow * G, sc, sizeof(float) * (size_t)G);
            if (send_src) send_src[wrow] = t;
            for (int k = 0; k < K; ++k) {
                int64_t e = topk_idx[(int64_t)t * K + k];
                int owned = (e >= (int64_t)r * epr && e < (int64_t)(r + 1) * epr);
                if (send_topk_idx) send_topk_idx[wrow * K + k] = owned ? e - (int64_t)r * epr : -1;
                if (send_topk_w) send_topk_w[wrow * K + k] = topk_w ? topk_w[(int64_t)t * K + k] : 1.0f;
            }
        }
    }

    /* padding rows of each local expert (expert-major layout only) */
    for (int j = 0; do_expand && j < epr; ++j) {
        for (int32_t s = psum[j] + cnt[lo + j]; s < psum[j + 1]; ++s) {
            if (zero_pad) {
                memset(rx + (size_t)s * row_bytes, 0, row_bytes);
                if (fp8) for (int g = 0; g < G; ++g) recv_scales[(size_t)s * G + g] = 0.0f;
            }
            if (recv_src) recv_src[s] = -1;
            if (recv_w) recv_w[s] = 0.0f;
        }
    }
    free(row);
    free(sc);
    return 0;
}

/* The receiver's copy epilogue: rows arrive destination-major (one per token sent to this rank, already in
 * the receive format) and are placed expert-major at their expert's rows ([DeepEP->MegaMoE] §2.4: load the
 * received row, take the row of its expert, store).  Reading: the received rows' layout is the same stable
 * counting sort as the sender's (oracle_layout over their local expert ids with one rank), so placement is
 * deterministic; padding rows as in oracle_dispatch. */
int oracle_dispatch_rows(const uint8_t* rows, int N, int row_bytes, const float* scales, int G, int K,
                         const float* topk_w, int E_local, int A, int zero_pad, const int32_t* cnt,
                         const int32_t* psum, const int32_t* slot, uint8_t* recv_x, float* recv_scales,
                         int32_t* recv_src, float* recv_w) {
    if (N < 0 || row_bytes < 1 || G < 0 || K < 1 || E_local < 1 || A < 1) return -1;
    for (int i = 0; i < N; ++i) {
        for (int k = 0; k < K; ++k) {
            int32_t s = slot[(int64_t)i * K + k];
            if (s < 0) continue;
            memcpy(recv_x + (size_t)s * row_bytes, rows + (size_t)i * row_bytes, (size_t)row_bytes);
            if (G > 0) memcpy(recv_scales + (size_t)s * G, scales + (size_t)i * G, sizeof(float) * (size_t)G);
            if (recv_src) recv_src[s] = i;
            if (recv_w) recv_w[s] = topk_w ? topk_w[(int64_t)i * K + k] : 1.0f;
        }
    }
    for (int j = 0; j < E_local; ++j) {
        for (int32_t s = psum[j] + cnt[j]; s < psum[j + 1]; ++s) {
            if (zero_pad) {
                memset(recv_x + (size_t)s * row_bytes, 0, (size_t)row_bytes);
                for (int g = 0; g < G; ++g) recv_scales[(size_t)s * G + g] = 0.0f;
            }
            if (recv_src) recv_src[s] = -1;
            if (recv_w) recv_w[s] = 0.0f;
        }
    }
    return 0;
}

/* ======================================================================================================
 * Combine
 * ====================================================================================================== */

/* Top-k reduction back to token order: out[t] = sum over the token's local slots of w[t,k] * y[slot],
 * plus the shared-expert bias.  The combine kernels accumulate expert outputs element-wise per token
 * ([DeepEP->MegaMoE] §2.3, §2.5; Mega MoE's accumulate of §3.2 phase 6) and the shared expert's output
 * enters as bias ([MoE-comm] §一).  Reading: with weights the rows are weighted (topk_w != NULL), without
 * them they are summed as already weighted; a token with no local slot gets its bias (or 0).
 * Computed in double: each product of a binary32 weight and a BF16 value is exact in double, so the only
 * rounding is in the at most K+1 additions. */
void oracle_combine(const uint16_t* y, int H, const int32_t* slot, const float* topk_w, int T, int K,
                    const uint16_t* bias, double* out) {
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) {
                int32_t s = slot[(int64_t)t * K + k];
                if (s < 0) continue;
                double w = topk_w ? (double)topk_w[(int64_t)t * K + k] : 1.0;
                acc += w * (double)oracle_bf16_to_f32(y[(size_t)s * H + h]);
            }
            if (bias) acc += (double)oracle_bf16_to_f32(bias[(size_t)t * H + h]);
            out[(size_t)t * H + h] = acc;
        }
    }
}

/* The source rank's reduce epilogue after the combine exchange: each rank that received token t returns one
 * row (its experts' weighted outputs for t, already summed, [DeepEP->MegaMoE] §2.3), and the source adds
 * them element-wise ([DeepEP->MegaMoE] §2.5: reduced[j] += source[j]) together with its own experts' part and
 * the shared-expert bias ([MoE-comm] §一).  Row j of window r belongs to the token with send_slot[t,r] = j
 * (r != rank).
 * In double; the order of the terms does not matter at this precision for at most R + 2 terms. */
void oracle_combine_reduce(const uint16_t* partials, int T, int H, int R, int rank, const int32_t* send_slot,
                           const uint16_t* local, const uint16_t* bias, double* out) {
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            double acc = 0.0;
            if (bias) acc += (double)oracle_bf16_to_f32(bias[(size_t)t * H + h]);
            if (local) acc += (double)oracle_bf16_to_f32(local[(size_t)t * H + h]);
            for (int r = 0; r < R; ++r) {
                int32_t j = send_slot[(int64_t)t * R + r];
                if (r == rank || j < 0) continue;
                acc += (double)oracle_bf16_to_f32(partials[((size_t)r * T + j) * H + h]);
            }
            out[(size_t)t * H + h] = acc;
        }
    }
}
