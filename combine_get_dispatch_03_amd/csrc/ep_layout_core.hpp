// ep_layout_core.hpp -- device-side pieces of the layout ([repo-map] §2.1; [DeepEP->MegaMoE] §2.2 and §2.4:
// counts, their aligned prefix sum, stable rows) that more than one kernel uses: the aligned scan of the local
// experts, the global counts, the padding-row lookup, and the per-token counting of a one-tile batch, shared
// by the layout kernels (ep_layout.hip) and the one-launch layout + dispatch kernel for small batches
// (ep_fused.hip).  The multi-tile counting sort lives in ep_layout.hip, which describes the scheme.
#pragma once

#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {

extern __shared__ __align__(16) unsigned char layout_smem[];   // dynamic LDS of the layout kernels

namespace {

constexpr int kTile = kLayoutTileTokens;   // 256 tokens per tile
constexpr int kThreads = 1024;             // every layout block: 16 waves
constexpr int kWaves = kThreads / 64;
constexpr int kBad = -2;                   // staged value of an entry < -1 or >= E
constexpr int kMaxEntriesPerThread = kTile * kMaxTopk / kThreads;   // 8: one staging pass covers a tile

// Block-wide exclusive scan of two ints per thread at once (kThreads threads).  Returns the exclusive
// prefixes in ex0/ex1 and the block totals in all0/all1.  `scratch` holds 2 * kWaves ints.
__device__ void block_exclusive_scan2(int v0, int v1, int* scratch, int& ex0, int& ex1, int& all0, int& all1) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int i0 = wave_inclusive_scan(v0), i1 = wave_inclusive_scan(v1);
    if (lane == 63) {
        scratch[w] = i0;
        scratch[kWaves + w] = i1;
    }
    __syncthreads();
    int b0 = 0, b1 = 0, a0 = 0, a1 = 0;
    for (int i = 0; i < kWaves; ++i) {
        const int s0 = scratch[i], s1 = scratch[kWaves + i];
        if (i < w) {
            b0 += s0;
            b1 += s1;
        }
        a0 += s0;
        a1 += s1;
    }
    ex0 = b0 + i0 - v0;
    ex1 = b1 + i1 - v1;
    all0 = a0;
    all1 = a1;
}

struct Outputs {
    int32_t* cnt_local;       // workspace
    int32_t* psum_ws;         // workspace
    int32_t* pad_rows;        // workspace, nullptr when A == 1
    int32_t* pad_total;       // workspace
    int32_t* ntok_rank;       // caller, nullable
    int32_t* ntok_expert;     // caller, nullable
    int32_t* psum;            // caller, nullable
    int32_t* invalid;         // caller, nullable
};

// ceil(c / A) * A for 0 <= c and c + A - 1 <= INT32_MAX (the receive-capacity limit), 1 <= A <= 65536: the fp64
// product n * (1 / A) is within 2^-21 of n / A, so its floor is off only when n / A is a whole number, and then
// by one, which the correction restores.  A few instructions instead of an integer division.
__device__ __forceinline__ int align_up(int c, int A, double inv_a) {
    const uint32_t n = (uint32_t)c + (uint32_t)A - 1u;
    uint32_t q = (uint32_t)((double)n * inv_a);
    if ((q + 1u) * (uint32_t)A <= n) ++q;
    return (int)(q * (uint32_t)A);
}

// Aligned exclusive scan of the local experts' counts (total[lo + j]) into psum[0..epr] and of their padding
// counts into padpre[0..epr], in LDS.  Every thread of the block calls it; it ends with a barrier.  Up to 256
// local experts one wave does it (4 consecutive experts per lane, two DPP wave scans, one barrier); beyond
// that the whole block scans.
__device__ void local_scan(int epr, int lo, int A, const int* total, int* psum, int* padpre, int* scratch) {
    const int tid = threadIdx.x;
    if (epr <= 4 * kWave) {
        if (tid < kWave) {
            int c[4], pad[4], gap[4], s0 = 0, s1 = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = total[lo + min(4 * tid + j, epr - 1)];   // issued together
            const double inv_a = 1.0 / (double)A;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int cj = 4 * tid + j < epr ? c[j] : 0;
                pad[j] = align_up(cj, A, inv_a);
                gap[j] = pad[j] - cj;
                s0 += pad[j];
                s1 += gap[j];
            }
            const int i0 = wave_inclusive_scan(s0), i1 = wave_inclusive_scan(s1);
            int r0 = i0 - s0, r1 = i1 - s1;          // exclusive prefix of this lane's first expert
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = 4 * tid + j;
                if (e < epr) {
                    psum[e] = r0;
                    padpre[e] = r1;
                }
                r0 += pad[j];
                r1 += gap[j];
            }
            if (tid == kWave - 1) {
                psum[epr] = i0;
                padpre[epr] = i1;
            }
        }
        __syncthreads();
        return;
    }
    const int c = tid < epr ? total[lo + tid] : 0;
    const int padded = align_up(c, A, 1.0 / (double)A);
    int ex, expad, all, allpad;
    block_exclusive_scan2(padded, padded - c, scratch, ex, expad, all, allpad);
    if (tid < epr) {
        psum[tid] = ex;
        padpre[tid] = expad;
    }
    if (tid == 0) {
        psum[epr] = all;
        padpre[epr] = allpad;
    }
    __syncthreads();
}

// Global counts, the local psum (the caller's copy and the workspace's), local counts, padding total and the
// invalid count, from the column totals and the scans.  One block calls it.
__device__ void write_counts(int E, int R, int lo, int epr, const int* total, const int* psum, const int* padpre,
                             const Outputs& o) {
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kThreads)
        if (o.ntok_expert) o.ntok_expert[e] = total[e];
    for (int j = tid; j <= epr; j += kThreads) {
        o.psum_ws[j] = psum[j];
        if (o.psum) o.psum[j] = psum[j];
        if (j < epr) o.cnt_local[j] = total[lo + j];
    }
    if (tid < R && o.ntok_rank) o.ntok_rank[tid] = total[E + tid];
    if (tid == 0) {
        *o.pad_total = padpre[epr];
        if (o.invalid) *o.invalid = total[E + R];
    }
}

// Padding row number q (0 <= q < padpre[epr]) -> its row: the expert j with padpre[j] <= q < padpre[j+1] (binary
// search in LDS), whose padding rows are the last padpre[j+1] - padpre[j] rows before psum[j+1].  The same
// order as the dense padding-row list.
__device__ __forceinline__ int pad_row_of(int q, int epr, const int* psum, const int* padpre) {
    int lo = 0, hi = epr;          // invariant: padpre[lo] <= q < padpre[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (padpre[mid] <= q) lo = mid;
        else hi = mid;
    }
    return psum[lo + 1] - (padpre[lo + 1] - q);
}

// ---- per-token layout of one tile (<= 256 tokens) ---------------------------------------------------------
// A token's rows follow from counts alone ([DeepEP->MegaMoE] §2.2: rows stable in (token, k) order): the
// expert-major row of its entry k is the aligned start of the expert, plus the expert's entries in the tokens
// before it, plus the copies of the expert among its entries 0..k-1; its row in rank r's window is the number
// of tokens before it with an expert on r.  A workgroup that writes token t stages the routing table and builds
// these counts with LDS atomic adds, and each token's set of ranks with atomic ORs (their order changes neither a
// count nor a set, so the result is deterministic), then the aligned scan of the local experts.
struct TokLds {
    uint64_t* tmask;   // [256]         the ranks each token has an expert on
    int* ent;          // [256 * K]     staged expert ids (-1 none, kBad invalid)
    int* tot;          // [E + R + 1]   column totals: entries per expert | tokens per rank | invalid entries
    int* bef;          // [E]           entries per expert in the tokens before t
    int* rbef;         // [R]           tokens before t with an expert on rank r
    int* psum;         // [epr + 1]     aligned prefix of the local experts
    int* padpre;       // [epr + 1]     padding prefix of the local experts
    int* scratch;      // [2 * kWaves]
};

__host__ __device__ inline size_t tok_lds_bytes(int E, int K, int R, int epr) {
    return sizeof(uint64_t) * kTile +
           sizeof(int) * ((size_t)kTile * K + 2 * (size_t)E + 2 * (size_t)R + 1 + 2 * (size_t)(epr + 1) +
                          2 * (size_t)kWaves);
}

__device__ inline TokLds carve_tok(unsigned char* base, int E, int K, int R, int epr) {
    TokLds L;
    L.tmask = reinterpret_cast<uint64_t*>(base);
    L.ent = reinterpret_cast<int*>(L.tmask + kTile);
    L.tot = L.ent + kTile * K;
    L.bef = L.tot + E + R + 1;
    L.rbef = L.bef + E;
    L.psum = L.rbef + R;
    L.padpre = L.psum + epr + 1;
    L.scratch = L.padpre + epr + 1;
    return L;
}

// expert -> owning rank as floor((e + 0.5) / epr) in fp32: exact for e < 1024, epr <= 1024
__device__ __forceinline__ int rank_of(int e, float inv_epr) { return (int)(((float)e + 0.5f) * inv_epr); }

// Stage the table, count (totals and counts before token t; t >= T counts nothing before), scan.  `pre` runs
// right after the entry loads are issued (loads that do not depend on the layout go there), `post` once the
// counts are complete, before the scan, which wave 0 runs alone (work of the other waves that needs the counts
// but not the scan overlaps it there).  Every thread of the block calls it; it ends with a barrier.
template <class Pre, class Post>
__device__ inline void tok_counts(const int64_t* __restrict__ idx, int T, int K, int E, int R, int epr, int A,
                                  int lo, int t, const TokLds& L, Pre pre, Post post) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int nent = T * K;
    const int npass = (nent + kThreads - 1) / kThreads;   // entries per thread (uniform): passes past it are skipped
    const int tb = t < T ? t : 0;                    // tokens counted as before: none for a workgroup past T
    static_assert(kTile * kMaxTopk <= kMaxEntriesPerThread * kThreads, "one staging pass per tile");
    int64_t v[kMaxEntriesPerThread];
#pragma unroll
    for (int u = 0; u < kMaxEntriesPerThread; ++u) {
        const int j = u * kThreads + tid;
        v[u] = (u < npass && j < nent) ? idx[j] : -1;
    }
    pre();
    for (int i = tid; i < E + R + 1; i += kThreads) L.tot[i] = 0;
    for (int i = tid; i < E; i += kThreads) L.bef[i] = 0;
    if (tid < R) L.rbef[tid] = 0;
    if (tid < kTile) L.tmask[tid] = 0ull;
    int st[kMaxEntriesPerThread];
#pragma unroll
    for (int u = 0; u < kMaxEntriesPerThread; ++u) {
        const int j = u * kThreads + tid;
        st[u] = (v[u] >= 0 && v[u] < E) ? (int)v[u] : (v[u] == -1 ? -1 : kBad);
        if (u < npass && j < nent) L.ent[j] = st[u];
    }
    __syncthreads();
    // per entry: its expert's total, its expert's count before token t, and its rank's bit in its token's mask
    const float inv_epr = 1.0f / (float)epr, inv_k = 1.0f / (float)K;
    int inv = 0;
#pragma unroll
    for (int u = 0; u < kMaxEntriesPerThread; ++u) {
        if (u >= npass) break;
        const int j = u * kThreads + tid;
        const int e = j < nent ? st[u] : -1;
        if (e >= 0) {
            atomicAdd(&L.tot[e], 1);
            if (j < tb * K) atomicAdd(&L.bef[e], 1);
            // token of entry j = floor((j + 0.5) / K) in fp32: exact for j < 2^13, K <= 32
            atomicOr(reinterpret_cast<unsigned long long*>(&L.tmask[(int)(((float)j + 0.5f) * inv_k)]),
                     1ull << rank_of(e, inv_epr));
        }
        inv += popc64(ballot(e == kBad));
    }
    if (lane == 0 && inv != 0) atomicAdd(&L.tot[E + R], inv);
    __syncthreads();
    // tokens per rank and those before t, from the token masks, on waves 4..7 (token tid - 256) while wave 0
    // scans: per rank present in the wave, one ballot for its tokens, one for those before t, one LDS add each
    // (nothing reads these counts before the scan's barrier)
    const int rt = tid - kTile;
    if (rt >= 0 && rt < kTile && (rt & ~(kWave - 1)) < T) {
        const uint64_t m = rt < T ? L.tmask[rt] : 0ull;
        const uint64_t present = R > 32 ? ((uint64_t)wave_or((uint32_t)(m >> 32)) << 32) | wave_or((uint32_t)m)
                                        : (uint64_t)wave_or((uint32_t)m);
        for (uint64_t rr = present; rr != 0; rr &= rr - 1) {
            const int r = __builtin_ctzll(rr);
            const bool bit = (m >> r) & 1ull;
            const int all = popc64(ballot(bit)), before = popc64(ballot(bit && rt < tb));
            if (lane == 0) {
                atomicAdd(&L.tot[E + r], all);
                if (before != 0) atomicAdd(&L.rbef[r], before);
            }
        }
    }
    post();
    local_scan(epr, lo, A, L.tot, L.psum, L.padpre, L.scratch);
}

// Token t's rows (t < T), in one wave: lane k < K gets the expert-major row of entry k (-1 if the expert is not
// local or the entry not valid), lane r < R the token's row in rank r's window (-1 if it has no expert on r).
// tok_row_counts needs the expert counts only (it can run while wave 0 scans); tok_row_slot adds the expert's
// aligned start from the scan, and tok_row_own reads the rank's count before t (complete, like the scan, at
// the scan's barrier).  Every lane reads all K entries of the token (the same LDS words for every lane, so
// broadcast reads issued together) and counts the copies of its own entry before it.
struct TokRow {
    int e;            // lane k < K: entry k
    int before;       // lane k < K: entries of e in the tokens before t, plus copies of e among entries 0..k-1
    uint64_t ranks;   // the ranks the token has an expert on
};

__device__ inline TokRow tok_row_counts(const TokLds& L, int t, int K) {
    const int lane = lane_id();
    const int* ent = L.ent + t * K;
    TokRow r;
    r.e = lane < K ? ent[lane] : -1;
    r.ranks = L.tmask[t];
    int dup = 0;
    for (int k0 = 0; k0 < K; k0 += 8) {
        int q[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) q[u] = ent[min(k0 + u, K - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) dup += (k0 + u < lane && q[u] == r.e) ? 1 : 0;
    }
    r.before = r.e >= 0 ? L.bef[r.e] + dup : 0;
    return r;
}

__device__ inline int tok_row_slot(const TokLds& L, const TokRow& r, int K, int lo, int epr) {
    return (lane_id() < K && r.e >= lo && r.e < lo + epr) ? L.psum[r.e - lo] + r.before : -1;
}

__device__ inline int tok_row_own(const TokLds& L, const TokRow& r, int R) {
    const int lane = lane_id();
    return (lane < R && ((r.ranks >> lane) & 1ull) != 0) ? L.rbef[lane] : -1;
}

}  // namespace
}  // namespace ep
