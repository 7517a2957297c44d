// ep_layout.hip -- layout of a routing table on gfx950: a stable counting sort of the routed entries by
// expert, plus per-rank membership ([repo-map] §2.1: layout.cu gives rank counts, expert counts and
// token-in-rank membership; [DeepEP->MegaMoE] §2.2: per-expert counts and their prefix sum; §2.4: the prefix
// sum is each expert's start cursor; the same page's cross-reference names the scheme a counting sort).
//
// Two launches, both deterministic (no atomics decide a position):
//   k_layout_count     one block per 256-token tile.  The tile's entries are staged in LDS with one
//                      cooperative load; each of 16 waves then ranks its 16 tokens' entries in flat order with
//                      key-bit ballots (peers = lanes holding the same expert) against a per-wave LDS
//                      histogram, and the block adds the earlier waves' counts.  Writes one row per tile
//                      (expert counts, token-in-rank counts, invalid entries) and each entry's tile-local rank.
//   k_layout_finalize  one block per tile.  Each block sums the tile histograms (all tiles for the totals,
//                      earlier tiles for its own base), scans the aligned local counts into psum, turns
//                      tile-local ranks into final rows, and writes part of the dense padding-row list; block
//                      0 also writes the global counts.
#include <mutex>

#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {

extern __shared__ __align__(16) unsigned char layout_smem[];   // dynamic LDS of k_layout_count

namespace {

constexpr int kTile = kLayoutTileTokens;   // 256 tokens per tile
constexpr int kCountThreads = 1024;        // k_layout_count: 16 waves, 16 tokens each
constexpr int kCountWaves = kCountThreads / 64;
constexpr int kFinalThreads = 1024;
constexpr int kPackShift = 11;             // packed entry: (tile-local rank << 11) | expert, or -1
constexpr int kPackMask = (1 << kPackShift) - 1;
constexpr int kBad = -2;                   // staged value of an entry < -1 or >= E

__global__ __launch_bounds__(kCountThreads) void k_layout_count(
    const int64_t* __restrict__ idx, int T, int K, int E, int R, int epr, int nbits,
    int32_t* __restrict__ tile_hist, int32_t* __restrict__ packed_out, int32_t* __restrict__ send_tmp,
    uint8_t* __restrict__ in_rank_out) {
    const int NC = E + R + 1;   // tile row: expert counts | rank counts | invalid entries
    uint16_t* cnt_w = reinterpret_cast<uint16_t*>(layout_smem);                  // [16][E] per-wave counts
    int32_t* ent = reinterpret_cast<int32_t*>(layout_smem + ((sizeof(uint16_t) * kCountWaves * E + 15) & ~(size_t)15));
    int32_t* rcnt_w = ent + kTile * K;                                           // [4][R]
    int32_t* inv_w = rcnt_w + 4 * R;                                             // [16]

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int tile = blockIdx.x;
    const int tok_tile0 = tile * kTile;
    const int64_t ent_tile0 = (int64_t)tok_tile0 * K;
    const int nent_tile = max(0, min(kTile, T - tok_tile0)) * K;

    // ---- stage the tile's entries (one round trip: all loads issued before any is used) ----------------
    for (int j0 = 0; j0 < nent_tile; j0 += 8 * kCountThreads) {
        int64_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + u * kCountThreads + tid;
            v[u] = j < nent_tile ? idx[ent_tile0 + j] : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + u * kCountThreads + tid;
            if (j < nent_tile) ent[j] = (v[u] >= 0 && v[u] < E) ? (int)v[u] : (v[u] == -1 ? -1 : kBad);
        }
    }
    for (int i = tid; i < kCountWaves * E; i += kCountThreads) cnt_w[i] = 0;
    __syncthreads();

    // ---- per wave: rank its 16 tokens' entries in flat order ---------------------------------------------
    const int tok_w = kTile / kCountWaves;                 // 16 tokens per wave
    const int nent_w = max(0, min(tok_w, T - (tok_tile0 + w * tok_w))) * K;
    int32_t* went = ent + w * tok_w * K;
    const uint64_t lt = lanemask_lt();
    uint16_t* cnt = cnt_w + w * E;
    int inv = 0;
    for (int j0 = 0; j0 < nent_w; j0 += 64) {
        const int j = j0 + lane;                           // entry index within the wave's tokens
        const int e = j < nent_w ? went[j] : -1;
        const bool ok = e >= 0;
        inv += popc64(ballot(e == kBad));
        const int key = ok ? e : 0;
        const uint64_t peers = match_peers(key, ok, nbits);
        const int base = ok ? cnt[key] : 0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (ok && (peers & lt) == 0) cnt[key] = (uint16_t)(base + popc64(peers));
        if (j < nent_w) went[j] = ok ? (((base + popc64(peers & lt)) << kPackShift) | key) : -1;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
    if (lane == 0) inv_w[w] = inv;
    __syncthreads();

    // ---- tile totals; per-wave counts become exclusive per-wave bases --------------------------------------
    for (int e = tid; e < E; e += kCountThreads) {
        int c[kCountWaves];
#pragma unroll
        for (int v = 0; v < kCountWaves; ++v) c[v] = cnt_w[v * E + e];
        int run = 0;
#pragma unroll
        for (int v = 0; v < kCountWaves; ++v) {
            cnt_w[v * E + e] = (uint16_t)run;
            run += c[v];
        }
        tile_hist[(int64_t)tile * NC + e] = run;
    }
    // threads 0..255 <-> tokens of the tile (waves 0..3, 64 tokens each): token-in-rank membership
    const int t = tok_tile0 + tid;
    const bool tv = tid < kTile && t < T;
    uint64_t mask = 0ull;                              // ranks this token's experts live on
    if (tv) {
        for (int k = 0; k < K; ++k) {
            const int p = ent[tid * K + k];
            if (p >= 0) mask |= 1ull << ((p & kPackMask) / epr);
        }
    }
    if (tv && in_rank_out != nullptr)
        for (int r = 0; r < R; ++r) in_rank_out[(int64_t)t * R + r] = (uint8_t)((mask >> r) & 1ull);
    if (w < 4) {
        for (int r = 0; r < R; ++r) {
            const uint64_t b = ballot((mask >> r) & 1ull);
            if (lane == 0) rcnt_w[w * R + r] = popc64(b);
        }
    }
    __syncthreads();
    if (tid < R) {
        const int c0 = rcnt_w[tid], c1 = rcnt_w[R + tid], c2 = rcnt_w[2 * R + tid], c3 = rcnt_w[3 * R + tid];
        rcnt_w[tid] = 0;
        rcnt_w[R + tid] = c0;
        rcnt_w[2 * R + tid] = c0 + c1;
        rcnt_w[3 * R + tid] = c0 + c1 + c2;
        tile_hist[(int64_t)tile * NC + E + tid] = c0 + c1 + c2 + c3;
    }
    if (tid == 0) {
        int s = 0;
        for (int v = 0; v < kCountWaves; ++v) s += inv_w[v];
        tile_hist[(int64_t)tile * NC + E + R] = s;
    }
    __syncthreads();

    // ---- tile-local ranks --------------------------------------------------------------------------------
    for (int j = tid; j < nent_tile; j += kCountThreads) {
        const int p = ent[j];
        const int wv = (j / K) / tok_w;
        packed_out[ent_tile0 + j] =
            p < 0 ? -1 : (((p >> kPackShift) + cnt_w[wv * E + (p & kPackMask)]) << kPackShift) | (p & kPackMask);
    }
    if (send_tmp != nullptr && w < 4) {
        for (int r = 0; r < R; ++r) {
            const bool bit = (mask >> r) & 1ull;
            const uint64_t b = ballot(bit);
            if (tv) send_tmp[(int64_t)t * R + r] = bit ? rcnt_w[w * R + r] + popc64(b & lt) : -1;
        }
    }
}

// Block-wide exclusive scan of two ints per thread at once (kFinalThreads threads).  Returns the exclusive
// prefixes in ex0/ex1 and the block totals in all0/all1.  `scratch` holds 2 * kFinalThreads / 64 ints.
__device__ void block_exclusive_scan2(int v0, int v1, int* scratch, int& ex0, int& ex1, int& all0, int& all1) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    constexpr int nw = kFinalThreads / 64;
    int i0 = v0, i1 = v1;
    for (int off = 1; off < 64; off <<= 1) {
        const int u0 = __shfl_up(i0, off), u1 = __shfl_up(i1, off);
        if (lane >= off) {
            i0 += u0;
            i1 += u1;
        }
    }
    if (lane == 63) {
        scratch[w] = i0;
        scratch[nw + w] = i1;
    }
    __syncthreads();
    int b0 = 0, b1 = 0, a0 = 0, a1 = 0;
    for (int i = 0; i < nw; ++i) {
        const int s0 = scratch[i], s1 = scratch[nw + i];
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

constexpr int kMaxEntriesPerThread = kTile * kMaxTopk / kFinalThreads;   // 8
constexpr int kMaxCols = kMaxExperts + kMaxRanks + 1;                   // columns of a tile row

__global__ __launch_bounds__(kFinalThreads) void k_layout_finalize(
    int T, int K, int E, int R, int rank, int epr, int A, int ntiles, const int32_t* __restrict__ tile_hist,
    int32_t* __restrict__ slot, int32_t* __restrict__ send_slot, int32_t* __restrict__ cnt_local,
    int32_t* __restrict__ psum_ws, int32_t* __restrict__ pad_rows, int32_t* __restrict__ pad_total,
    int32_t* __restrict__ out_ntok_rank, int32_t* __restrict__ out_ntok_expert, int32_t* __restrict__ out_psum,
    int32_t* __restrict__ out_invalid) {
    __shared__ int part_before[kMaxCols];
    __shared__ int part_total[kMaxCols];
    __shared__ int before[kMaxCols];
    __shared__ int total[kMaxCols];
    __shared__ int psum[kMaxExperts + 1];
    __shared__ int padpre[kMaxExperts + 1];
    __shared__ int scan_scratch[2 * kFinalThreads / 64];

    const int tid = threadIdx.x;
    const int tile = blockIdx.x;
    const int lo = rank * epr;
    const int NC = E + R + 1;                          // columns: experts | ranks | invalid
    const int tok_tile0 = tile * kTile;
    const int ntok = tile < ntiles ? min(kTile, T - tok_tile0) : 0;
    const int64_t ent0 = (int64_t)tok_tile0 * K;

    // prefetch this tile's packed entries (independent of the sums below)
    int pk[kMaxEntriesPerThread];
#pragma unroll
    for (int i = 0; i < kMaxEntriesPerThread; ++i) {
        const int j = tid + i * kFinalThreads;
        pk[i] = j < ntok * K ? slot[ent0 + j] : -1;
    }

    // ---- column sums of the tile rows: (part, column) per thread, all loads independent -------------------
    const int P = NC <= kFinalThreads ? kFinalThreads / NC : 1;
    for (int q = tid; q < P * NC; q += kFinalThreads) {
        const int col = q % NC, part = q / NC;
        const int t0 = (int)((int64_t)part * ntiles / P), t1 = (int)((int64_t)(part + 1) * ntiles / P);
        int sb = 0, st = 0;
        int ti = t0;
        for (; ti + 4 <= t1; ti += 4) {
            const int v0 = tile_hist[(int64_t)ti * NC + col], v1 = tile_hist[(int64_t)(ti + 1) * NC + col];
            const int v2 = tile_hist[(int64_t)(ti + 2) * NC + col], v3 = tile_hist[(int64_t)(ti + 3) * NC + col];
            st += v0 + v1 + v2 + v3;
            sb += (ti < tile ? v0 : 0) + (ti + 1 < tile ? v1 : 0) + (ti + 2 < tile ? v2 : 0) + (ti + 3 < tile ? v3 : 0);
        }
        for (; ti < t1; ++ti) {
            const int v = tile_hist[(int64_t)ti * NC + col];
            st += v;
            if (ti < tile) sb += v;
        }
        part_before[q] = sb;
        part_total[q] = st;
    }
    __syncthreads();
    for (int col = tid; col < NC; col += kFinalThreads) {
        int sb = 0, st = 0;
        for (int p = 0; p < P; ++p) {
            sb += part_before[p * NC + col];
            st += part_total[p * NC + col];
        }
        before[col] = sb;
        total[col] = st;
    }
    __syncthreads();

    // ---- aligned exclusive starts of the local experts, and the padding-row prefix --------------------------
    {
        const int c = tid < epr ? total[lo + tid] : 0;
        const int padded = ((c + A - 1) / A) * A;
        int ex, expad, all, allpad;
        block_exclusive_scan2(padded, padded - c, scan_scratch, ex, expad, all, allpad);
        if (tid < epr) {
            psum[tid] = ex;
            padpre[tid] = expad;
        }
        if (tid == 0) {
            psum[epr] = all;
            padpre[epr] = allpad;
        }
    }
    __syncthreads();

    if (tile == 0) {
        for (int e = tid; e < E; e += kFinalThreads)
            if (out_ntok_expert) out_ntok_expert[e] = total[e];
        for (int j = tid; j <= epr; j += kFinalThreads) {
            psum_ws[j] = psum[j];
            if (out_psum) out_psum[j] = psum[j];
            if (j < epr) cnt_local[j] = total[lo + j];
        }
        if (tid < R && out_ntok_rank) out_ntok_rank[tid] = total[E + tid];
        if (tid == 0) {
            *pad_total = padpre[epr];
            if (out_invalid) *out_invalid = total[E + R];
        }
    }

    // ---- dense list of padding rows: this block's share of the local experts ---------------------------------
    if (pad_rows != nullptr) {
        // this block's share: local experts j = blockIdx.x + i * gridDim.x; item q = (i, r) with r < A - 1
        const int nexp = (epr - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
        for (int q = tid; q < nexp * (A - 1); q += kFinalThreads) {
            const int i = q / (A - 1), r = q % (A - 1);
            const int j = blockIdx.x + i * gridDim.x;
            const int first = psum[j] + total[lo + j];
            if (r < psum[j + 1] - first) pad_rows[padpre[j] + r] = first + r;
        }
    }
    if (tile >= ntiles) return;   // T == 0: the single block only wrote the global outputs

    // ---- final rows of this tile's entries ---------------------------------------------------------------
#pragma unroll
    for (int i = 0; i < kMaxEntriesPerThread; ++i) {
        const int j = tid + i * kFinalThreads;
        if (j < ntok * K) {
            const int p = pk[i];
            int s = -1;
            if (p >= 0) {
                const int e = p & kPackMask;
                if (e >= lo && e < lo + epr) s = psum[e - lo] + before[e] + (p >> kPackShift);
            }
            slot[ent0 + j] = s;
        }
    }
    if (send_slot != nullptr) {
        for (int q = tid; q < ntok * R; q += kFinalThreads) {
            const int r = q % R;
            const int64_t i = (int64_t)tok_tile0 * R + q;
            const int v = send_slot[i];
            send_slot[i] = (r != rank && v >= 0) ? before[E + r] + v : -1;
        }
    }
}

}  // namespace

hipError_t launch_layout(const Handle& h, const LayoutOutputs& out, hipStream_t stream) {
    const int epr = h.El;
    int nbits = 0;
    while ((1 << nbits) < h.E) ++nbits;
    int32_t* send = h.R > 1 ? h.ws.send_slot : nullptr;
    if (h.ntiles > 0) {
        const size_t lds = ((sizeof(uint16_t) * kCountWaves * (size_t)h.E + 15) & ~(size_t)15) +
                           sizeof(int32_t) * ((size_t)kTile * h.K + 4 * (size_t)h.R + kCountWaves);
        if (lds > 65536) {   // only large E and K together: opt in to more than 64 KiB of LDS (gfx950 has 160 KiB)
            static std::once_flag once;
            static hipError_t attr_err = hipSuccess;
            std::call_once(once, [] {
                const size_t max_lds = sizeof(uint16_t) * kCountWaves * kMaxExperts +
                                       sizeof(int32_t) * ((size_t)kTile * kMaxTopk + 4 * kMaxRanks + kCountWaves);
                attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(k_layout_count),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)max_lds);
            });
            if (attr_err != hipSuccess) return attr_err;
        }
        hipLaunchKernelGGL(k_layout_count, dim3(h.ntiles), dim3(kCountThreads), lds, stream, h.topk_idx, h.T, h.K, h.E, h.R,
                           epr, nbits, h.ws.tile_hist, h.ws.slot, send, out.is_token_in_rank);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(k_layout_finalize, dim3(h.ntiles > 0 ? h.ntiles : 1), dim3(kFinalThreads), 0, stream, h.T, h.K,
                       h.E, h.R, h.rank, epr, h.A, h.ntiles, h.ws.tile_hist, h.ws.slot, send, h.ws.cnt_local, h.ws.psum, h.ws.pad_rows, h.ws.pad_total, out.num_tokens_per_rank,
                       out.num_tokens_per_expert, out.psum, out.num_invalid);
    return hipGetLastError();
}

}  // namespace ep
