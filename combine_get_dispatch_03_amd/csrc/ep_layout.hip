// ep_layout.hip -- layout of a routing table on gfx950: a stable counting sort of the routed entries by
// expert, plus per-rank membership ([repo-map] §2.1: layout.cu gives rank counts, expert counts and
// token-in-rank membership; [DeepEP->MegaMoE] §2.2: per-expert counts and their prefix sum; §2.4: the prefix
// sum is each expert's start cursor; the same page's cross-reference names the scheme a counting sort).
//
// Deterministic throughout (no atomics decide a position).  Work is cut into 256-token tiles.
//   counting phase     (one 1024-thread block per tile) the tile's entries are staged in LDS with one
//                      cooperative load; each of 16 waves ranks its 16 tokens' entries in flat order with
//                      key-bit ballots (peers = lanes holding the same expert) against a per-wave LDS
//                      histogram; the block turns per-wave counts into per-wave bases and tile totals
//                      (expert counts | token-in-rank counts | invalid entries).
//   finalizing phase   totals over all tiles and each tile's base from the tiles before it, one fused scan of
//                      (aligned count, padding count) over the local experts into psum and the padding
//                      prefix, global counts, the dense padding-row list, and the final row of every entry.
// More than one tile: k_layout_count (counting, tile rows + tile-local ranks to the workspace) then
// k_layout_finalize (one block per tile, each re-summing the tile rows it needs).  One tile (<= 256 tokens,
// the decode shape): k_layout_single does both phases in one block without leaving LDS, in one launch.
#include <mutex>

#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {

extern __shared__ __align__(16) unsigned char layout_smem[];   // dynamic LDS of the counting phase

namespace {

constexpr int kTile = kLayoutTileTokens;   // 256 tokens per tile
constexpr int kThreads = 1024;             // every layout block: 16 waves
constexpr int kWaves = kThreads / 64;
constexpr int kTokPerWave = kTile / kWaves;   // 16 tokens ranked per wave
constexpr int kPackShift = 11;             // packed entry: (rank << 11) | expert, or -1
constexpr int kPackMask = (1 << kPackShift) - 1;
constexpr int kBad = -2;                   // staged value of an entry < -1 or >= E
constexpr int kMaxEntriesPerThread = kTile * kMaxTopk / kThreads;   // 8
constexpr int kMaxCols = kMaxExperts + kMaxRanks + 1;               // columns of a tile row

// ---- LDS of the counting phase ---------------------------------------------------------------------------
struct CountLds {
    uint16_t* cnt_w;   // [16][E]   per-wave counts, then per-wave exclusive bases within the tile
    int32_t* ent;      // [256*K]   staged entries, then (wave-local rank << 11) | expert, or -1
    int32_t* rcnt_w;   // [4][R]    per-wave token-in-rank counts, then exclusive bases (waves 0..3)
    int32_t* inv_w;    // [16]      per-wave invalid entries
    int32_t* row;      // [E+R+1]   tile totals: expert counts | token-in-rank counts | invalid
};

__host__ __device__ constexpr size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

__host__ __device__ size_t count_lds_bytes(int E, int K, int R) {
    return align16(sizeof(uint16_t) * kWaves * (size_t)E) +
           sizeof(int32_t) * ((size_t)kTile * K + 4 * (size_t)R + kWaves + (size_t)(E + R + 1));
}

__device__ CountLds carve_count(unsigned char* base, int E, int K, int R) {
    CountLds L;
    L.cnt_w = reinterpret_cast<uint16_t*>(base);
    L.ent = reinterpret_cast<int32_t*>(base + align16(sizeof(uint16_t) * kWaves * (size_t)E));
    L.rcnt_w = L.ent + kTile * K;
    L.inv_w = L.rcnt_w + 4 * R;
    L.row = L.inv_w + kWaves;
    return L;
}

// Counting phase for one tile.  Every thread of the block calls it; it ends with a barrier.  Returns, for
// threads 0..255, the bit mask of ranks that token (tile start + tid) has an expert on (0 for others).
__device__ uint64_t count_tile(const int64_t* __restrict__ idx, int T, int K, int E, int R, int epr, int nbits,
                               int tile, const CountLds& L, uint8_t* __restrict__ in_rank_out) {
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int tok_tile0 = tile * kTile;
    const int64_t ent_tile0 = (int64_t)tok_tile0 * K;
    const int nent_tile = max(0, min(kTile, T - tok_tile0)) * K;

    // stage the tile's entries (one round trip: all loads issued before any is used)
    for (int j0 = 0; j0 < nent_tile; j0 += 8 * kThreads) {
        int64_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + u * kThreads + tid;
            v[u] = j < nent_tile ? idx[ent_tile0 + j] : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + u * kThreads + tid;
            if (j < nent_tile) L.ent[j] = (v[u] >= 0 && v[u] < E) ? (int)v[u] : (v[u] == -1 ? -1 : kBad);
        }
    }
    for (int i = tid; i < kWaves * E; i += kThreads) L.cnt_w[i] = 0;
    __syncthreads();

    // each wave ranks its 16 tokens' entries in flat order
    const int nent_w = max(0, min(kTokPerWave, T - (tok_tile0 + w * kTokPerWave))) * K;
    int32_t* went = L.ent + w * kTokPerWave * K;
    const uint64_t lt = lanemask_lt();
    uint16_t* cnt = L.cnt_w + w * E;
    int inv = 0;
    for (int j0 = 0; j0 < nent_w; j0 += 64) {
        const int j = j0 + lane;
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
    if (lane == 0) L.inv_w[w] = inv;
    __syncthreads();

    // per-wave counts -> per-wave exclusive bases; tile totals
    for (int e = tid; e < E; e += kThreads) {
        int c[kWaves];
#pragma unroll
        for (int v = 0; v < kWaves; ++v) c[v] = L.cnt_w[v * E + e];
        int run = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            L.cnt_w[v * E + e] = (uint16_t)run;
            run += c[v];
        }
        L.row[e] = run;
    }
    // threads 0..255 <-> tokens of the tile (waves 0..3): token-in-rank membership
    const int t = tok_tile0 + tid;
    const bool tv = tid < kTile && t < T;
    uint64_t mask = 0ull;
    if (tv) {
        for (int k = 0; k < K; ++k) {
            const int p = L.ent[tid * K + k];
            if (p >= 0) mask |= 1ull << ((p & kPackMask) / epr);
        }
    }
    if (tv && in_rank_out != nullptr)
        for (int r = 0; r < R; ++r) in_rank_out[(int64_t)t * R + r] = (uint8_t)((mask >> r) & 1ull);
    if (w < 4) {
        for (int r = 0; r < R; ++r) {
            const uint64_t b = ballot((mask >> r) & 1ull);
            if (lane == 0) L.rcnt_w[w * R + r] = popc64(b);
        }
    }
    __syncthreads();
    if (tid < R) {
        const int c0 = L.rcnt_w[tid], c1 = L.rcnt_w[R + tid], c2 = L.rcnt_w[2 * R + tid], c3 = L.rcnt_w[3 * R + tid];
        L.rcnt_w[tid] = 0;
        L.rcnt_w[R + tid] = c0;
        L.rcnt_w[2 * R + tid] = c0 + c1;
        L.rcnt_w[3 * R + tid] = c0 + c1 + c2;
        L.row[E + tid] = c0 + c1 + c2 + c3;
    }
    if (tid == 0) {
        int s = 0;
        for (int v = 0; v < kWaves; ++v) s += L.inv_w[v];
        L.row[E + R] = s;
    }
    __syncthreads();
    return mask;
}

// Per-rank token rows of the tile's tokens, from the rank masks of count_tile: the rank of the token among the
// tile's earlier tokens with an expert on r (tile-local), or -1 when it has none there.
__device__ void send_rows(const CountLds& L, uint64_t mask, int T, int R, int tile, int32_t* __restrict__ out) {
    const int tid = threadIdx.x, w = tid >> 6;
    if (w >= 4) return;
    const int t = tile * kTile + tid;
    const bool tv = t < T;
    const uint64_t lt = lanemask_lt();
    for (int r = 0; r < R; ++r) {
        const bool bit = (mask >> r) & 1ull;
        const uint64_t b = ballot(bit);
        if (tv) out[(int64_t)t * R + r] = bit ? L.rcnt_w[w * R + r] + popc64(b & lt) : -1;
    }
}

// Block-wide exclusive scan of two ints per thread at once (kThreads threads).  Returns the exclusive
// prefixes in ex0/ex1 and the block totals in all0/all1.  `scratch` holds 2 * kWaves ints.
__device__ void block_exclusive_scan2(int v0, int v1, int* scratch, int& ex0, int& ex1, int& all0, int& all1) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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

// Finalizing phase shared by both paths.  `total` holds the column totals over all tiles (experts | ranks |
// invalid).  Computes psum / padpre (LDS), block 0 writes the global outputs, and every block writes its
// share (experts blockIdx.x + i * gridDim.x) of the dense padding-row list.
__device__ void finalize_core(int E, int R, int rank, int epr, int A, const int* total, int* psum, int* padpre,
                              int* scratch, const Outputs& o) {
    const int tid = threadIdx.x;
    const int lo = rank * epr;
    {
        const int c = tid < epr ? total[lo + tid] : 0;
        const int padded = ((c + A - 1) / A) * A;
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
    }
    __syncthreads();
    if (blockIdx.x == 0) {
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
    if (o.pad_rows != nullptr) {
        // this block's share: local experts blockIdx.x + i * gridDim.x, one expert per wave, lanes over its rows
        const int nexp = (epr - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
        const int w = tid >> 6, lane = tid & 63;
        for (int i = w; i < nexp; i += kWaves) {
            const int j = blockIdx.x + i * gridDim.x;
            const int first = psum[j] + total[lo + j];
            const int n = psum[j + 1] - first;
            int32_t* dst = o.pad_rows + padpre[j];
            for (int r = lane; r < n; r += 64) dst[r] = first + r;
        }
    }
}

// ---- multi-tile path -------------------------------------------------------------------------------------

__global__ __launch_bounds__(kThreads) void k_layout_count(
    const int64_t* __restrict__ idx, int T, int K, int E, int R, int epr, int nbits,
    int32_t* __restrict__ tile_hist, int32_t* __restrict__ packed_out, int32_t* __restrict__ send_tmp,
    uint8_t* __restrict__ in_rank_out) {
    const CountLds L = carve_count(layout_smem, E, K, R);
    const int tid = threadIdx.x;
    const int tile = blockIdx.x;
    const int NC = E + R + 1;
    const uint64_t mask = count_tile(idx, T, K, E, R, epr, nbits, tile, L, in_rank_out);
    for (int c = tid; c < NC; c += kThreads) tile_hist[(int64_t)tile * NC + c] = L.row[c];
    const int64_t ent_tile0 = (int64_t)tile * kTile * K;
    const int nent_tile = max(0, min(kTile, T - tile * kTile)) * K;
    for (int j = tid; j < nent_tile; j += kThreads) {
        const int p = L.ent[j];
        const int wv = (j / K) / kTokPerWave;
        packed_out[ent_tile0 + j] =
            p < 0 ? -1 : (((p >> kPackShift) + L.cnt_w[wv * E + (p & kPackMask)]) << kPackShift) | (p & kPackMask);
    }
    send_rows(L, mask, T, R, tile, send_tmp);   // tile-local; finalize adds the earlier tiles' counts
}

__global__ __launch_bounds__(kThreads) void k_layout_finalize(
    int T, int K, int E, int R, int rank, int epr, int A, int ntiles, const int32_t* __restrict__ tile_hist,
    int32_t* __restrict__ slot, int32_t* __restrict__ send_slot, Outputs o) {
    __shared__ int part_before[kMaxCols];
    __shared__ int part_total[kMaxCols];
    __shared__ int before[kMaxCols];
    __shared__ int total[kMaxCols];
    __shared__ int psum[kMaxExperts + 1];
    __shared__ int padpre[kMaxExperts + 1];
    __shared__ int scan_scratch[2 * kWaves];

    const int tid = threadIdx.x;
    const int tile = blockIdx.x;
    const int lo = rank * epr;
    const int NC = E + R + 1;
    const int tok_tile0 = tile * kTile;
    const int ntok = tile < ntiles ? min(kTile, T - tok_tile0) : 0;
    const int64_t ent0 = (int64_t)tok_tile0 * K;

    // prefetch this tile's packed entries (independent of the sums below)
    int pk[kMaxEntriesPerThread];
#pragma unroll
    for (int i = 0; i < kMaxEntriesPerThread; ++i) {
        const int j = tid + i * kThreads;
        pk[i] = j < ntok * K ? slot[ent0 + j] : -1;
    }

    // column sums of the tile rows: (part, column) per thread, all loads independent
    const int P = NC <= kThreads ? kThreads / NC : 1;
    for (int q = tid; q < P * NC; q += kThreads) {
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
    for (int col = tid; col < NC; col += kThreads) {
        int sb = 0, st = 0;
        for (int p = 0; p < P; ++p) {
            sb += part_before[p * NC + col];
            st += part_total[p * NC + col];
        }
        before[col] = sb;
        total[col] = st;
    }
    __syncthreads();

    finalize_core(E, R, rank, epr, A, total, psum, padpre, scan_scratch, o);
    if (tile >= ntiles) return;   // T == 0: the single block only wrote the global outputs

    // final rows of this tile's entries
#pragma unroll
    for (int i = 0; i < kMaxEntriesPerThread; ++i) {
        const int j = tid + i * kThreads;
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
    for (int q = tid; q < ntok * R; q += kThreads) {
        const int r = q % R;
        const int64_t i = (int64_t)tok_tile0 * R + q;
        const int v = send_slot[i];
        send_slot[i] = v >= 0 ? before[E + r] + v : -1;
    }
}

// ---- single-tile path (T <= 256): both phases in one block, one launch ------------------------------------

__global__ __launch_bounds__(kThreads) void k_layout_single(
    const int64_t* __restrict__ idx, int T, int K, int E, int R, int rank, int epr, int A, int nbits,
    int32_t* __restrict__ slot, int32_t* __restrict__ send_slot, uint8_t* __restrict__ in_rank_out, Outputs o) {
    const CountLds L = carve_count(layout_smem, E, K, R);
    int* psum = reinterpret_cast<int*>(layout_smem + count_lds_bytes(E, K, R));   // [epr + 1]
    int* padpre = psum + epr + 1;                                                 // [epr + 1]
    int* scratch = padpre + epr + 1;                                              // [2 * kWaves]
    const int tid = threadIdx.x;
    const int lo = rank * epr;
    const uint64_t mask = count_tile(idx, T, K, E, R, epr, nbits, 0, L, in_rank_out);
    finalize_core(E, R, rank, epr, A, L.row, psum, padpre, scratch, o);
    for (int j = tid; j < T * K; j += kThreads) {
        const int p = L.ent[j];
        int s = -1;
        if (p >= 0) {
            const int e = p & kPackMask;
            const int wv = (j / K) / kTokPerWave;
            if (e >= lo && e < lo + epr) s = psum[e - lo] + L.cnt_w[wv * E + e] + (p >> kPackShift);
        }
        slot[j] = s;
    }
    send_rows(L, mask, T, R, 0, send_slot);
}

size_t single_lds_bytes(int E, int K, int R, int epr) {
    return count_lds_bytes(E, K, R) + sizeof(int) * (2 * (size_t)(epr + 1) + 2 * kWaves);
}

// Opt a kernel in to more than 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU); once per kernel.
hipError_t allow_lds(const void* kernel, size_t max_bytes, std::once_flag& once, hipError_t& err) {
    std::call_once(once, [&] {
        err = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)max_bytes);
    });
    return err;
}

}  // namespace

hipError_t launch_layout(const Handle& h, const LayoutOutputs& out, hipStream_t stream) {
    const int epr = h.El;
    int nbits = 0;
    while ((1 << nbits) < h.E) ++nbits;
    int32_t* send = h.ws.send_slot;
    const Outputs o{h.ws.cnt_local, h.ws.psum, h.ws.pad_rows, h.ws.pad_total, out.num_tokens_per_rank,
                    out.num_tokens_per_expert, out.psum, out.num_invalid};

    if (h.ntiles == 1) {
        const size_t lds = single_lds_bytes(h.E, h.K, h.R, epr);
        if (lds > 65536) {
            static std::once_flag once;
            static hipError_t err = hipSuccess;
            if (allow_lds(reinterpret_cast<const void*>(k_layout_single),
                          single_lds_bytes(kMaxExperts, kMaxTopk, kMaxRanks, kMaxExperts), once, err) != hipSuccess)
                return err;
        }
        hipLaunchKernelGGL(k_layout_single, dim3(1), dim3(kThreads), lds, stream, h.topk_idx, h.T, h.K, h.E, h.R,
                           h.rank, epr, h.A, nbits, h.ws.slot, send, out.is_token_in_rank, o);
        return hipGetLastError();
    }
    if (h.ntiles > 1) {
        const size_t lds = count_lds_bytes(h.E, h.K, h.R);
        if (lds > 65536) {
            static std::once_flag once;
            static hipError_t err = hipSuccess;
            if (allow_lds(reinterpret_cast<const void*>(k_layout_count),
                          count_lds_bytes(kMaxExperts, kMaxTopk, kMaxRanks), once, err) != hipSuccess)
                return err;
        }
        hipLaunchKernelGGL(k_layout_count, dim3(h.ntiles), dim3(kThreads), lds, stream, h.topk_idx, h.T, h.K, h.E,
                           h.R, epr, nbits, h.ws.tile_hist, h.ws.slot, send, out.is_token_in_rank);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // T == 0 lands here with ntiles == 0: one finalize block writes the (zero) global outputs
    hipLaunchKernelGGL(k_layout_finalize, dim3(h.ntiles > 0 ? h.ntiles : 1), dim3(kThreads), 0, stream, h.T, h.K,
                       h.E, h.R, h.rank, epr, h.A, h.ntiles, h.ws.tile_hist, h.ws.slot, send, o);
    return hipGetLastError();
}

}  // namespace ep
