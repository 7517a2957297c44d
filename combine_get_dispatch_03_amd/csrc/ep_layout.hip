// ep_layout.hip -- layout of a routing table on gfx950: a stable counting sort of the routed entries by
// expert, plus per-rank membership ([repo-map] §2.1: layout.cu gives rank counts, expert counts and
// token-in-rank membership; [DeepEP->MegaMoE] §2.2: per-expert counts and their prefix sum; §2.4: the prefix
// sum is each expert's start cursor; the same page's cross-reference names the scheme a counting sort).
//
// Deterministic throughout: no atomic operation decides a position (the one-tile path counts with LDS atomic
// adds, whose totals do not depend on their order).  Work is cut into 256-token tiles.
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
// the decode shape): k_layout_tokens, one launch of one workgroup per token; each stages the table, counts the
// column totals and the entries and tokens before its own token, scans, and writes that token's rows, which
// follow from those counts alone (no ranking of the table).
#include <algorithm>

#include "ep_layout_core.hpp"

namespace ep {

namespace {

// ---- multi-tile path: counting phase, finalizing phase --------------------------------------------------

constexpr int kPackShift = 11;             // packed entry: (rank << 11) | expert, or -1
constexpr int kPackMask = (1 << kPackShift) - 1;
// The token-mask work runs on the last 4 waves, so that for E <= 768 it overlaps the per-expert bases loop (which
// runs on threads 0..E-1) instead of following it on the same threads.
constexpr int kTokThread0 = kThreads - kTile;
constexpr int kTokWave0 = kTokThread0 / 64;
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

// Tokens ranked per wave in tile `tile`: the tile's tokens spread evenly over the 16 waves (16 for a full tile,
// fewer for a ragged last tile, so that no wave runs two ranking rounds while others idle).  Wave w ranks tokens
// [w * tpw, (w + 1) * tpw) of the tile; every reader of the per-wave bases uses the same split.
__device__ __forceinline__ int tokens_per_wave(int T, int tile) {
    const int ntok = max(0, min(kTile, T - tile * kTile));
    return max(1, (ntok + kWaves - 1) / kWaves);
}

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

// Counting phase for one tile.  Every thread of the block calls it; it ends with a barrier.  Returns, for the
// token threads (the last 256 threads: token = tile start + tid - kTokThread0), the bit mask of ranks that the
// token has an expert on (0 for the other threads).
__device__ uint64_t count_tile(const int64_t* __restrict__ idx, int T, int K, int E, int R, int epr, int nbits,
                               int tile, const CountLds& L, uint8_t* __restrict__ in_rank_out) {
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int tok_tile0 = tile * kTile;
    const int64_t ent_tile0 = (int64_t)tok_tile0 * K;
    const int nent_tile = max(0, min(kTile, T - tok_tile0)) * K;

    // stage the tile's entries: at most 256 * 32 = 8 per thread, all loads issued before any is used
    static_assert(kTile * kMaxTopk <= kMaxEntriesPerThread * kThreads, "one staging pass per tile");
    int64_t v[kMaxEntriesPerThread];
#pragma unroll
    for (int u = 0; u < kMaxEntriesPerThread; ++u) {
        const int j = u * kThreads + tid;
        v[u] = j < nent_tile ? idx[ent_tile0 + j] : -1;
    }
#pragma unroll
    for (int u = 0; u < kMaxEntriesPerThread; ++u) {
        const int j = u * kThreads + tid;
        if (j < nent_tile) L.ent[j] = (v[u] >= 0 && v[u] < E) ? (int)v[u] : (v[u] == -1 ? -1 : kBad);
    }
    for (int i = tid; i < kWaves * E; i += kThreads) L.cnt_w[i] = 0;
    __syncthreads();

    // each wave ranks its 16 tokens' entries in flat order
    const int tpw = tokens_per_wave(T, tile);
    const int nent_w = max(0, min(tpw, T - (tok_tile0 + w * tpw))) * K;
    int32_t* went = L.ent + w * tpw * K;
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
    // token threads (waves kTokWave0..kTokWave0+3) <-> tokens of the tile: token-in-rank membership
    const int tt = tid - kTokThread0;
    const int t = tok_tile0 + tt;
    const bool tv = tt >= 0 && t < T;
    // expert -> owning rank as floor((e + 0.5) / epr) in fp32: exact here, since for e < 1024 and epr <= 1024 the
    // quotient lies at least 0.5 / epr >= 2^-11 from an integer and the two roundings move it by < 2^-13
    const float inv_epr = 1.0f / (float)epr;
    uint64_t mask = 0ull;
    if (tv) {
        for (int k = 0; k < K; ++k) {
            const int p = L.ent[tt * K + k];
            if (p >= 0) mask |= 1ull << (int)(((float)(p & kPackMask) + 0.5f) * inv_epr);
        }
    }
    if (tv && in_rank_out != nullptr)
        for (int r = 0; r < R; ++r) in_rank_out[(int64_t)t * R + r] = (uint8_t)((mask >> r) & 1ull);
    if (w >= kTokWave0) {
        for (int r = 0; r < R; ++r) {
            const uint64_t b = ballot((mask >> r) & 1ull);
            if (lane == 0) L.rcnt_w[(w - kTokWave0) * R + r] = popc64(b);
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
// tile's earlier tokens with an expert on r (tile-local), or -1 when it has none there; handed to
// put(t, r, row).  The token threads of count_tile (one token each) take part.
template <class Put>
__device__ __forceinline__ void token_rows(const CountLds& L, uint64_t mask, int T, int R, int tile, Put put) {
    const int tid = threadIdx.x, w = tid >> 6;
    if (w < kTokWave0) return;
    const int t = tile * kTile + tid - kTokThread0;
    const bool tv = t < T;
    const uint64_t lt = lanemask_lt();
    for (int r = 0; r < R; ++r) {
        const bool bit = (mask >> r) & 1ull;
        const uint64_t b = ballot(bit);
        if (tv) put(t, r, bit ? L.rcnt_w[(w - kTokWave0) * R + r] + popc64(b & lt) : -1);
    }
}

__device__ void send_rows(const CountLds& L, uint64_t mask, int T, int R, int tile, int32_t* __restrict__ out) {
    token_rows(L, mask, T, R, tile, [&](int t, int r, int v) { out[(int64_t)t * R + r] = v; });
}

// Finalizing phase of the multi-tile path.  `total` holds the column totals over all tiles (experts |
// ranks | invalid).  Computes psum / padpre (LDS), block 0 writes the global outputs, and each of the nblk
// layout blocks writes its share (experts blockIdx.x + i * nblk) of the dense padding-row list.
__device__ void finalize_core(int E, int R, int rank, int epr, int A, const int* total, int* psum, int* padpre,
                              int* scratch, const Outputs& o, int nblk) {
    const int tid = threadIdx.x;
    const int lo = rank * epr;
    local_scan(epr, lo, A, total, psum, padpre, scratch);
    if (blockIdx.x == 0) write_counts(E, R, lo, epr, total, psum, padpre, o);
    if (o.pad_rows != nullptr) {
        // this block's share: local experts blockIdx.x + i * nblk, one expert per wave, lanes over its rows
        const int nexp = (epr - (int)blockIdx.x + nblk - 1) / nblk;
        const int w = tid >> 6, lane = tid & 63;
        for (int i = w; i < nexp; i += kWaves) {
            const int j = blockIdx.x + i * nblk;
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
    const int tpw = tokens_per_wave(T, tile);
    for (int j = tid; j < nent_tile; j += kThreads) {
        const int p = L.ent[j];
        const int wv = (j / K) / tpw;
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

    // column sums of the tile rows: (part, column) per thread; its tiles are read 8 at a time, all 8 loads in
    // flight together (one round trip per 8 tiles)
    const int P = NC <= kThreads ? kThreads / NC : 1;
    for (int q = tid; q < P * NC; q += kThreads) {
        const int col = q % NC, part = q / NC;
        const int t0 = (int)((int64_t)part * ntiles / P), t1 = (int)((int64_t)(part + 1) * ntiles / P);
        int sb = 0, st = 0;
        for (int ti = t0; ti < t1; ti += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = ti + u < t1 ? tile_hist[(int64_t)(ti + u) * NC + col] : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                st += v[u];
                sb += ti + u < tile ? v[u] : 0;
            }
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

    finalize_core(E, R, rank, epr, A, total, psum, padpre, scan_scratch, o, (int)gridDim.x);
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

// ---- single-tile path (T <= 256): one launch, one workgroup per token -------------------------------------
// Workgroup t stages the table and counts in LDS (tok_counts in ep_layout_core.hpp), then its last wave writes
// token t's slots, per-rank rows and membership; block 0 writes the counts; wave g of the grid writes the
// padding rows of the local experts g, g + waves, ...
__global__ __launch_bounds__(kThreads) void k_layout_tokens(
    const int64_t* __restrict__ idx, int T, int K, int E, int R, int rank, int epr, int A,
    int32_t* __restrict__ slot, int32_t* __restrict__ send_slot, uint8_t* __restrict__ in_rank_out, Outputs o) {
    // idx, 7 ints (+ 4 bytes of alignment), 3 pointers, then o
    constexpr int kArgBytes = 8 + 7 * 4 + 4 + 3 * 8 + (int)sizeof(Outputs);
    static_assert(kArgBytes == 128, "k_layout_tokens arguments");
    touch_kernargs<kArgBytes>();
    const TokLds L = carve_tok(layout_smem, E, K, R, epr);
    const int lo = rank * epr, t = blockIdx.x, lane = lane_id(), w = threadIdx.x >> 6;
    // the token's rows on the last wave: their counting part runs while wave 0 scans
    const bool mine = t < T && w == kWaves - 1;
    TokRow tr;
    tok_counts(idx, T, K, E, R, epr, A, lo, t, L, [] {}, [&] {
        if (mine) tr = tok_row_counts(L, t, K);
    });
    if (blockIdx.x == 0) write_counts(E, R, lo, epr, L.tot, L.psum, L.padpre, o);
    if (mine) {
        const int sexp = tok_row_slot(L, tr, K, lo, epr), own = tok_row_own(L, tr, R);
        if (lane < K) slot[(int64_t)t * K + lane] = sexp;
        if (lane < R) {
            send_slot[(int64_t)t * R + lane] = own;
            if (in_rank_out) in_rank_out[(int64_t)t * R + lane] = own >= 0 ? 1 : 0;
        }
    }
    if (o.pad_rows != nullptr) {
        const int nw = (int)gridDim.x * kWaves;
        for (int j = w * (int)gridDim.x + (int)blockIdx.x; j < epr; j += nw) {
            const int first = L.psum[j] + L.tot[lo + j];
            const int n = L.psum[j + 1] - first;
            int32_t* dst = o.pad_rows + L.padpre[j];
            for (int r = lane; r < n; r += kWave) dst[r] = first + r;
        }
    }
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
        const size_t lds = tok_lds_bytes(h.E, h.K, h.R, epr);
        if (lds > 65536) {
            const hipError_t err = allow_dynamic_lds(reinterpret_cast<const void*>(k_layout_tokens), (int)lds);
            if (err != hipSuccess) return err;
        }
        // one workgroup per token, each repeating the counts in LDS
        hipLaunchKernelGGL(k_layout_tokens, dim3((unsigned)h.T), dim3(kThreads), lds, stream, h.topk_idx, h.T, h.K,
                           h.E, h.R, h.rank, epr, h.A, h.ws.slot, send,
                           out.is_token_in_rank, o);
        return hipGetLastError();
    }
    if (h.ntiles > 1) {
        const size_t lds = count_lds_bytes(h.E, h.K, h.R);
        if (lds > 65536) {
            const hipError_t err = allow_dynamic_lds(reinterpret_cast<const void*>(k_layout_count), (int)lds);
            if (err != hipSuccess) return err;
        }
        hipLaunchKernelGGL(k_layout_count, dim3((unsigned)h.ntiles), dim3(kThreads), lds, stream, h.topk_idx, h.T,
                           h.K, h.E, h.R, epr, nbits, h.ws.tile_hist, h.ws.slot, send, out.is_token_in_rank);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // T == 0 lands here with ntiles == 0: one finalize block writes the (zero) global outputs
    const unsigned nb_final = h.ntiles > 0 ? (unsigned)h.ntiles : 1u;
    hipLaunchKernelGGL(k_layout_finalize, dim3(nb_final), dim3(kThreads), 0, stream, h.T, h.K, h.E, h.R, h.rank,
                       epr, h.A, h.ntiles, h.ws.tile_hist, h.ws.slot, send, o);
    return hipGetLastError();
}

}  // namespace ep
