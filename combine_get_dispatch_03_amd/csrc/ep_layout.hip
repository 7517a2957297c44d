// ep_layout.hip -- layout of a routing table on gfx950: a stable counting sort of the routed entries by
// expert, plus per-rank membership ([repo-map] §2.1: layout.cu gives rank counts, expert counts and
// token-in-rank membership; [DeepEP->MegaMoE] §2.2: per-expert counts and their prefix sum; §2.4: the prefix
// sum is each expert's start cursor; "counting sort" is how the same page's cross-reference names it).
//
// Two launches, both deterministic (no atomics decide a position):
//   k_layout_count     one block per 256-token tile.  Each wave ranks its 64 tokens' entries in flat order
//                      with key-bit ballots (peers = lanes with the same expert) and a per-wave LDS
//                      histogram, then the block adds the earlier waves' counts.  Writes the tile's expert
//                      and rank histograms and each entry's tile-local rank.
//   k_layout_finalize  one block per tile.  Each block sums the tile histograms (all tiles for the totals,
//                      earlier tiles for its own base), scans the aligned local counts into psum, and turns
//                      tile-local ranks into final rows; block 0 also writes the global counts.
#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {
namespace {

constexpr int kTile = kLayoutTileTokens;   // 256 tokens = 4 waves x 64
constexpr int kFinalThreads = 1024;
constexpr int kPackShift = 11;             // packed entry: (tile-local rank << 11) | expert, or -1

__global__ __launch_bounds__(kTile) void k_layout_count(
    const int64_t* __restrict__ idx, int T, int K, int E, int R, int epr, int nbits,
    int32_t* __restrict__ tile_hist, int32_t* __restrict__ tile_rank, int32_t* __restrict__ tile_inv,
    int32_t* __restrict__ packed_out, int32_t* __restrict__ send_tmp, uint8_t* __restrict__ in_rank_out) {
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned long long* tokmask = reinterpret_cast<unsigned long long*>(smem);   // [256]
    int32_t* cnt_w = reinterpret_cast<int32_t*>(smem + sizeof(unsigned long long) * kTile);  // [4][E]
    int32_t* rcnt_w = cnt_w + 4 * E;                                             // [4][R]
    int32_t* inv_w = rcnt_w + 4 * R;                                             // [4]
    int32_t* packed = inv_w + 4;                                                 // [256 * K]

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int tile = blockIdx.x;
    const int tok_tile0 = tile * kTile;
    const int64_t ent_tile0 = (int64_t)tok_tile0 * K;

    for (int i = tid; i < 4 * E; i += kTile) cnt_w[i] = 0;
    tokmask[tid] = 0ull;
    __syncthreads();

    // ---- per wave: rank its 64 tokens' entries in flat order -------------------------------------------
    const int tok0 = tok_tile0 + w * 64;
    const int nent_w = max(0, min(64, T - tok0)) * K;
    const uint64_t lt = lanemask_lt();
    int32_t* cnt = cnt_w + w * E;
    int inv = 0;
    for (int c = 0; c < K; ++c) {
        const int j = c * 64 + lane;                       // entry index within the wave's tokens
        const bool in = j < nent_w;
        const int64_t e = in ? idx[(int64_t)tok0 * K + j] : -1;
        const bool ok = in && e >= 0 && e < E;
        inv += popc64(ballot(in && (e < -1 || e >= E)));
        const int key = ok ? (int)e : 0;
        const uint64_t peers = match_peers(key, ok, nbits);
        const int base = ok ? cnt[key] : 0;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (ok && (peers & lt) == 0) cnt[key] = base + popc64(peers);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        packed[w * 64 * K + j] = ok ? (((base + popc64(peers & lt)) << kPackShift) | key) : -1;
        if (ok) atomicOr(&tokmask[w * 64 + j / K], 1ull << (key / epr));
    }
    if (lane == 0) inv_w[w] = inv;
    __syncthreads();

    // ---- tile totals; turn the per-wave counts into exclusive per-wave bases ------------------------------
    for (int e = tid; e < E; e += kTile) {
        const int c0 = cnt_w[e], c1 = cnt_w[E + e], c2 = cnt_w[2 * E + e], c3 = cnt_w[3 * E + e];
        cnt_w[e] = 0;
        cnt_w[E + e] = c0;
        cnt_w[2 * E + e] = c0 + c1;
        cnt_w[3 * E + e] = c0 + c1 + c2;
        tile_hist[(int64_t)tile * E + e] = c0 + c1 + c2 + c3;
    }
    // thread tid <-> token tok_tile0 + tid (wave w holds its own 64 tokens)
    const int t = tok_tile0 + tid;
    const bool tv = t < T;
    const uint64_t mask = tv ? tokmask[tid] : 0ull;
    if (tv && in_rank_out != nullptr)
        for (int r = 0; r < R; ++r) in_rank_out[(int64_t)t * R + r] = (uint8_t)((mask >> r) & 1ull);
    for (int r = 0; r < R; ++r) {
        const uint64_t b = ballot((mask >> r) & 1ull);
        if (lane == 0) rcnt_w[w * R + r] = popc64(b);
    }
    __syncthreads();
    if (tid < R) {
        const int c0 = rcnt_w[tid], c1 = rcnt_w[R + tid], c2 = rcnt_w[2 * R + tid], c3 = rcnt_w[3 * R + tid];
        rcnt_w[tid] = 0;
        rcnt_w[R + tid] = c0;
        rcnt_w[2 * R + tid] = c0 + c1;
        rcnt_w[3 * R + tid] = c0 + c1 + c2;
        tile_rank[(int64_t)tile * R + tid] = c0 + c1 + c2 + c3;
    }
    if (tid == 0) tile_inv[tile] = inv_w[0] + inv_w[1] + inv_w[2] + inv_w[3];
    __syncthreads();

    // ---- tile-local ranks --------------------------------------------------------------------------------
    const int nent_tile = max(0, min(kTile, T - tok_tile0)) * K;
    for (int j = tid; j < nent_tile; j += kTile) {
        const int p = packed[j];
        const int wv = (j / K) >> 6;
        packed_out[ent_tile0 + j] =
            p < 0 ? -1 : (((p >> kPackShift) + cnt_w[wv * E + (p & ((1 << kPackShift) - 1))]) << kPackShift) |
                             (p & ((1 << kPackShift) - 1));
    }
    if (send_tmp != nullptr) {
        for (int r = 0; r < R; ++r) {
            const bool bit = (mask >> r) & 1ull;
            const uint64_t b = ballot(bit);
            if (tv) send_tmp[(int64_t)t * R + r] = bit ? rcnt_w[w * R + r] + popc64(b & lt) : -1;
        }
    }
}

// Block-wide exclusive scan of one int per thread (kFinalThreads threads); returns the exclusive prefix and
// sets *total.  `scratch` holds kFinalThreads / 64 ints.
__device__ int block_exclusive_scan(int v, int* scratch, int* total) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int incl = v;
    for (int off = 1; off < 64; off <<= 1) {
        const int u = __shfl_up(incl, off);
        if (lane >= off) incl += u;
    }
    if (lane == 63) scratch[w] = incl;
    __syncthreads();
    int wbase = 0, all = 0;
    for (int i = 0; i < kFinalThreads / 64; ++i) {
        const int s = scratch[i];
        if (i < w) wbase += s;
        all += s;
    }
    __syncthreads();
    *total = all;
    return wbase + incl - v;
}

__global__ __launch_bounds__(kFinalThreads) void k_layout_finalize(
    int T, int K, int E, int R, int rank, int epr, int A, int ntiles,
    const int32_t* __restrict__ tile_hist, const int32_t* __restrict__ tile_rank,
    const int32_t* __restrict__ tile_inv, int32_t* __restrict__ slot, int32_t* __restrict__ send_slot,
    int32_t* __restrict__ cnt_local, int32_t* __restrict__ psum_ws,
    int32_t* __restrict__ out_ntok_rank, int32_t* __restrict__ out_ntok_expert, int32_t* __restrict__ out_psum,
    int32_t* __restrict__ out_invalid) {
    __shared__ int part_before[kFinalThreads];
    __shared__ int part_total[kFinalThreads];
    __shared__ int before[kMaxExperts];
    __shared__ int total[kMaxExperts];
    __shared__ int psum[kMaxExperts + 1];
    __shared__ int rank_before[kMaxRanks];
    __shared__ int scan_scratch[kFinalThreads / 64];

    const int tid = threadIdx.x;
    const int tile = blockIdx.x;
    const int lo = rank * epr;

    // ---- column sums of the tile histograms: parts x experts threads ------------------------------------
    const int P = kFinalThreads / E;                   // >= 1 since E <= 1024
    if (tid < P * E) {
        const int e = tid % E, part = tid / E;
        const int t0 = (int)((int64_t)part * ntiles / P), t1 = (int)((int64_t)(part + 1) * ntiles / P);
        int sb = 0, st = 0;
        for (int ti = t0; ti < t1; ++ti) {
            const int v = tile_hist[(int64_t)ti * E + e];
            st += v;
            if (ti < tile) sb += v;
        }
        part_before[tid] = sb;
        part_total[tid] = st;
    }
    __syncthreads();
    for (int e = tid; e < E; e += kFinalThreads) {
        int sb = 0, st = 0;
        for (int p = 0; p < P; ++p) {
            sb += part_before[p * E + e];
            st += part_total[p * E + e];
        }
        before[e] = sb;
        total[e] = st;
    }
    if (tid < R) {
        int sb = 0;
        for (int ti = 0; ti < tile && ti < ntiles; ++ti) sb += tile_rank[(int64_t)ti * R + tid];
        rank_before[tid] = sb;
    }
    __syncthreads();

    // ---- aligned exclusive starts of the local experts ----------------------------------------------------
    {
        const int c = tid < epr ? total[lo + tid] : 0;
        const int padded = ((c + A - 1) / A) * A;
        int all = 0;
        const int ex = block_exclusive_scan(padded, scan_scratch, &all);
        if (tid < epr) psum[tid] = ex;
        if (tid == 0) psum[epr] = all;
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
        if (tid < R && out_ntok_rank) {
            int s = 0;
            for (int ti = 0; ti < ntiles; ++ti) s += tile_rank[(int64_t)ti * R + tid];
            out_ntok_rank[tid] = s;
        }
        if (tid == 0 && out_invalid) {
            int s = 0;
            for (int ti = 0; ti < ntiles; ++ti) s += tile_inv[ti];
            *out_invalid = s;
        }
    }
    if (tile >= ntiles) return;   // T == 0: the single block only wrote the global outputs

    // ---- final rows of this tile's entries ---------------------------------------------------------------
    const int tok_tile0 = tile * kTile;
    const int ntok = min(kTile, T - tok_tile0);
    const int64_t ent0 = (int64_t)tok_tile0 * K;
    const int mask = (1 << kPackShift) - 1;
    for (int j = tid; j < ntok * K; j += kFinalThreads) {
        const int p = slot[ent0 + j];
        int s = -1;
        if (p >= 0) {
            const int e = p & mask;
            if (e >= lo && e < lo + epr) s = psum[e - lo] + before[e] + (p >> kPackShift);
        }
        slot[ent0 + j] = s;
    }
    if (send_slot != nullptr) {
        for (int q = tid; q < ntok * R; q += kFinalThreads) {
            const int r = q % R;
            const int64_t i = (int64_t)tok_tile0 * R + q;
            const int v = send_slot[i];
            send_slot[i] = (r != rank && v >= 0) ? rank_before[r] + v : -1;
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
        const size_t lds = sizeof(unsigned long long) * kTile + sizeof(int32_t) * (4 * (size_t)h.E + 4 * (size_t)h.R + 4 +
                                                                                  (size_t)kTile * h.K);
        hipLaunchKernelGGL(k_layout_count, dim3(h.ntiles), dim3(kTile), lds, stream, h.topk_idx, h.T, h.K, h.E, h.R,
                           epr, nbits, h.ws.tile_hist, h.ws.tile_rank, h.ws.tile_inv, h.ws.slot, send,
                           out.is_token_in_rank);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(k_layout_finalize, dim3(h.ntiles > 0 ? h.ntiles : 1), dim3(kFinalThreads), 0, stream, h.T, h.K,
                       h.E, h.R, h.rank, epr, h.A, h.ntiles, h.ws.tile_hist, h.ws.tile_rank, h.ws.tile_inv, h.ws.slot,
                       send, h.ws.cnt_local, h.ws.psum, out.num_tokens_per_rank, out.num_tokens_per_expert, out.psum,
                       out.num_invalid);
    return hipGetLastError();
}

}  // namespace ep
