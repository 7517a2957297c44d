// ep_fused.hip -- one launch for the layout and the dispatch of a small batch (<= 256 tokens, the decode shape)
// on gfx950 ([DeepEP->MegaMoE] §4.3: at small batches the launches, not the bytes, set the time; [DeepEP-hotdry]
// 性能基准 and [MoE-comm] §一: the low-latency decode path dispatches with the layout of the same call).
//
// Every block computes the whole layout of the routing table in LDS -- the counting sort of k_layout_single:
// stage the entries, rank them per wave with key-bit ballots, per-wave bases, the aligned scans of counts and
// padding -- and then runs its share of the dispatch work items with the rows taken from LDS.  No block waits
// for another, so one launch replaces the layout launch and the dispatch launch; the price is that each block
// repeats the (small, latency-bound) layout work.
//
// The handle's workspace and the layout outputs are written along the way, so the handle is complete
// afterwards (ep_dispatch and ep_combine can reuse it as if ep_get_layout had built it): block 0 writes the
// counts and the psum; the wave of a token's segment 0 writes its slots, its per-rank token rows and its
// membership; the padding waves write the padding-row list.
//   token item (t, s)       as in the dispatch kernels (FP8 cast, or 16-byte copies), destinations from LDS;
//                           its source loads are issued before the layout work, so they overlap it;
//   padding-list lanes      lane q of the pass over padding row numbers finds its row by a binary search of
//                           the padding prefix in LDS, writes the list entry and (without zero padding) the
//                           row's metadata;
//   zero-padding items      (row number, segment) pairs, zeros written as in the dispatch kernels.
#include <algorithm>

#include "ep_dispatch_core.hpp"
#include "ep_layout_core.hpp"

namespace ep {
namespace {

constexpr int kMaxPadWaves = 4096;   // padding passes loop beyond this many waves instead of growing the grid
constexpr int kMinBlocks = 256;      // at least one workgroup per CU of an MI355X: the stores of the dispatch need
                                     // the store paths of the whole chip, and the layout repeated per workgroup is
                                     // latency, not throughput
constexpr uint16_t kNoRow = 0xFFFF;  // per-rank token row "none" in LDS (rows are < 256)

__device__ __forceinline__ int row_or_none(uint16_t v) { return v == kNoRow ? -1 : (int)v; }

__host__ __device__ size_t fused_lds_bytes(int E, int K, int R, int epr) {
    return count_lds_bytes(E, K, R) + sizeof(int) * (2 * (size_t)(epr + 1) + 2 * kWaves) +
           sizeof(uint16_t) * (size_t)kTile * R;
}

struct FusedArgs {
    const int64_t* idx;
    int E, A, nbits;
    Outputs o;               // counts, psum, padding list and total
    int32_t* slot_ws;        // [T, K] workspace slot map
    int32_t* rows_ws;        // [T, R] workspace per-rank token rows
    uint8_t* in_rank;        // [T, R] caller output, nullable
};

template <bool FP8>
__global__ __launch_bounds__(kThreads) void k_layout_dispatch_small(FusedArgs f, Params p) {
    const int T = p.T, K = p.K, R = p.R, E = f.E, epr = p.epr, lo = p.rank * epr;
    const CountLds L = carve_count(layout_smem, E, K, R);
    int* psum = reinterpret_cast<int*>(layout_smem + count_lds_bytes(E, K, R));   // [epr + 1]
    int* padpre = psum + epr + 1;                                                 // [epr + 1]
    int* scratch = padpre + epr + 1;                                              // [2 * kWaves]
    uint16_t* trow = reinterpret_cast<uint16_t*>(scratch + 2 * kWaves);           // [256 * R], kNoRow = none

    // the token item's source bytes do not depend on the layout: their loads are issued together with the
    // layout's entry loads and stay in flight through the layout work
    const int lane = lane_id();
    // work items are strided over the workgroups (item = wave * workgroups + workgroup), so that a grid larger
    // than the items spreads them over every CU instead of filling the first workgroups
    const int64_t gw = (int64_t)(threadIdx.x >> 6) * gridDim.x + blockIdx.x;
    const bool tok = gw < p.ntok_items;
    const int t = tok ? (int)(gw / p.nstep) : 0, st = tok ? (int)(gw % p.nstep) : 0;
    Fp8Src v8;
    u32x4 vr;
    TokenEntry te;
    auto prefetch = [&] {
        if (tok) {
            if (FP8) v8 = fp8_load(p, t, st, lane);
            else vr = raw_load(p, t, st, lane);
            if (st == 0) te = token_entry(p, t, lane);
        }
    };

    // the layout, in LDS
    const uint64_t mask = count_tile(f.idx, T, K, E, R, epr, f.nbits, 0, L, nullptr, prefetch);
    local_scan(epr, lo, f.A, L.row, psum, padpre, scratch);
    token_rows(L, mask, T, R, 0, [&](int t, int r, int v) { trow[t * R + r] = v < 0 ? kNoRow : (uint16_t)v; });
    __syncthreads();
    if (blockIdx.x == 0) write_counts(E, R, lo, epr, L.row, psum, padpre, f.o);

    // token item
    if (tok) {
        int sexp = -1;                                 // expert-major row of entry (t, lane)
        if (lane < K) {
            const int pk = L.ent[t * K + lane];
            if (pk >= 0) {
                const int e = pk & kPackMask;
                if (e >= lo && e < lo + epr)
                    sexp = psum[e - lo] + L.cnt_w[(t / tokens_per_wave(T, 0)) * E + e] + (pk >> kPackShift);
            }
        }
        const int own = lane < R ? row_or_none(trow[t * R + lane]) : -1;
        const int ds = p.token_major ? (lane == 0 ? row_or_none(trow[t * R + p.rank]) : -1) : sexp;
        const int js = (p.send_slot != nullptr && lane != p.rank) ? own : -1;
        const uint64_t lmask = ballot(ds >= 0), smask = ballot(js >= 0);
        if (st == 0) {
            if (lane < K) f.slot_ws[(int64_t)t * K + lane] = sexp;
            if (lane < R) {
                f.rows_ws[(int64_t)t * R + lane] = own;
                if (f.in_rank) f.in_rank[(int64_t)t * R + lane] = own >= 0 ? 1 : 0;
            }
            token_meta(p, t, lane, ds, js, lmask, smask, &te);
        }
        if ((lmask | smask) != 0) {
            if (FP8) fp8_emit(p, st, lane, v8, ds, js, lmask, smask);
            else raw_emit(p, t, st, lane, vr, ds, js, lmask, smask);
        }
    }

    // padding: the row list (and, without zero padding, the rows' metadata), one row number per lane
    const int npad = padpre[epr];
    const bool meta_only = !p.token_major && !p.zero_pad && (p.recv_src != nullptr || p.recv_w != nullptr);
    for (int64_t q = gw * kWave + lane; q < npad; q += p.nwaves * kWave) {
        const int row = pad_row_of((int)q, epr, psum, padpre);
        if (f.o.pad_rows) f.o.pad_rows[q] = row;
        if (meta_only) pad_meta_row(p, row);
    }
    // zero padding: (row number, segment) items
    if (p.zero_pad && !p.token_major) {
        const int64_t nitems = (int64_t)npad * p.nstep;
        for (int64_t i = gw; i < nitems; i += p.nwaves) {
            const int q = (int)(i / p.nstep);
            pad_zero_segment<FP8>(p, pad_row_of(q, epr, psum, padpre), (int)(i % p.nstep), lane);
        }
    }
}

}  // namespace

hipError_t launch_layout_dispatch(const Handle& h, const LayoutOutputs& out, const DispatchArgs& a,
                                  hipStream_t stream) {
    if (h.ntiles != 1 || a.mode == DispatchArgs::kRows) {   // T == 0, or more than one tile: two launches
        // the layout launches read the dispatch's source rows ahead of it (into the memory-side cache)
        const size_t src_bytes = (size_t)h.T * (a.mode == DispatchArgs::kRows ? (size_t)a.row_bytes : 2 * (size_t)a.hidden);
        const hipError_t e = launch_layout(h, out, stream, a.x, src_bytes);
        if (e != hipSuccess) return e;
        return launch_dispatch(h, a, stream);
    }
    const bool fp8 = a.mode == DispatchArgs::kFp8;
    Params p = dispatch_params(h, a);
    const int64_t max_pad = (int64_t)h.El * (h.A - 1);
    int64_t nwaves = p.ntok_items;
    int64_t pad_waves = (max_pad + kWave - 1) / kWave;
    if (p.zero_pad && !p.token_major) pad_waves = std::max(pad_waves, (max_pad * p.nstep + kPadItemsPerWave - 1) / kPadItemsPerWave);
    nwaves = std::max(nwaves, std::min(pad_waves, (int64_t)kMaxPadWaves));
    const int64_t nblocks = std::max<int64_t>((nwaves + kWaves - 1) / kWaves, kMinBlocks);
    p.nwaves = nblocks * kWaves;

    FusedArgs f;
    f.idx = h.topk_idx;
    f.E = h.E;
    f.A = h.A;
    f.nbits = 0;
    while ((1 << f.nbits) < h.E) ++f.nbits;
    f.o = Outputs{h.ws.cnt_local, h.ws.psum, h.ws.pad_rows, h.ws.pad_total, out.num_tokens_per_rank,
                  out.num_tokens_per_expert, out.psum, out.num_invalid};
    f.slot_ws = h.ws.slot;
    f.rows_ws = h.ws.send_slot;
    f.in_rank = out.is_token_in_rank;

    const size_t lds = fused_lds_bytes(h.E, h.K, h.R, h.El);
    if (lds > 65536) {
        const void* k = fp8 ? reinterpret_cast<const void*>(k_layout_dispatch_small<true>)
                            : reinterpret_cast<const void*>(k_layout_dispatch_small<false>);
        const hipError_t e = allow_dynamic_lds(k, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (fp8)
        hipLaunchKernelGGL(k_layout_dispatch_small<true>, dim3((unsigned)nblocks), dim3(kThreads), lds, stream, f, p);
    else
        hipLaunchKernelGGL(k_layout_dispatch_small<false>, dim3((unsigned)nblocks), dim3(kThreads), lds, stream, f, p);
    return hipGetLastError();
}

}  // namespace ep
