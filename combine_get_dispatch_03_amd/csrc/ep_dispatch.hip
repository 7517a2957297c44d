// ep_dispatch.hip -- expert-major dispatch on gfx950 ([DeepEP->MegaMoE] §2.2: each token row is loaded once
// and stored to the send buffer; §2.4: rows are placed expert-major at their expert's cursor; [MoE-comm] §一:
// expert_alignment and do_zero_padding; [DeepEP-hotdry] key techniques: FP8 dispatch).
//
// Work items are row segments, so that many short waves keep the write path busy:
//   token item (t, s)  FP8: channels [1024 s, 1024 s + 1024) of token t, cast once and stored to every
//                      destination row of the token (its local slots and its send-window rows).
//                      BF16, and rows already in their receive format (the receiver's copy epilogue,
//                      [DeepEP->MegaMoE] §2.4): up to kRawSegs consecutive 1 KiB segments of 16-byte
//                      copies, all source loads issued first, plus the row's scales with segment 0.
//   padding item (p, s) segment s of padding row pad_rows[p] (zeros; its metadata on segment 0).
// Token-major mode (do_expand off, [MoE-comm] §一 dispatch arguments): the token's only local destination is
// its row among this rank's tokens, with the token's K local expert ids and weights as metadata; no padding.
// Wave w runs token item w (if any) and then padding items w, w + W, w + 2W, ... (at most kPadItemsPerWave of
// them).  The grid is sized on the host from the number of tokens and the worst-case padding; the actual
// padding count is read on the device.
// Nothing here decides a position: every row index comes from the layout.
#include "ep_dispatch_core.hpp"

namespace ep {
namespace {

constexpr int kBlock = 256;                 // 4 waves
constexpr int kWavesPerBlock = kBlock / kWave;
// 1024-channel segments per FP8 token item: 1 measured fastest on the prefill shape (2 and 4, which give longer
// contiguous writes per destination row, were 1-5% slower once the padding items share the waves).
constexpr int kFp8SegsPerItem = 1;
// 1 KiB segments per copy item: a copy wave does little besides its two round trips (destinations, then the
// source), so 4 segments per wave measured 11% faster than 1 for the receiver placement (2 was within 1% of 4).
constexpr int kRawSegs = 4;

// Per-token destinations from the layout in the workspace: the local rows (expert-major: lanes < K hold the
// token's slots; token-major: lane 0 holds its row among this rank's tokens) and the send rows (lanes r < R,
// r != rank).
__device__ __forceinline__ void token_dests(const Params& p, int t, int lane, int& ds, int& js, uint64_t& lmask,
                                            uint64_t& smask) {
    if (p.own_row == nullptr) ds = lane < p.K ? p.slot[(int64_t)t * p.K + lane] : -1;
    else ds = lane == 0 ? p.own_row[(int64_t)t * p.R + p.rank] : -1;
    js = (p.send_slot != nullptr && lane < p.R && lane != p.rank) ? p.send_slot[(int64_t)t * p.R + lane] : -1;
    lmask = ballot(ds >= 0);
    smask = ballot(js >= 0);
}

// Padding items of wave gw are gw + j * nwaves for j < kPadItemsPerWave (the grid is sized so that no wave
// has more).  Their row indices are fetched before the token work so the loads overlap it.  Without zero
// padding only the rows' metadata is written, one padding row per lane: wave gw takes rows 64 gw .. 64 gw + 63.
struct PadWork {
    int64_t nitems;
    int row[kPadItemsPerWave];
};

__device__ __forceinline__ void pad_prefetch(const Params& p, int64_t gw, int lane, PadWork& pw) {
    pw.nitems = p.pad_sub == 0 ? 0 : (int64_t)(*p.pad_total) * p.pad_sub;
    if (!p.zero_pad) {
        const int64_t i = gw * kWave + lane;
        pw.row[0] = i < pw.nitems ? p.pad_rows[i] : 0;
        return;
    }
#pragma unroll
    for (int j = 0; j < kPadItemsPerWave; ++j) {
        const int64_t i = gw + j * p.nwaves;
        pw.row[j] = i < pw.nitems ? p.pad_rows[i / p.pad_sub] : 0;
    }
}

template <bool FP8>
__device__ __forceinline__ void pad_items(const Params& p, int64_t gw, int lane, const PadWork& pw) {
    if (!p.zero_pad) {
        if (gw * kWave + lane < pw.nitems) pad_meta_row(p, pw.row[0]);
        return;
    }
#pragma unroll
    for (int j = 0; j < kPadItemsPerWave; ++j) {
        const int64_t i = gw + j * p.nwaves;
        if (i >= pw.nitems) break;
        pad_zero_segment<FP8>(p, pw.row[j], (int)(i % p.pad_sub), lane);
    }
}

// FP8 token items cover SPW consecutive 1024-channel segments of a row (all loads first, then the casts and
// stores segment by segment): longer contiguous writes per destination row than one segment per wave.
// EARLY (send windows present): the source loads are issued before the destination loads, so that the two
// round trips overlap (5% faster at 8 ranks); without windows issuing them after measured faster.  It is a
// template parameter, not a runtime flag: with both paths in one kernel the compiler cannot tell that the
// early loads' registers are never pending on the late path, and puts a full wait (for every load and store
// in flight, the segment-0 metadata stores included) in front of the late loads.
template <int SPW, bool EARLY>
__global__ __launch_bounds__(kBlock) void k_dispatch_fp8(Params p) {
    const int lane = lane_id();
    const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    PadWork pw;
    pad_prefetch(p, gw, lane, pw);
    if (gw < p.ntok_items) {
        const int nit = (p.nstep + SPW - 1) / SPW;
        const int t = (int)(gw / nit), it = (int)(gw % nit);
        Fp8Src v[SPW];
        if (EARLY) {
#pragma unroll
            for (int j = 0; j < SPW; ++j)
                if (it * SPW + j < p.nstep) v[j] = fp8_load(p, t, it * SPW + j, lane);
        }
        int ds, js;
        uint64_t lmask, smask;
        token_dests(p, t, lane, ds, js, lmask, smask);
        const bool any = (lmask | smask) != 0;
        if (!EARLY && any) {
#pragma unroll
            for (int j = 0; j < SPW; ++j)
                if (it * SPW + j < p.nstep) v[j] = fp8_load(p, t, it * SPW + j, lane);
        }
        // the metadata (segment 0) follows the source loads, which then never wait behind its stores
        if (it == 0) token_meta(p, t, lane, ds, js, lmask, smask);
        if (any) {
#pragma unroll
            for (int j = 0; j < SPW; ++j)
                if (it * SPW + j < p.nstep) fp8_emit(p, it * SPW + j, lane, v[j], ds, js, lmask, smask);
        }
    }
    pad_items<true>(p, gw, lane, pw);
}

__global__ __launch_bounds__(kBlock) void k_dispatch_raw(Params p) {
    const int lane = lane_id();
    const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    PadWork pw;
    pad_prefetch(p, gw, lane, pw);
    if (gw < p.ntok_items) {
        const int nit = (p.nstep + kRawSegs - 1) / kRawSegs;
        const int t = (int)(gw / nit), it = (int)(gw % nit);
        int ds, js;
        uint64_t lmask, smask;
        token_dests(p, t, lane, ds, js, lmask, smask);
        if ((lmask | smask) != 0) {
            // unpredicated loads (a lane past the row's end re-reads chunk 0 and stores nothing), so the compiler
            // keeps all kRawSegs in flight
            u32x4 v[kRawSegs];
            const int nchunk = p.row_bytes / 16;
#pragma unroll
            for (int j = 0; j < kRawSegs; ++j) {
                const int c = (it * kRawSegs + j) * kWave + lane;
                v[j] = reinterpret_cast<const u32x4*>(p.src + (int64_t)t * p.row_bytes)[c < nchunk ? c : 0];
            }
            if (it == 0) token_meta(p, t, lane, ds, js, lmask, smask);
#pragma unroll
            for (int j = 0; j < kRawSegs; ++j)
                if (it * kRawSegs + j < p.nstep) raw_emit(p, t, it * kRawSegs + j, lane, v[j], ds, js, lmask, smask);
        } else if (it == 0) {
            token_meta(p, t, lane, ds, js, lmask, smask);
        }
    }
    pad_items<false>(p, gw, lane, pw);
}

}  // namespace

hipError_t launch_dispatch(const Handle& h, const DispatchArgs& a, hipStream_t stream) {
    if (h.T == 0) return hipSuccess;
    Params p = dispatch_params(h, a);
    const bool fp8 = a.mode == DispatchArgs::kFp8;
    if (fp8) p.ntok_items = (int64_t)h.T * ((p.nstep + kFp8SegsPerItem - 1) / kFp8SegsPerItem);
    else p.ntok_items = (int64_t)h.T * ((p.nstep + kRawSegs - 1) / kRawSegs);
    const int64_t max_pad_items = (int64_t)h.El * (h.A - 1) * p.pad_sub;
    int64_t nwaves = p.ntok_items;
    const int64_t per_wave = a.zero_pad ? kPadItemsPerWave : kWave;
    const int64_t pad_waves = (max_pad_items + per_wave - 1) / per_wave;
    if (pad_waves > nwaves) nwaves = pad_waves;
    const int64_t nblocks = (nwaves + kWavesPerBlock - 1) / kWavesPerBlock;
    p.nwaves = nblocks * kWavesPerBlock;
    if (fp8 && p.send_slot != nullptr)
        hipLaunchKernelGGL((k_dispatch_fp8<kFp8SegsPerItem, true>), dim3((unsigned)nblocks), dim3(kBlock), 0, stream, p);
    else if (fp8)
        hipLaunchKernelGGL((k_dispatch_fp8<kFp8SegsPerItem, false>), dim3((unsigned)nblocks), dim3(kBlock), 0, stream,
                           p);
    else
        hipLaunchKernelGGL(k_dispatch_raw, dim3((unsigned)nblocks), dim3(kBlock), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ep
