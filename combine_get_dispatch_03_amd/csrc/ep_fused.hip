// ep_fused.hip -- one launch for the layout and the dispatch of a small batch (<= 256 tokens, the decode shape)
// on gfx950 ([DeepEP->MegaMoE] §4.3: at small batches the launches, not the bytes, set the time; [DeepEP-hotdry]
// 性能基准 and [MoE-comm] §一: the low-latency decode path dispatches with the layout of the same call).
//
// Workgroup t < T owns token t.  A token's rows need only counts, not a sort: its expert-major row for entry k is
// the aligned start of the expert, plus the expert's entries in the tokens before t, plus the copies of the
// expert among entries 0..k-1 of t; its row in rank r's window is the number of tokens before t that have an
// expert on r.  So every workgroup stages the routing table in LDS and builds, with LDS atomic adds, the column
// totals (experts | ranks | invalid) and the counts before its own token, runs the aligned scan of the local
// experts, and writes its token; no workgroup waits for another, and the per-workgroup layout work is two
// atomic adds per entry instead of a ranking of the whole table.
//
// The handle's workspace and the layout outputs are written along the way, so the handle is complete
// afterwards (ep_dispatch and ep_combine can reuse it as if ep_get_layout had built it): block 0 writes the
// counts and the psum; the first token wave of token t's workgroup writes its slots, its per-rank token rows and
// its membership; the padding waves write the padding-row list.
//   token segments          segment s of token t on wave 16 - nt + s % 16 of workgroup t (nt = min(segments, 16):
//                           the last waves, clear of the scan on wave 0), as in the dispatch kernels (FP8 cast,
//                           or 16-byte copies); the first segment's loads are issued before the layout work, so
//                           they overlap it, and its FP8 cast runs while wave 0 scans;
//   padding-list lanes      lane q of the pass over padding row numbers finds its row by a binary search of
//                           the padding prefix in LDS, writes the list entry and (without zero padding) the
//                           row's metadata;
//   zero-padding items      (row number, segment) pairs, zeros written as in the dispatch kernels.
// The padding runs on the waves that have no token segment (at hidden 7168, waves 0..8 of every token's
// workgroup), beside the token segments instead of after them.
#include <algorithm>

#include "ep_dispatch_core.hpp"
#include "ep_layout_core.hpp"

namespace ep {
namespace {

constexpr int kMaxPadWaves = 4096;   // padding passes loop beyond this many waves instead of growing the grid

struct FusedArgs {
    const int64_t* idx;
    int E, A;
    Outputs o;               // counts, psum, padding list and total
    int32_t* slot_ws;        // [T, K] workspace slot map
    int32_t* rows_ws;        // [T, R] workspace per-rank token rows
    uint8_t* in_rank;        // [T, R] caller output, nullable
};

template <bool FP8>
__global__ __launch_bounds__(kThreads) void k_layout_dispatch_small(FusedArgs f, Params p) {
    touch_kernargs<sizeof(FusedArgs) + sizeof(Params)>();
    const int T = p.T, K = p.K, R = p.R, E = f.E, epr = p.epr, lo = p.rank * epr;
    const TokLds L = carve_tok(layout_smem, E, K, R, epr);
    const int lane = lane_id(), w = threadIdx.x >> 6;
    const int t = blockIdx.x;                         // this workgroup's token (the grid has >= T workgroups)
    const bool tok = t < T;
    // the token's segments go to the last nt waves (segment s on wave 16 - nt + s % 16), clear of wave 0, which
    // runs the scan (and, up to 6 segments, of waves 4..7, which count the tokens per rank meanwhile)
    const int nt = min(p.nstep, kWaves);
    const int tw = w - (kWaves - nt);                 // >= 0 on the token's waves
    const bool seg = tok && tw >= 0;

    // the token's first segments and its metadata do not depend on the layout: their loads are issued with the
    // routing table's and stay in flight through the layout work
    Fp8Src v8;
    Fp8Row c8;
    u32x4 vr;
    TokenEntry te;
    TokRow tr;
    tok_counts(f.idx, T, K, E, R, epr, f.A, lo, t, L, [&] {
        // every wave issues them, with clamped operands (T >= 1 here): loads behind a branch would make the
        // staging of the table wait for them too
        const int tc = tok ? t : 0, sc = min(max(tw, 0), p.nstep - 1);
        if (FP8) v8 = fp8_load_clamped(p, tc, sc, lane);
        else vr = raw_load_clamped(p, tc, sc, lane);
        te = token_entry(p, tc, lane);
    }, [&] {
        // while wave 0 scans: the FP8 cast of the segment and the token's rows up to the experts' starts
        if (seg) {
            if (FP8) c8 = fp8_cast(v8);
            tr = tok_row_counts(L, t, K);
        }
    });
    if (blockIdx.x == 0) write_counts(E, R, lo, epr, L.tot, L.psum, L.padpre, f.o);

    // token t: its rows (lane k < K: expert-major row of entry k; lane r < R: row in rank r's window), then its
    // segments
    if (seg) {
        const int sexp = tok_row_slot(L, tr, K, lo, epr), own = tok_row_own(L, tr, R);
        const int own_here = readlane(own, p.rank);        // the token's row among this rank's tokens
        const int ds = p.token_major ? (lane == 0 ? own_here : -1) : sexp;
        const int js = (p.send_slot != nullptr && lane < R && lane != p.rank) ? own : -1;
        const uint64_t lmask = ballot(ds >= 0), smask = ballot(js >= 0);
        if (tw == 0) {
            if (lane < K) f.slot_ws[(int64_t)t * K + lane] = sexp;
            if (lane < R) {
                f.rows_ws[(int64_t)t * R + lane] = own;
                if (f.in_rank) f.in_rank[(int64_t)t * R + lane] = own >= 0 ? 1 : 0;
            }
            token_meta(p, t, lane, ds, js, lmask, smask, &te);
        }
        if ((lmask | smask) != 0) {
            for (int s = tw; s < p.nstep; s += kWaves) {
                if (FP8) fp8_store(p, s, lane, s == tw ? c8 : fp8_cast(fp8_load(p, t, s, lane)), ds, js, lmask, smask);
                else raw_emit(p, t, s, lane, s == tw ? vr : raw_load(p, t, s, lane), ds, js, lmask, smask);
            }
        }
        return;
    }

    // padding, on the waves without a token segment (waves 0 .. 15 - nt of the token workgroups, every wave of
    // the workgroups past T), so that it runs beside the token segments: the row list (and, without zero
    // padding, the rows' metadata), one row number per lane; then, with zero padding, (row number, segment) items
    const int64_t iw = tok ? (int64_t)blockIdx.x * (kWaves - nt) + w
                           : (int64_t)T * (kWaves - nt) + ((int64_t)blockIdx.x - T) * kWaves + w;
    const int npad = L.padpre[epr];
    const bool meta_only = !p.token_major && !p.zero_pad && (p.recv_src != nullptr || p.recv_w != nullptr);
    for (int64_t q = iw * kWave + lane; q < npad; q += p.nwaves * kWave) {
        const int row = pad_row_of((int)q, epr, L.psum, L.padpre);
        if (f.o.pad_rows) f.o.pad_rows[q] = row;
        if (meta_only) pad_meta_row(p, row);
    }
    if (p.zero_pad && !p.token_major) {
        const int64_t nitems = (int64_t)npad * p.nstep;
        for (int64_t i = iw; i < nitems; i += p.nwaves) {
            const int q = (int)(i / p.nstep);
            pad_zero_segment<FP8>(p, pad_row_of(q, epr, L.psum, L.padpre), (int)(i % p.nstep), lane);
        }
    }
}

}  // namespace

hipError_t launch_layout_dispatch(const Handle& h, const LayoutOutputs& out, const DispatchArgs& a,
                                  hipStream_t stream) {
    if (h.ntiles != 1 || a.mode == DispatchArgs::kRows) {   // T == 0, or more than one tile: two launches
        const hipError_t e = launch_layout(h, out, stream);
        if (e != hipSuccess) return e;
        return launch_dispatch(h, a, stream);
    }
    const bool fp8 = a.mode == DispatchArgs::kFp8;
    Params p = dispatch_params(h, a);
    const int64_t max_pad = (int64_t)h.El * (h.A - 1);
    int64_t pad_waves = (max_pad + kWave - 1) / kWave;
    if (p.zero_pad && !p.token_major) pad_waves = std::max(pad_waves, (max_pad * p.nstep + kPadItemsPerWave - 1) / kPadItemsPerWave);
    const int64_t want = std::min(pad_waves, (int64_t)kMaxPadWaves);   // 0 without any padding
    // one workgroup per token (workgroup t owns token t), more only if its idle waves (those without a token
    // segment) are too few for the padding passes: workgroups without a token were measured to cost time
    // (decode 8.12 -> 8.06 us, one token 6.04 -> 5.92 us without the 256 that one per CU would give)
    const int64_t idle_per_tok = kWaves - std::min(p.nstep, kWaves);
    const int64_t have = (int64_t)h.T * idle_per_tok;
    const int64_t nblocks = h.T + (have >= want ? 0 : (want - have + kWaves - 1) / kWaves);
    // the padding waves, the stride of the padding passes (>= 1 whenever a wave runs a padding pass)
    p.nwaves = have + (nblocks - h.T) * kWaves;

    FusedArgs f;
    f.idx = h.topk_idx;
    f.E = h.E;
    f.A = h.A;
    f.o = Outputs{h.ws.cnt_local, h.ws.psum, h.ws.pad_rows, h.ws.pad_total, out.num_tokens_per_rank,
                  out.num_tokens_per_expert, out.psum, out.num_invalid};
    f.slot_ws = h.ws.slot;
    f.rows_ws = h.ws.send_slot;
    f.in_rank = out.is_token_in_rank;

    const size_t lds = tok_lds_bytes(h.E, h.K, h.R, h.El);
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
