// ep_dispatch.hip -- expert-major dispatch on gfx950 ([DeepEP->MegaMoE] §2.2: each token row is loaded once
// and stored to the send buffer; §2.4: rows are placed expert-major at their expert's cursor; [MoE-comm] §一:
// expert_alignment and do_zero_padding; [DeepEP-hotdry] key techniques: FP8 dispatch).
//
// Work items are row segments, so that many short waves keep the write path busy:
//   token item (t, s)  FP8: channels [1024 s, 1024 s + 1024) of token t.  Each lane loads 32 contiguous bytes
//                      (16 bf16 channels), eight lanes form one 128-channel group whose max |x| comes from
//                      three xor-shuffles, the lane casts its 16 channels to 16 e4m3 bytes and stores them as
//                      one 16-byte vector to every destination row of the token (its local slots and its
//                      send-window rows), together with the segment's 8 group scales.
//                      BF16, and rows already in their receive format (the receiver's copy epilogue,
//                      [DeepEP->MegaMoE] §2.4): one 1 KiB segment of 16-byte copies, plus the row's scales.
//   padding item (p, s) segment s of padding row pad_rows[p] (zeros; its metadata on segment 0).
// Token-major mode (do_expand off, [MoE-comm] §一 dispatch arguments): the token's only local destination is
// its row among this rank's tokens, with the token's K local expert ids and weights as metadata; no padding.
// Wave w runs token item w (if any) and then padding items w, w + W, w + 2W, ... (at most kPadItemsPerWave of
// them).  The grid is sized on the host from the number of tokens and the worst-case padding; the actual
// padding count is read on the device.
// Nothing here decides a position: every row index comes from the layout.
#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {
namespace {

constexpr int kBlock = 256;                 // 4 waves
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kPadItemsPerWave = 2;         // worst-case padding items per wave used to size the grid

struct Params {
    const uint8_t* src;          // token rows: bf16 [T, H] (FP8 kernel) or row_bytes-byte rows (raw kernel)
    const float* src_scales;     // raw kernel: [T, G] scales travelling with the rows, or nullptr
    const float* w;
    const int64_t* topk_idx;
    const int32_t* slot;
    const int32_t* send_slot;    // [T, R] send-window rows (windows only), else nullptr
    const int32_t* own_row;      // token-major mode: [T, R] per-rank token rows (column rank), else nullptr
    const int32_t* pad_rows;
    const int32_t* pad_total;
    uint8_t* recv_x;
    float* recv_scales;
    int32_t* recv_src;
    float* recv_w;               // [rows] (expert-major) or [T, K] (token-major)
    int64_t* recv_topk_idx;      // token-major: [T, K] local expert ids or -1
    uint8_t* send_x;
    float* send_scales;
    int32_t* send_src;
    int64_t* send_topk_idx;
    float* send_topk_w;
    int T, H, K, R, rank, epr;
    int row_bytes;    // bytes of one destination row
    int G;            // fp32 scales per row (FP8: H / 128; raw: as given, 0 for none)
    int nstep;        // segments per row
    int64_t ntok_items;   // T * nstep
    int pad_sub;      // padding items per padding row (nstep with zero padding, 1 for metadata only, 0 none)
    int zero_pad;
    int64_t nwaves;   // waves in the grid
};

// Per-token destinations: the local rows (expert-major: lanes < K hold the token's slots; token-major: lane 0
// holds its row among this rank's tokens) and the send rows (lanes r < R, r != rank); segment 0 also writes
// the per-row metadata.
__device__ __forceinline__ void token_dests(const Params& p, int t, bool meta, int lane, int& ds, int& js,
                                            uint64_t& lmask, uint64_t& smask) {
    if (p.own_row == nullptr) ds = lane < p.K ? p.slot[(int64_t)t * p.K + lane] : -1;
    else ds = lane == 0 ? p.own_row[(int64_t)t * p.R + p.rank] : -1;
    js = (p.send_slot != nullptr && lane < p.R && lane != p.rank) ? p.send_slot[(int64_t)t * p.R + lane] : -1;
    lmask = ballot(ds >= 0);
    smask = ballot(js >= 0);
    if (!meta) return;
    const float wk = (lane < p.K && p.w != nullptr) ? p.w[(int64_t)t * p.K + lane] : 1.0f;
    const bool need_e = (smask != 0 && p.send_topk_idx != nullptr) ||
                        (p.own_row != nullptr && lmask != 0 && p.recv_topk_idx != nullptr);
    const int64_t e = (need_e && lane < p.K) ? p.topk_idx[(int64_t)t * p.K + lane] : -1;
    if (p.own_row == nullptr) {
        if (ds >= 0) {
            if (p.recv_src) p.recv_src[ds] = t;
            if (p.recv_w) p.recv_w[ds] = wk;
        }
    } else if (lmask != 0) {
        const int64_t j = readlane(ds, 0);
        if (lane == 0 && p.recv_src) p.recv_src[j] = t;
        if (lane < p.K) {
            const int64_t lo = (int64_t)p.rank * p.epr;
            if (p.recv_topk_idx) p.recv_topk_idx[j * p.K + lane] = (e >= lo && e < lo + p.epr) ? e - lo : -1;
            if (p.recv_w) p.recv_w[j * p.K + lane] = wk;
        }
    }
    if (smask != 0 && (p.send_src || p.send_topk_idx || p.send_topk_w)) {
        for (uint64_t m = smask; m != 0; m &= m - 1) {
            const int r = __builtin_ctzll(m);
            const int64_t row = (int64_t)r * p.T + readlane(js, r);
            if (lane == 0 && p.send_src) p.send_src[row] = t;
            if (lane < p.K) {
                const bool owned = e >= (int64_t)r * p.epr && e < (int64_t)(r + 1) * p.epr;
                if (p.send_topk_idx) p.send_topk_idx[row * p.K + lane] = owned ? e - (int64_t)r * p.epr : -1;
                if (p.send_topk_w) p.send_topk_w[row * p.K + lane] = wk;
            }
        }
    }
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
        if (gw * kWave + lane < pw.nitems) {
            if (p.recv_src) p.recv_src[pw.row[0]] = -1;
            if (p.recv_w) p.recv_w[pw.row[0]] = 0.0f;
        }
        return;
    }
    const int G = p.G;
    const int nchunk = p.row_bytes / 16;            // 16-byte chunks per row
    const int64_t row_bytes = p.row_bytes;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < kPadItemsPerWave; ++j) {
        const int64_t i = gw + j * p.nwaves;
        if (i >= pw.nitems) break;
        const int s = (int)(i % p.pad_sub);
        const int row = pw.row[j];
        if (p.zero_pad) {
            const int c = s * kWave + lane;
            if (c < nchunk) st_nt(reinterpret_cast<u32x4*>(p.recv_x + row * row_bytes) + c, z);
            if (FP8) {
                if (lane < 8 && s * 8 + lane < G) p.recv_scales[(int64_t)row * G + s * 8 + lane] = 0.0f;
            } else if (s == 0) {
                for (int g = lane; g < G; g += kWave) p.recv_scales[(int64_t)row * G + g] = 0.0f;
            }
        }
        if (s == 0 && lane == 0) {
            if (p.recv_src) p.recv_src[row] = -1;
            if (p.recv_w) p.recv_w[row] = 0.0f;
        }
    }
}

__global__ __launch_bounds__(kBlock) void k_dispatch_fp8(Params p) {
    const int lane = lane_id();
    const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    PadWork pw;
    pad_prefetch(p, gw, lane, pw);
    if (gw < p.ntok_items) {
        const int t = (int)(gw / p.nstep), st = (int)(gw % p.nstep);
        int ds, js;
        uint64_t lmask, smask;
        token_dests(p, t, st == 0, lane, ds, js, lmask, smask);
        if ((lmask | smask) != 0) {
            const int H = p.H, G = H / 128;
            const int ch = (st * kWave + lane) * 16;      // first channel of this lane
            const bool active = ch < H;
            u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
            if (active) {
                const u32x4* src = reinterpret_cast<const u32x4*>(p.src + ((int64_t)t * H + ch) * 2);
                a = ld_nt(src);
                b = ld_nt(src + 1);
            }
            float f[16];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                f[2 * k] = bf16lo(a[k]);
                f[2 * k + 1] = bf16hi(a[k]);
                f[8 + 2 * k] = bf16lo(b[k]);
                f[8 + 2 * k + 1] = bf16hi(b[k]);
            }
            float m = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k) m = fmaxf(m, fabsf(f[k]));
            m = group8_max(m);
            const float amax = fmaxf(m, 1e-4f);
            const float scale = amax / 448.0f;           // IEEE division (correctly rounded)
            const float inv = 448.0f / amax;
            u32x4 q;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                q[k] = pack_e4m3x4(f[4 * k] * inv, f[4 * k + 1] * inv, f[4 * k + 2] * inv, f[4 * k + 3] * inv);
            // lane g < 8 takes the scale of group 8 st + g, held by lane 8 g
            const float sg = __shfl(scale, 8 * (lane & 7));
            const int g = st * 8 + lane;
            const bool sc_lane = lane < 8 && g < G;
            for (uint64_t mm = lmask; mm != 0; mm &= mm - 1) {
                const int s = readlane(ds, __builtin_ctzll(mm));
                if (active) st_nt(reinterpret_cast<u32x4*>(p.recv_x + (int64_t)s * H) + st * kWave + lane, q);
                if (sc_lane) p.recv_scales[(int64_t)s * G + g] = sg;
            }
            for (uint64_t mm = smask; mm != 0; mm &= mm - 1) {
                const int r = __builtin_ctzll(mm);
                const int64_t row = (int64_t)r * p.T + readlane(js, r);
                if (active) st_nt(reinterpret_cast<u32x4*>(p.send_x + row * H) + st * kWave + lane, q);
                if (sc_lane) p.send_scales[row * G + g] = sg;
            }
        }
    }
    pad_items<true>(p, gw, lane, pw);
}

// Rows that need no conversion (BF16 dispatch, and received rows that already carry their receive format):
// 16-byte copies of one 1 KiB segment per wave; segment 0 also copies the row's scales, if any.
__global__ __launch_bounds__(kBlock) void k_dispatch_raw(Params p) {
    const int lane = lane_id();
    const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    PadWork pw;
    pad_prefetch(p, gw, lane, pw);
    if (gw < p.ntok_items) {
        const int t = (int)(gw / p.nstep), st = (int)(gw % p.nstep);
        int ds, js;
        uint64_t lmask, smask;
        token_dests(p, t, st == 0, lane, ds, js, lmask, smask);
        const int c = st * kWave + lane;                  // 16-byte chunk of the row
        const bool active = c < p.row_bytes / 16;
        if ((lmask | smask) != 0) {
            const int64_t rb = p.row_bytes;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (active) v = ld_nt(reinterpret_cast<const u32x4*>(p.src + (int64_t)t * rb) + c);
            for (uint64_t mm = lmask; mm != 0; mm &= mm - 1) {
                const int s = readlane(ds, __builtin_ctzll(mm));
                if (active) st_nt(reinterpret_cast<u32x4*>(p.recv_x + (int64_t)s * rb) + c, v);
            }
            for (uint64_t mm = smask; mm != 0; mm &= mm - 1) {
                const int r = __builtin_ctzll(mm);
                const int64_t row = (int64_t)r * p.T + readlane(js, r);
                if (active) st_nt(reinterpret_cast<u32x4*>(p.send_x + row * rb) + c, v);
            }
            if (st == 0 && p.G > 0) {
                for (int g = lane; g < p.G; g += kWave) {
                    const float sc = p.src_scales[(int64_t)t * p.G + g];
                    for (uint64_t mm = lmask; mm != 0; mm &= mm - 1)
                        p.recv_scales[(int64_t)readlane(ds, __builtin_ctzll(mm)) * p.G + g] = sc;
                    for (uint64_t mm = smask; mm != 0; mm &= mm - 1) {
                        const int r = __builtin_ctzll(mm);
                        p.send_scales[((int64_t)r * p.T + readlane(js, r)) * p.G + g] = sc;
                    }
                }
            }
        }
    }
    pad_items<false>(p, gw, lane, pw);
}

}  // namespace

hipError_t launch_dispatch(const Handle& h, const DispatchArgs& a, hipStream_t stream) {
    if (h.T == 0) return hipSuccess;
    const bool fp8 = a.mode == DispatchArgs::kFp8;
    const bool raw_rows = a.mode == DispatchArgs::kRows;
    Params p;
    p.src = static_cast<const uint8_t*>(a.x);
    p.src_scales = raw_rows ? a.x_scales : nullptr;
    p.w = a.topk_weights;
    p.topk_idx = h.topk_idx;
    p.slot = h.ws.slot;
    p.send_slot = h.ws.send_slot;
    p.own_row = (a.expand || raw_rows) ? nullptr : h.ws.send_slot;
    p.pad_rows = h.ws.pad_rows;
    p.pad_total = h.ws.pad_total;
    p.recv_x = static_cast<uint8_t*>(a.out.recv_x);
    p.recv_scales = a.out.recv_x_scales;
    p.recv_src = a.out.recv_src_idx;
    p.recv_w = a.out.recv_topk_weights;
    p.recv_topk_idx = p.own_row != nullptr ? a.out.recv_topk_idx : nullptr;
    const bool windows = h.R > 1 && !raw_rows;
    p.send_x = windows ? static_cast<uint8_t*>(a.out.send_x) : nullptr;
    p.send_scales = windows ? a.out.send_x_scales : nullptr;
    p.send_src = windows ? a.out.send_src_idx : nullptr;
    p.send_topk_idx = windows ? a.out.send_topk_idx : nullptr;
    p.send_topk_w = windows ? a.out.send_topk_weights : nullptr;
    if (!windows) p.send_slot = nullptr;
    p.T = h.T;
    p.H = a.hidden;
    p.K = h.K;
    p.R = h.R;
    p.rank = h.rank;
    p.epr = h.El;
    p.zero_pad = a.zero_pad ? 1 : 0;
    if (fp8) {
        p.row_bytes = a.hidden;
        p.G = a.hidden / 128;
        p.nstep = (a.hidden + 1023) / 1024;
    } else {
        p.row_bytes = raw_rows ? a.row_bytes : 2 * a.hidden;
        p.G = raw_rows ? a.nscales : 0;
        p.nstep = (p.row_bytes / 16 + kWave - 1) / kWave;
    }
    if (p.G == 0) p.recv_scales = nullptr;
    p.ntok_items = (int64_t)h.T * p.nstep;
    const bool meta = p.recv_src != nullptr || p.recv_w != nullptr;
    p.pad_sub = (h.A > 1 && p.own_row == nullptr) ? (a.zero_pad ? p.nstep : (meta ? 1 : 0)) : 0;
    const int64_t max_pad_items = (int64_t)h.El * (h.A - 1) * p.pad_sub;
    int64_t nwaves = p.ntok_items;
    const int64_t per_wave = a.zero_pad ? kPadItemsPerWave : kWave;
    const int64_t pad_waves = (max_pad_items + per_wave - 1) / per_wave;
    if (pad_waves > nwaves) nwaves = pad_waves;
    const int64_t nblocks = (nwaves + kWavesPerBlock - 1) / kWavesPerBlock;
    p.nwaves = nblocks * kWavesPerBlock;
    if (fp8)
        hipLaunchKernelGGL(k_dispatch_fp8, dim3((unsigned)nblocks), dim3(kBlock), 0, stream, p);
    else
        hipLaunchKernelGGL(k_dispatch_raw, dim3((unsigned)nblocks), dim3(kBlock), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ep
