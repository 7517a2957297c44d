// ep_dispatch_core.hpp -- per-item device code of the dispatch ([DeepEP->MegaMoE] §2.2: each token row is loaded
// once and stored to every destination; §2.4: rows are placed expert-major; [MoE-comm] §一: expert_alignment,
// do_zero_padding and do_expand; [DeepEP-hotdry] key techniques: FP8 dispatch), shared by the dispatch kernels
// (ep_dispatch.hip) and the one-launch layout + dispatch kernel for small batches (ep_fused.hip).  The callers
// decide where a token's destinations come from (the layout in the workspace, or the layout in LDS); the code
// here moves the bytes and writes the per-row metadata.
#pragma once

#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {
namespace {

constexpr int kPadItemsPerWave = 2;   // worst-case zero-padding items per wave used to size the grids
constexpr int kFp8Channels = 1024;    // channels per FP8 token item (64 lanes x 16)
constexpr int kRawChunks = kWave;     // 16-byte chunks per raw token item (1 KiB)

struct Params {
    const uint8_t* src;          // token rows: bf16 [T, H] (FP8 items) or row_bytes-byte rows (raw items)
    const float* src_scales;     // raw items: [T, G] scales travelling with the rows, or nullptr
    const float* w;
    const int64_t* topk_idx;
    const int32_t* slot;         // [T, K] expert-major rows (workspace)
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
    int token_major;  // do_expand off: one local row per token, K-entry metadata
    int row_bytes;    // bytes of one destination row
    int G;            // fp32 scales per row (FP8: H / 128; raw: as given, 0 for none)
    int nstep;        // segments per row
    int64_t ntok_items;   // token work items: T x items per token (set by the dispatch launcher)
    int pad_sub;      // padding items per padding row (nstep with zero padding, 1 for metadata only, 0 none)
    int zero_pad;
    int64_t nwaves;   // waves in the grid
};

// Metadata of token t's rows, written by the wave of its segment 0.  ds (lanes < K expert-major, lane 0
// token-major) and js (lanes < R) are the token's local and send rows, lmask / smask their ballots.
// The token's routing weight and expert id for lane k < K, as loaded ahead of token_meta by token_entry.  The
// loads take the entry index clamped into the token's entries and a valid address in place of absent weights, so
// that they need no branch; the values are raw (lanes >= K hold entry K - 1, and without weights the weight is a
// bit pattern of the ids), and token_meta applies the masks where it uses them, so that no early use makes a wait
// for these loads wait for every load issued before them.
struct TokenEntry {
    float w;
    int64_t e;
};

__device__ __forceinline__ TokenEntry token_entry(const Params& p, int t, int lane) {
    const int64_t j = (int64_t)t * p.K + min(lane, p.K - 1);
    const float* w = p.w != nullptr ? p.w : reinterpret_cast<const float*>(p.topk_idx);   // T*K*8 bytes
    TokenEntry te;
    te.w = w[j];
    te.e = p.topk_idx[j];
    return te;
}

__device__ __forceinline__ void token_meta(const Params& p, int t, int lane, int ds, int js, uint64_t lmask,
                                           uint64_t smask, const TokenEntry* pre = nullptr) {
    const bool need_e = (smask != 0 && p.send_topk_idx != nullptr) ||
                        (p.token_major && lmask != 0 && p.recv_topk_idx != nullptr);
    float wk;
    int64_t e;
    if (pre != nullptr) {   // token_entry's raw values, masked here
        wk = (lane < p.K && p.w != nullptr) ? pre->w : 1.0f;
        e = lane < p.K ? pre->e : -1;
    } else {
        wk = (lane < p.K && p.w != nullptr) ? p.w[(int64_t)t * p.K + lane] : 1.0f;
        e = (need_e && lane < p.K) ? p.topk_idx[(int64_t)t * p.K + lane] : -1;
    }
    if (!p.token_major) {
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

// FP8 segment st of token t: channels [1024 st, 1024 st + 1024).  Each lane loads 32 contiguous bytes (16 bf16
// channels); eight lanes form one 128-channel group whose max |x| comes from three DPP lane swaps; the lane casts
// its 16 channels to 16 e4m3 bytes and stores them as one 16-byte vector to every destination row, together
// with the segment's 8 group scales.
// The segment's source bytes, loaded by fp8_load before the destinations are known (so the loads can overlap
// other work) and consumed by fp8_emit.
// Source rows are read with plain (cached) loads, here and in raw_load: each row is read once, but unlike
// non-temporal loads they leave it in the memory-side cache, where a dispatch of the same rows right after finds
// it (prefill: 75.9 -> 66.9 us back to back); with the cache cleared first they are also faster (80.1 -> 78.7 us).
struct Fp8Src {
    u32x4 a, b;
};

__device__ __forceinline__ Fp8Src fp8_load(const Params& p, int t, int st, int lane) {
    Fp8Src v;
    v.a = u32x4{0u, 0u, 0u, 0u};
    v.b = u32x4{0u, 0u, 0u, 0u};
    const int ch = (st * kWave + lane) * 16;      // first channel of this lane
    if (ch < p.H) {
        const u32x4* src = reinterpret_cast<const u32x4*>(p.src + ((int64_t)t * p.H + ch) * 2);
        v.a = src[0];
        v.b = src[1];
    }
    return v;
}

// fp8_load with the lane's channel clamped into the row (H is a multiple of 128, so a lane past the row belongs to
// a group past the row, whose bytes and scale are never stored): no branch around the loads.
__device__ __forceinline__ Fp8Src fp8_load_clamped(const Params& p, int t, int st, int lane) {
    const int ch = min((st * kWave + lane) * 16, p.H - 16);
    const u32x4* src = reinterpret_cast<const u32x4*>(p.src + ((int64_t)t * p.H + ch) * 2);
    Fp8Src v;
    v.a = src[0];
    v.b = src[1];
    return v;
}

// The cast of one lane's 16 channels: 16 e4m3 bytes and its group's scale.
struct Fp8Row {
    u32x4 q;
    float scale;
};

__device__ __forceinline__ Fp8Row fp8_cast(const Fp8Src& v) {
    const u32x4 a = v.a, b = v.b;
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
    Fp8Row r;
    r.scale = amax / 448.0f;                     // IEEE division (correctly rounded)
    const float inv = 448.0f / amax;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        r.q[k] = pack_e4m3x4(f[4 * k] * inv, f[4 * k + 1] * inv, f[4 * k + 2] * inv, f[4 * k + 3] * inv);
    return r;
}

// Stores of segment st's cast bytes and scales to every destination row (local rows, then send rows).
__device__ __forceinline__ void fp8_store(const Params& p, int st, int lane, const Fp8Row& c, int ds, int js,
                                          uint64_t lmask, uint64_t smask) {
    const int H = p.H, G = H / 128;
    const bool active = (st * kWave + lane) * 16 < H;
    // lane 8 j stores the scale of group 8 st + j: the 8 stores of a segment are contiguous (one 32-byte write)
    const int g = st * 8 + (lane >> 3);
    const bool sc_lane = (lane & 7) == 0 && g < G;
    for (uint64_t mm = lmask; mm != 0; mm &= mm - 1) {
        const int s = readlane(ds, __builtin_ctzll(mm));
        if (active) st_nt(reinterpret_cast<u32x4*>(p.recv_x + (int64_t)s * H) + st * kWave + lane, c.q);
        if (sc_lane) p.recv_scales[(int64_t)s * G + g] = c.scale;
    }
    for (uint64_t mm = smask; mm != 0; mm &= mm - 1) {
        const int r = __builtin_ctzll(mm);
        const int64_t row = (int64_t)r * p.T + readlane(js, r);
        if (active) st_nt(reinterpret_cast<u32x4*>(p.send_x + row * H) + st * kWave + lane, c.q);
        if (sc_lane) p.send_scales[row * G + g] = c.scale;
    }
}

__device__ __forceinline__ void fp8_emit(const Params& p, int st, int lane, const Fp8Src& v, int ds, int js,
                                         uint64_t lmask, uint64_t smask) {
    fp8_store(p, st, lane, fp8_cast(v), ds, js, lmask, smask);
}


// Raw segment st of row t (BF16 dispatch, and received rows that already carry their receive format): 16-byte
// copies of one 1 KiB segment; segment 0 also copies the row's scales, if any.
__device__ __forceinline__ u32x4 raw_load(const Params& p, int t, int st, int lane) {
    const int c = st * kWave + lane;                  // 16-byte chunk of the row
    u32x4 v = {0u, 0u, 0u, 0u};
    if (c < p.row_bytes / 16) v = reinterpret_cast<const u32x4*>(p.src + (int64_t)t * p.row_bytes)[c];
    return v;
}

// raw_load with the chunk clamped into the row (row_bytes >= 16; chunks past the row are never stored).
__device__ __forceinline__ u32x4 raw_load_clamped(const Params& p, int t, int st, int lane) {
    const int c = min(st * kWave + lane, p.row_bytes / 16 - 1);
    return reinterpret_cast<const u32x4*>(p.src + (int64_t)t * p.row_bytes)[c];
}

__device__ __forceinline__ void raw_emit(const Params& p, int t, int st, int lane, u32x4 v, int ds, int js,
                                         uint64_t lmask, uint64_t smask) {
    const int c = st * kWave + lane;                  // 16-byte chunk of the row
    const bool active = c < p.row_bytes / 16;
    const int64_t rb = p.row_bytes;
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


// Zero-padding item: segment s of padding row `row` gets zero bytes (and its share of the scales); segment 0
// also writes the row's metadata.
template <bool FP8>
__device__ __forceinline__ void pad_zero_segment(const Params& p, int row, int s, int lane) {
    const int G = p.G;
    const int nchunk = p.row_bytes / 16;            // 16-byte chunks per row
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int c = s * kWave + lane;
    if (c < nchunk) st_nt(reinterpret_cast<u32x4*>(p.recv_x + (int64_t)row * p.row_bytes) + c, z);
    if (FP8) {
        if (lane < 8 && s * 8 + lane < G) p.recv_scales[(int64_t)row * G + s * 8 + lane] = 0.0f;
    } else if (s == 0) {
        for (int g = lane; g < G; g += kWave) p.recv_scales[(int64_t)row * G + g] = 0.0f;
    }
    if (s == 0 && lane == 0) {
        if (p.recv_src) p.recv_src[row] = -1;
        if (p.recv_w) p.recv_w[row] = 0.0f;
    }
}

// Metadata of one padding row (without zero padding only the metadata is written).
__device__ __forceinline__ void pad_meta_row(const Params& p, int row) {
    if (p.recv_src) p.recv_src[row] = -1;
    if (p.recv_w) p.recv_w[row] = 0.0f;
}

// Kernel parameters of one dispatch call (everything except the grid-dependent nwaves).
inline Params dispatch_params(const Handle& h, const DispatchArgs& a) {
    const bool fp8 = a.mode == DispatchArgs::kFp8;
    const bool raw_rows = a.mode == DispatchArgs::kRows;
    const bool token_major = !a.expand && !raw_rows;
    Params p;
    p.src = static_cast<const uint8_t*>(a.x);
    p.src_scales = raw_rows ? a.x_scales : nullptr;
    p.w = a.topk_weights;
    p.topk_idx = h.topk_idx;
    p.slot = h.ws.slot;
    p.own_row = token_major ? h.ws.send_slot : nullptr;
    p.pad_rows = h.ws.pad_rows;
    p.pad_total = h.ws.pad_total;
    p.recv_x = static_cast<uint8_t*>(a.out.recv_x);
    p.recv_scales = a.out.recv_x_scales;
    p.recv_src = a.out.recv_src_idx;
    p.recv_w = a.out.recv_topk_weights;
    p.recv_topk_idx = token_major ? a.out.recv_topk_idx : nullptr;
    const bool windows = h.R > 1 && !raw_rows;
    p.send_slot = windows ? h.ws.send_slot : nullptr;
    p.send_x = windows ? static_cast<uint8_t*>(a.out.send_x) : nullptr;
    p.send_scales = windows ? a.out.send_x_scales : nullptr;
    p.send_src = windows ? a.out.send_src_idx : nullptr;
    p.send_topk_idx = windows ? a.out.send_topk_idx : nullptr;
    p.send_topk_w = windows ? a.out.send_topk_weights : nullptr;
    p.T = h.T;
    p.H = a.hidden;
    p.K = h.K;
    p.R = h.R;
    p.rank = h.rank;
    p.epr = h.El;
    p.token_major = token_major ? 1 : 0;
    p.zero_pad = a.zero_pad ? 1 : 0;
    if (fp8) {
        p.row_bytes = a.hidden;
        p.G = a.hidden / 128;
        p.nstep = (a.hidden + kFp8Channels - 1) / kFp8Channels;
    } else {
        p.row_bytes = raw_rows ? a.row_bytes : 2 * a.hidden;
        p.G = raw_rows ? a.nscales : 0;
        p.nstep = (p.row_bytes / 16 + kRawChunks - 1) / kRawChunks;
    }
    if (p.G == 0) p.recv_scales = nullptr;
    p.ntok_items = 0;
    const bool meta = p.recv_src != nullptr || p.recv_w != nullptr;
    p.pad_sub = (h.A > 1 && !token_major) ? (a.zero_pad ? p.nstep : (meta ? 1 : 0)) : 0;
    p.nwaves = 0;
    return p;
}

}  // namespace
}  // namespace ep
