// ep_dispatch.hip -- expert-major dispatch on gfx950 ([DeepEP->MegaMoE] §2.2: each token row is loaded once
// and stored to the send buffer; §2.4: rows are placed expert-major at their expert's cursor; [MoE-comm] §一:
// expert_alignment and do_zero_padding; [DeepEP-hotdry] key techniques: FP8 dispatch).
//
// One wave per token.  FP8: each lane loads 32 contiguous bytes (16 bf16 channels) per 1024-channel
// step, eight lanes form one 128-channel group whose max |x| is reduced with three xor-shuffles, and the
// lane casts its 16 channels to 16 e4m3 bytes, which it then stores as one 16-byte vector to every
// destination row (the token's local slots and its send-window rows).  The group scales go through LDS so
// each destination gets them in one contiguous store.  BF16: 16-byte bit copies.
// Padding rows are handled by extra blocks after the token blocks, one group of blocks per local expert.
// Nothing here decides a position: every row index comes from the layout's slot maps.
#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {
namespace {

constexpr int kBlock = 256;                 // 4 waves
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kSeg = 8;                     // steps held in registers before the stores
constexpr int kPadRowsPerPart = 16;         // padding rows per pad block
constexpr int kMaxGroups = kMaxHidden / 128;

struct Params {
    const uint16_t* x;
    const float* w;
    const int64_t* topk_idx;
    const int32_t* slot;
    const int32_t* send_slot;
    const int32_t* cnt_local;
    const int32_t* psum;
    uint8_t* recv_x;
    float* recv_scales;
    int32_t* recv_src;
    float* recv_w;
    uint8_t* send_x;
    float* send_scales;
    int32_t* send_src;
    int64_t* send_topk_idx;
    float* send_topk_w;
    int T, H, K, R, epr;
    int ntok_blocks;
    int pad_parts;
    int zero_pad;
};

// Metadata of the token's destinations; returns (via refs) the slot and send-row masks.
__device__ __forceinline__ void token_meta(const Params& p, int t, int lane, int& ds, int& js, uint64_t& lmask,
                                           uint64_t& smask) {
    ds = lane < p.K ? p.slot[(int64_t)t * p.K + lane] : -1;
    const float wk = (lane < p.K && p.w != nullptr) ? p.w[(int64_t)t * p.K + lane] : 1.0f;
    if (ds >= 0) {
        if (p.recv_src) p.recv_src[ds] = t;
        if (p.recv_w) p.recv_w[ds] = wk;
    }
    js = (p.send_slot != nullptr && lane < p.R) ? p.send_slot[(int64_t)t * p.R + lane] : -1;
    lmask = ballot(ds >= 0);
    smask = ballot(js >= 0);
    if (smask != 0 && (p.send_src || p.send_topk_idx || p.send_topk_w)) {
        const int64_t e = lane < p.K ? p.topk_idx[(int64_t)t * p.K + lane] : -1;
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

__global__ __launch_bounds__(kBlock) void k_dispatch_fp8(Params p) {
    __shared__ float sc_lds[kWavesPerBlock][kMaxGroups];
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    if ((int)blockIdx.x >= p.ntok_blocks) {
        // ---- padding rows of local expert j ------------------------------------------------------------------
        const int pb = blockIdx.x - p.ntok_blocks;
        const int j = pb / p.pad_parts, part = pb % p.pad_parts;
        const int start = p.psum[j] + p.cnt_local[j], end = p.psum[j + 1];
        const int r0 = start + part * kPadRowsPerPart, r1 = min(end, r0 + kPadRowsPerPart);
        const int G = p.H / 128;
        for (int row = r0 + wv; row < r1; row += kWavesPerBlock) {
            if (lane == 0) {
                if (p.recv_src) p.recv_src[row] = -1;
                if (p.recv_w) p.recv_w[row] = 0.0f;
            }
            if (p.zero_pad) {
                u32x4* dst = reinterpret_cast<u32x4*>(p.recv_x + (int64_t)row * p.H);
                const u32x4 z = {0u, 0u, 0u, 0u};
                for (int c = lane; c < p.H / 16; c += kWave) st_nt(dst + c, z);
                for (int g = lane; g < G; g += kWave) p.recv_scales[(int64_t)row * G + g] = 0.0f;
            }
        }
        return;
    }

    const int t = blockIdx.x * kWavesPerBlock + wv;
    if (t >= p.T) return;
    int ds, js;
    uint64_t lmask, smask;
    token_meta(p, t, lane, ds, js, lmask, smask);
    if ((lmask | smask) == 0) return;

    const int H = p.H, G = H / 128;
    const int nstep = (H + 1023) / 1024;
    const uint16_t* xrow = p.x + (int64_t)t * H;
    float* sc = sc_lds[wv];
    for (int seg = 0; seg < nstep; seg += kSeg) {
        u32x4 q[kSeg];
#pragma unroll
        for (int i = 0; i < kSeg; ++i) {
            const int st = seg + i;
            const int ch = (st * kWave + lane) * 16;
            const bool active = st < nstep && ch < H;
            u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
            if (active) {
                const u32x4* src = reinterpret_cast<const u32x4*>(xrow + ch);
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
            if (st < nstep) m = group8_max(m);           // uniform condition: all lanes shuffle together
            const float amax = fmaxf(m, 1e-4f);
            const float scale = amax / 448.0f;           // IEEE division (correctly rounded)
            const float inv = 448.0f / amax;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                q[i][k] = pack_e4m3x4(f[4 * k] * inv, f[4 * k + 1] * inv, f[4 * k + 2] * inv, f[4 * k + 3] * inv);
            if (active && (lane & 7) == 0) sc[st * 8 + (lane >> 3)] = scale;
        }
        // stores: every destination row gets the same 16-byte vectors
        for (uint64_t m = lmask; m != 0; m &= m - 1) {
            const int s = readlane(ds, __builtin_ctzll(m));
            u32x4* dst = reinterpret_cast<u32x4*>(p.recv_x + (int64_t)s * H);
#pragma unroll
            for (int i = 0; i < kSeg; ++i) {
                const int st = seg + i;
                const int ch = (st * kWave + lane) * 16;
                if (st < nstep && ch < H) st_nt(dst + ch / 16, q[i]);
            }
        }
        for (uint64_t m = smask; m != 0; m &= m - 1) {
            const int r = __builtin_ctzll(m);
            const int64_t row = (int64_t)r * p.T + readlane(js, r);
            u32x4* dst = reinterpret_cast<u32x4*>(p.send_x + row * H);
#pragma unroll
            for (int i = 0; i < kSeg; ++i) {
                const int st = seg + i;
                const int ch = (st * kWave + lane) * 16;
                if (st < nstep && ch < H) st_nt(dst + ch / 16, q[i]);
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int g0 = 0; g0 < G; g0 += kWave) {
        const int g = g0 + lane;
        const float s_g = g < G ? sc[g] : 0.0f;
        for (uint64_t m = lmask; m != 0; m &= m - 1) {
            const int s = readlane(ds, __builtin_ctzll(m));
            if (g < G) p.recv_scales[(int64_t)s * G + g] = s_g;
        }
        for (uint64_t m = smask; m != 0; m &= m - 1) {
            const int r = __builtin_ctzll(m);
            const int64_t row = (int64_t)r * p.T + readlane(js, r);
            if (g < G) p.send_scales[row * G + g] = s_g;
        }
    }
}

__global__ __launch_bounds__(kBlock) void k_dispatch_bf16(Params p) {
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    const int nchunk = p.H / 8;                            // 16-byte chunks per row
    if ((int)blockIdx.x >= p.ntok_blocks) {
        const int pb = blockIdx.x - p.ntok_blocks;
        const int j = pb / p.pad_parts, part = pb % p.pad_parts;
        const int start = p.psum[j] + p.cnt_local[j], end = p.psum[j + 1];
        const int r0 = start + part * kPadRowsPerPart, r1 = min(end, r0 + kPadRowsPerPart);
        for (int row = r0 + wv; row < r1; row += kWavesPerBlock) {
            if (lane == 0) {
                if (p.recv_src) p.recv_src[row] = -1;
                if (p.recv_w) p.recv_w[row] = 0.0f;
            }
            if (p.zero_pad) {
                u32x4* dst = reinterpret_cast<u32x4*>(p.recv_x + (int64_t)row * p.H * 2);
                const u32x4 z = {0u, 0u, 0u, 0u};
                for (int c = lane; c < nchunk; c += kWave) st_nt(dst + c, z);
            }
        }
        return;
    }

    const int t = blockIdx.x * kWavesPerBlock + wv;
    if (t >= p.T) return;
    int ds, js;
    uint64_t lmask, smask;
    token_meta(p, t, lane, ds, js, lmask, smask);
    if ((lmask | smask) == 0) return;

    const int nstep = (nchunk + kWave - 1) / kWave;
    const u32x4* src = reinterpret_cast<const u32x4*>(p.x + (int64_t)t * p.H);
    for (int seg = 0; seg < nstep; seg += kSeg) {
        u32x4 v[kSeg];
#pragma unroll
        for (int i = 0; i < kSeg; ++i) {
            const int c = (seg + i) * kWave + lane;
            if (seg + i < nstep && c < nchunk) v[i] = ld_nt(src + c);
        }
        for (uint64_t m = lmask; m != 0; m &= m - 1) {
            const int s = readlane(ds, __builtin_ctzll(m));
            u32x4* dst = reinterpret_cast<u32x4*>(p.recv_x + (int64_t)s * p.H * 2);
#pragma unroll
            for (int i = 0; i < kSeg; ++i) {
                const int c = (seg + i) * kWave + lane;
                if (seg + i < nstep && c < nchunk) st_nt(dst + c, v[i]);
            }
        }
        for (uint64_t m = smask; m != 0; m &= m - 1) {
            const int r = __builtin_ctzll(m);
            const int64_t row = (int64_t)r * p.T + readlane(js, r);
            u32x4* dst = reinterpret_cast<u32x4*>(p.send_x + row * p.H * 2);
#pragma unroll
            for (int i = 0; i < kSeg; ++i) {
                const int c = (seg + i) * kWave + lane;
                if (seg + i < nstep && c < nchunk) st_nt(dst + c, v[i]);
            }
        }
    }
}

}  // namespace

hipError_t launch_dispatch(const Handle& h, const DispatchArgs& a, hipStream_t stream) {
    if (h.T == 0) return hipSuccess;
    Params p;
    p.x = static_cast<const uint16_t*>(a.x);
    p.w = a.topk_weights;
    p.topk_idx = h.topk_idx;
    p.slot = h.ws.slot;
    p.send_slot = h.R > 1 ? h.ws.send_slot : nullptr;
    p.cnt_local = h.ws.cnt_local;
    p.psum = h.ws.psum;
    p.recv_x = static_cast<uint8_t*>(a.out.recv_x);
    p.recv_scales = a.fp8 ? a.out.recv_x_scales : nullptr;
    p.recv_src = a.out.recv_src_idx;
    p.recv_w = a.out.recv_topk_weights;
    p.send_x = h.R > 1 ? static_cast<uint8_t*>(a.out.send_x) : nullptr;
    p.send_scales = (h.R > 1 && a.fp8) ? a.out.send_x_scales : nullptr;
    p.send_src = h.R > 1 ? a.out.send_src_idx : nullptr;
    p.send_topk_idx = h.R > 1 ? a.out.send_topk_idx : nullptr;
    p.send_topk_w = h.R > 1 ? a.out.send_topk_weights : nullptr;
    p.T = h.T;
    p.H = a.hidden;
    p.K = h.K;
    p.R = h.R;
    p.epr = h.El;
    p.zero_pad = a.zero_pad ? 1 : 0;
    p.ntok_blocks = (h.T + kWavesPerBlock - 1) / kWavesPerBlock;
    const bool pads = h.A > 1 && (a.zero_pad || p.recv_src != nullptr || p.recv_w != nullptr);
    p.pad_parts = pads ? (h.A - 1 + kPadRowsPerPart - 1) / kPadRowsPerPart : 1;
    const int64_t nblocks = (int64_t)p.ntok_blocks + (pads ? (int64_t)h.El * p.pad_parts : 0);
    if (a.fp8)
        hipLaunchKernelGGL(k_dispatch_fp8, dim3((unsigned)nblocks), dim3(kBlock), 0, stream, p);
    else
        hipLaunchKernelGGL(k_dispatch_bf16, dim3((unsigned)nblocks), dim3(kBlock), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ep
