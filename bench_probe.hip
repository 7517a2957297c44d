// bench_probe.hip -- measurement probes for bench.py (not part of the library, and not behind include/ep.h).
//
// The two dispatch probes each replay one half of the FP8 dispatch's memory traffic with the dispatch's own work
// split and launch shape (one wave per 1024-channel segment of a token, then padding segments), so that bench.py
// can time what the hardware gives for that address stream alone; the other two are a cache flush and a plain
// copy:
//   probe_dispatch_writes  every store of an FP8 dispatch with zero padding -- the routed rows' e4m3 bytes
//                          (16-byte non-temporal stores to each destination row), their scales and row metadata,
//                          and the zero-padding rows -- and no source reads;
//   probe_dispatch_reads   every source read of that dispatch -- the token rows (32 bytes per lane, plain loads
//                          as in the dispatch) and the slot map -- and no stores;
//   probe_send_writes      the stores of an FP8 dispatch with send windows and no zero padding -- each token's
//                          e4m3 bytes and scales to its local expert-major rows and to its row in every other
//                          rank's window, the local rows' metadata and the window rows' source index -- and no
//                          source reads;
//   probe_combine_gathers  every gather of the weighted combine -- 16-byte non-temporal loads of each token's rows
//                          of y, one wave per (token, 1 KiB segment), issued as the combine issues them (one row
//                          at a time for 8 or more rows in a grid of 16,384 waves or more, else in batches of up
//                          to 8) -- and no stores;
//   probe_row_writes       the combine's output stream alone: one wave per (token, 1 KiB segment), one 16-byte
//                          non-temporal store per lane, nothing read;
//   probe_flush            plain loads over a large buffer (a cache flush between timed samples);
//   probe_copy             a flat copy, one wave per 1 KiB (a 16-byte non-temporal load, then a store per lane):
//                          the rate this chip gives a 1 : 1 read / write stream, as context for the kernels.
// The dispatch and combine probes store a constant pattern (or nothing), so they say nothing about correctness;
// with both streams coming from HBM, a kernel's reads alone plus its writes alone bound its time from below: the
// reads and the writes share each channel's data bus.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kPadPerWave = 2;   // padding segments per wave, as the dispatch's grid is sized

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct WriteArgs {
    const int32_t* token_rows;   // [T, K] destination row of each entry, -1 none
    const int32_t* pad_rows;     // [npad] padding rows
    uint8_t* recv_x;             // [rows, H] e4m3 bytes
    float* recv_scales;          // [rows, H / 128]
    int32_t* recv_src;           // [rows]
    float* recv_w;               // [rows]
    int T, K, H, npad;
    int nstep;                   // 1024-channel segments per row
    int64_t ntok_items, nwaves;
};

__global__ __launch_bounds__(kBlock) void k_probe_writes(WriteArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    const int G = a.H / 128;
    const int64_t npad_items = (int64_t)a.npad * a.nstep;
    int prow[kPadPerWave];
#pragma unroll
    for (int j = 0; j < kPadPerWave; ++j) {
        const int64_t i = gw + j * a.nwaves;
        prow[j] = i < npad_items ? a.pad_rows[i / a.nstep] : 0;
    }
    if (gw < a.ntok_items) {
        const int t = (int)(gw / a.nstep), s = (int)(gw % a.nstep);
        const int d = lane < a.K ? a.token_rows[(int64_t)t * a.K + lane] : -1;
        const uint64_t m = __builtin_amdgcn_ballot_w64(d >= 0);
        const u32x4 q = {0x3C3C3C3Cu, 0x3C3C3C3Cu, 0x3C3C3C3Cu, 0x3C3C3C3Cu};
        const bool sc_lane = (lane & 7) == 0;
        const int g = s * 8 + (lane >> 3);
        for (uint64_t mm = m; mm != 0; mm &= mm - 1) {
            const int row = __builtin_amdgcn_readlane(d, __builtin_ctzll(mm));
            __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(a.recv_x + (int64_t)row * a.H) + s * kWave + lane);
            if (sc_lane && g < G) a.recv_scales[(int64_t)row * G + g] = 1.0f;
        }
        if (s == 0 && d >= 0) {
            a.recv_src[d] = t;
            a.recv_w[d] = 0.125f;
        }
    }
#pragma unroll
    for (int j = 0; j < kPadPerWave; ++j) {
        const int64_t i = gw + j * a.nwaves;
        if (i >= npad_items) break;
        const int s = (int)(i % a.nstep);
        const u32x4 z = {0u, 0u, 0u, 0u};
        __builtin_nontemporal_store(z, reinterpret_cast<u32x4*>(a.recv_x + (int64_t)prow[j] * a.H) + s * kWave + lane);
        if (lane < 8 && s * 8 + lane < G) a.recv_scales[(int64_t)prow[j] * G + s * 8 + lane] = 0.0f;
        if (s == 0 && lane == 0) {
            a.recv_src[prow[j]] = -1;
            a.recv_w[prow[j]] = 0.0f;
        }
    }
}

struct SendArgs {
    const int32_t* token_rows;   // [T, K] local expert-major row of each entry, -1 none
    const int32_t* send_rows;    // [T, R] row in rank r's window, -1 none (the own rank's column is -1)
    uint8_t* recv_x;
    float* recv_scales;
    int32_t* recv_src;
    float* recv_w;
    uint8_t* send_x;             // [R * T, H]
    float* send_scales;          // [R * T, H / 128]
    int32_t* send_src;           // [R * T]
    int T, K, R, H, nstep;
    int64_t ntok_items;
};

__global__ __launch_bounds__(kBlock) void k_probe_send_writes(SendArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (gw >= a.ntok_items) return;
    const int G = a.H / 128;
    const int t = (int)(gw / a.nstep), s = (int)(gw % a.nstep);
    const int d = lane < a.K ? a.token_rows[(int64_t)t * a.K + lane] : -1;
    const int j = lane < a.R ? a.send_rows[(int64_t)t * a.R + lane] : -1;
    const uint64_t m = __builtin_amdgcn_ballot_w64(d >= 0), ms = __builtin_amdgcn_ballot_w64(j >= 0);
    const u32x4 q = {0x3C3C3C3Cu, 0x3C3C3C3Cu, 0x3C3C3C3Cu, 0x3C3C3C3Cu};
    const bool sc_lane = (lane & 7) == 0;
    const int g = s * 8 + (lane >> 3);
    for (uint64_t mm = m; mm != 0; mm &= mm - 1) {
        const int row = __builtin_amdgcn_readlane(d, __builtin_ctzll(mm));
        __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(a.recv_x + (int64_t)row * a.H) + s * kWave + lane);
        if (sc_lane && g < G) a.recv_scales[(int64_t)row * G + g] = 1.0f;
    }
    for (uint64_t mm = ms; mm != 0; mm &= mm - 1) {
        const int r = __builtin_ctzll(mm);
        const int64_t row = (int64_t)r * a.T + __builtin_amdgcn_readlane(j, r);
        __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(a.send_x + row * a.H) + s * kWave + lane);
        if (sc_lane && g < G) a.send_scales[row * G + g] = 1.0f;
    }
    if (s == 0) {
        if (d >= 0) {
            a.recv_src[d] = t;
            a.recv_w[d] = 0.125f;
        }
        if (j >= 0) a.send_src[(int64_t)lane * a.T + j] = t;
    }
}

struct ReadArgs {
    const uint8_t* x;            // [T, 2H] bf16 rows
    const int32_t* token_rows;   // [T, K]
    int T, K, H, nstep;
    int64_t ntok_items;
    int32_t* sink;               // written only if the loads' xor equals `never` (it does not)
    uint32_t never;
};

__global__ __launch_bounds__(kBlock) void k_probe_reads(ReadArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (gw >= a.ntok_items) return;
    const int t = (int)(gw / a.nstep), s = (int)(gw % a.nstep);
    const int d = lane < a.K ? a.token_rows[(int64_t)t * a.K + lane] : 0;
    const int ch = (s * kWave + lane) * 16;
    uint32_t acc = (uint32_t)d;
    if (ch < a.H) {
        const u32x4* src = reinterpret_cast<const u32x4*>(a.x + ((int64_t)t * a.H + ch) * 2);
        const u32x4 v0 = src[0];
        const u32x4 v1 = src[1];
        acc ^= v0[0] ^ v0[1] ^ v0[2] ^ v0[3] ^ v1[0] ^ v1[1] ^ v1[2] ^ v1[3];
    }
    if (acc == a.never) a.sink[0] = (int32_t)acc;
}

struct GatherArgs {
    const u32x4* y;              // [rows, nchunk] bf16 rows as 16-byte chunks
    const int32_t* token_rows;   // [T, K] rows of each token's entries, valid ones first, -1 past them
    int T, K, nchunk, nseg;      // nchunk: 16-byte chunks per row; nseg: 1 KiB segments per row
    int64_t nitems;
    int stream_one;              // a wave with 8 or more rows loads them one at a time
    int32_t* sink;               // written only if the loads' xor equals `never` (it does not)
    uint32_t never;
};

template <int N>
__device__ __forceinline__ uint32_t gather_xor(const u32x4* base, int rows, int nchunk, int kb) {
    u32x4 v[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
        v[i] = __builtin_nontemporal_load(base + (int64_t)__builtin_amdgcn_readlane(rows, kb + i) * nchunk);
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
    return x;
}

__global__ __launch_bounds__(kBlock) void k_probe_gathers(GatherArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (gw >= a.nitems) return;
    const int t = (int)(gw / a.nseg), s = (int)(gw % a.nseg);
    const int r = lane < a.K ? a.token_rows[(int64_t)t * a.K + lane] : -1;
    const int nv = __builtin_popcountll(__builtin_amdgcn_ballot_w64(r >= 0));
    const int c = s * kWave + lane;
    const u32x4* base = a.y + (c < a.nchunk ? c : 0);
    uint32_t acc = 0;
    if (a.stream_one && nv >= 8) {
        for (int k = 0; k < nv; ++k) acc ^= gather_xor<1>(base, r, a.nchunk, k);
    } else {
        int kb = 0;
        for (; kb + 8 <= nv; kb += 8) acc ^= gather_xor<8>(base, r, a.nchunk, kb);
        switch (nv - kb) {
            case 1: acc ^= gather_xor<1>(base, r, a.nchunk, kb); break;
            case 2: acc ^= gather_xor<2>(base, r, a.nchunk, kb); break;
            case 3: acc ^= gather_xor<3>(base, r, a.nchunk, kb); break;
            case 4: acc ^= gather_xor<4>(base, r, a.nchunk, kb); break;
            case 5: acc ^= gather_xor<5>(base, r, a.nchunk, kb); break;
            case 6: acc ^= gather_xor<6>(base, r, a.nchunk, kb); break;
            case 7: acc ^= gather_xor<7>(base, r, a.nchunk, kb); break;
            default: break;
        }
    }
    if (acc == a.never) a.sink[0] = (int32_t)acc;
}

__global__ __launch_bounds__(kBlock) void k_probe_row_writes(u32x4* out, int nchunk, int nseg, int64_t nitems) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (gw >= nitems) return;
    const int64_t t = gw / nseg;
    const int c = (int)(gw % nseg) * kWave + lane;
    const u32x4 z = {0u, 0u, 0u, 0u};
    if (c < nchunk) __builtin_nontemporal_store(z, out + t * nchunk + c);
}

__global__ __launch_bounds__(kBlock) void k_probe_flush(const u32x4* p, int64_t n16, int32_t* sink, uint32_t never) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n16; i += 4 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = p[i + u * stride < n16 ? i + u * stride : i];
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][3];
    }
    if (acc == never) sink[0] = (int32_t)acc;
}

__global__ __launch_bounds__(kBlock) void k_probe_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                       int64_t n16) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

extern "C" {

// Returns 0, or -1 on an argument outside what the probe handles (nothing is launched then), or the HIP error.
int probe_dispatch_writes(const int32_t* token_rows, int T, int K, const int32_t* pad_rows, int npad, void* recv_x,
                          float* recv_scales, int32_t* recv_src, float* recv_w, int H, void* stream) {
    if (T < 1 || K < 1 || K > kWave || npad < 0 || H < 1024 || H % 1024 != 0) return -1;
    WriteArgs a;
    a.token_rows = token_rows;
    a.pad_rows = pad_rows;
    a.recv_x = static_cast<uint8_t*>(recv_x);
    a.recv_scales = recv_scales;
    a.recv_src = recv_src;
    a.recv_w = recv_w;
    a.T = T;
    a.K = K;
    a.H = H;
    a.npad = npad;
    a.nstep = H / 1024;
    a.ntok_items = (int64_t)T * a.nstep;
    int64_t nwaves = a.ntok_items;
    const int64_t pad_waves = ((int64_t)npad * a.nstep + kPadPerWave - 1) / kPadPerWave;
    if (pad_waves > nwaves) nwaves = pad_waves;
    const int64_t nblocks = (nwaves + kWavesPerBlock - 1) / kWavesPerBlock;
    a.nwaves = nblocks * kWavesPerBlock;
    hipLaunchKernelGGL(k_probe_writes, dim3((unsigned)nblocks), dim3(kBlock), 0, static_cast<hipStream_t>(stream), a);
    return (int)hipGetLastError();
}

// Returns 0, or -1 on an argument outside what the probe handles (nothing is launched then), or the HIP error.
int probe_send_writes(const int32_t* token_rows, const int32_t* send_rows, int T, int K, int R, void* recv_x,
                      float* recv_scales, int32_t* recv_src, float* recv_w, void* send_x, float* send_scales,
                      int32_t* send_src, int H, void* stream) {
    if (T < 1 || K < 1 || K > kWave || R < 1 || R > kWave || H < 1024 || H % 1024 != 0) return -1;
    SendArgs a;
    a.token_rows = token_rows;
    a.send_rows = send_rows;
    a.recv_x = static_cast<uint8_t*>(recv_x);
    a.recv_scales = recv_scales;
    a.recv_src = recv_src;
    a.recv_w = recv_w;
    a.send_x = static_cast<uint8_t*>(send_x);
    a.send_scales = send_scales;
    a.send_src = send_src;
    a.T = T;
    a.K = K;
    a.R = R;
    a.H = H;
    a.nstep = H / 1024;
    a.ntok_items = (int64_t)T * a.nstep;
    const int64_t nblocks = (a.ntok_items + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(k_probe_send_writes, dim3((unsigned)nblocks), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                       a);
    return (int)hipGetLastError();
}

int probe_dispatch_reads(const void* x, const int32_t* token_rows, int T, int K, int H, int32_t* sink, void* stream) {
    if (T < 1 || K < 1 || K > kWave || H < 1024 || H % 1024 != 0) return -1;
    ReadArgs a;
    a.x = static_cast<const uint8_t*>(x);
    a.token_rows = token_rows;
    a.T = T;
    a.K = K;
    a.H = H;
    a.nstep = H / 1024;
    a.ntok_items = (int64_t)T * a.nstep;
    a.sink = sink;
    a.never = 0x9E3779B9u;
    const int64_t nblocks = (a.ntok_items + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(k_probe_reads, dim3((unsigned)nblocks), dim3(kBlock), 0, static_cast<hipStream_t>(stream), a);
    return (int)hipGetLastError();
}

// y: rows of H bf16 values; token_rows [T, K] as for probe_dispatch_reads.
int probe_combine_gathers(const void* y, const int32_t* token_rows, int T, int K, int H, int32_t* sink, void* stream) {
    if (T < 1 || K < 1 || K > kWave || H < 8 || H % 8 != 0) return -1;
    GatherArgs a;
    a.y = static_cast<const u32x4*>(y);
    a.token_rows = token_rows;
    a.T = T;
    a.K = K;
    a.nchunk = H / 8;
    a.nseg = (a.nchunk + kWave - 1) / kWave;
    a.nitems = (int64_t)T * a.nseg;
    a.stream_one = a.nitems >= 16384 ? 1 : 0;
    a.sink = sink;
    a.never = 0x9E3779B9u;
    const int64_t nblocks = (a.nitems + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(k_probe_gathers, dim3((unsigned)nblocks), dim3(kBlock), 0, static_cast<hipStream_t>(stream), a);
    return (int)hipGetLastError();
}

// out: [T, H] bf16 rows, overwritten with zeros.
int probe_row_writes(void* out, int T, int H, void* stream) {
    if (T < 1 || H < 8 || H % 8 != 0) return -1;
    const int nchunk = H / 8, nseg = (nchunk + kWave - 1) / kWave;
    const int64_t nitems = (int64_t)T * nseg;
    const int64_t nblocks = (nitems + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(k_probe_row_writes, dim3((unsigned)nblocks), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                       static_cast<u32x4*>(out), nchunk, nseg, nitems);
    return (int)hipGetLastError();
}

int probe_flush(const void* buf, int64_t bytes, int32_t* sink, void* stream) {
    if (bytes < 16) return -1;
    hipLaunchKernelGGL(k_probe_flush, dim3(2048), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(buf), bytes / 16, sink, 0x9E3779B9u);
    return (int)hipGetLastError();
}

int probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (bytes < 16 || bytes % 16 != 0 || bytes / 16 / kBlock >= (int64_t)1 << 31) return -1;
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(k_probe_copy, dim3((unsigned)((n16 + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
    return (int)hipGetLastError();
}

}  // extern "C"
