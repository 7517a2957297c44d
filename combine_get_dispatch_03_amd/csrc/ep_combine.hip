// ep_combine.hip -- top-k reduction back to token order on gfx950 ([DeepEP->MegaMoE] §2.3 and §2.5: per
// token, element-wise accumulation of the top-k expert output rows; §3.2 phase 6: accumulate then store the
// token's output row; [MoE-comm] §一: the shared-expert output enters as bias).
//
// The same kernel moves the token-major rows back (do_expand off): one slot per token, its row among this
// rank's tokens, with unit weight.
//
// Work items are 1 KiB output segments (512 channels): item (t, s) is segment s of token t's output row, so
// a token's row is produced by several short waves instead of one long one, which keeps more gathers in
// flight across the chip.  The token's valid (slot, weight) pairs are compacted into lanes 0..nv-1 and read
// back as scalars, so every gather is a 64-lane x 16-byte row segment at a uniform base.  The gathers are
// straight-line code with no per-lane predicate (lanes past the row's end read chunk 0 and store nothing): a
// predicated load whose consumer sits in another branch makes the compiler wait for every earlier load
// before issuing it, so a batch would never have more than one gather in flight.  fp32 accumulation in
// ascending k, one RNE rounding to bf16 at the end.
#include <climits>

#include "ep_device.hpp"
#include "ep_internal.hpp"

namespace ep {
namespace {

constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
// Streaming a wave's rows one at a time pays only when the grid keeps HBM saturated by itself: with at least
// kStreamMinWaves waves (twice what the chip holds at once) a wave with at least kCombineStreamRows rows
// (kReduceStreamRows for the reduce, which also reads a local and a bias row) streams them; smaller grids are
// latency-bound and issue every row in batches of 8.  Measured: prefill combine (57,344 waves of 8 rows)
// about 1% faster streaming; decode combine (1,792 waves of 8 rows) 23% faster batched.
constexpr int kCombineStreamRows = 8;
constexpr int kReduceStreamRows = 4;
constexpr int64_t kStreamMinWaves = 16384;

struct Params {
    const uint16_t* y;
    const float* w;
    const uint16_t* bias;
    uint16_t* out;
    const int32_t* slot;   // row of entry k of token t at slot[t * stride + k]
    int T, H, K, stride;
    int nseg;          // 1 KiB segments per row
    int64_t nitems;    // T * nseg
    int stream_min;    // a wave with at least this many rows streams them
};

__device__ __forceinline__ void fma8(float* acc, float wgt, u32x4 v) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        acc[2 * k] = fmaf(wgt, bf16lo(v[k]), acc[2 * k]);
        acc[2 * k + 1] = fmaf(wgt, bf16hi(v[k]), acc[2 * k + 1]);
    }
}

__device__ __forceinline__ void add8(float* acc, u32x4 v) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        acc[2 * k] += bf16lo(v[k]);
        acc[2 * k + 1] += bf16hi(v[k]);
    }
}

__device__ __forceinline__ u32x4 pack8(const float* acc) {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = pack_bf16x2(acc[2 * k], acc[2 * k + 1]);
    return r;
}

// N rows gathered from base + rows[kb + i] * stride (compacted in lanes, read back as scalars), all N issued
// before the first use, then acc += w[kb + i] * row (WEIGHTED) or acc += row, in ascending i.
template <int N, bool WEIGHTED>
__device__ __forceinline__ void gather_acc(float* acc, const u32x4* base, int64_t stride, int rows, float w,
                                           int kb) {
    u32x4 v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = ld_nt(base + (int64_t)readlane(rows, kb + i) * stride);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (WEIGHTED)
            fma8(acc, readlane_f(w, kb + i), v[i]);
        else
            add8(acc, v[i]);
    }
}

// All nv compacted rows: streamed one at a time when nv >= stream_min, else issued in unrolled batches of 8
// (full batches, then one remainder batch of 1..7).
template <bool WEIGHTED>
__device__ __forceinline__ void gather_all(float* acc, const u32x4* base, int64_t stride, int rows, float w,
                                           int nv, int stream_min) {
    if (nv >= stream_min) {
        for (int k = 0; k < nv; ++k) gather_acc<1, WEIGHTED>(acc, base, stride, rows, w, k);
        return;
    }
    int kb = 0;
    for (; kb + 8 <= nv; kb += 8) gather_acc<8, WEIGHTED>(acc, base, stride, rows, w, kb);
    switch (nv - kb) {
        case 1: gather_acc<1, WEIGHTED>(acc, base, stride, rows, w, kb); break;
        case 2: gather_acc<2, WEIGHTED>(acc, base, stride, rows, w, kb); break;
        case 3: gather_acc<3, WEIGHTED>(acc, base, stride, rows, w, kb); break;
        case 4: gather_acc<4, WEIGHTED>(acc, base, stride, rows, w, kb); break;
        case 5: gather_acc<5, WEIGHTED>(acc, base, stride, rows, w, kb); break;
        case 6: gather_acc<6, WEIGHTED>(acc, base, stride, rows, w, kb); break;
        case 7: gather_acc<7, WEIGHTED>(acc, base, stride, rows, w, kb); break;
        default: break;
    }
}

__global__ __launch_bounds__(kBlock) void k_combine(Params p) {
    // both argument lines in one round trip (the fields are read on demand otherwise, one miss after another):
    // decode combine 3.29 -> 3.12 us, prefill 87.1 -> 86.4 us (in the dispatch kernels the same cost time)
    touch_kernargs<sizeof(Params)>();
    __shared__ int cs_lds[kWavesPerBlock][kWave];
    __shared__ float cw_lds[kWavesPerBlock][kWave];
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wv;
    if (item >= p.nitems) return;
    const int t = (int)(item / p.nseg), seg = (int)(item % p.nseg);

    // compact the token's valid slots (ascending k) into lanes 0..nv-1
    const int s = lane < p.K ? p.slot[(int64_t)t * p.stride + lane] : -1;
    const float wk = lane < p.K ? (p.w != nullptr ? p.w[(int64_t)t * p.K + lane] : 1.0f) : 0.0f;
    const uint64_t vm = ballot(s >= 0);
    const int nv = popc64(vm);
    if (s >= 0) {
        const int pos = popc64(vm & lanemask_lt());
        cs_lds[wv][pos] = s;
        cw_lds[wv][pos] = wk;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int cs = lane < nv ? cs_lds[wv][lane] : 0;
    const float cw = lane < nv ? cw_lds[wv][lane] : 0.0f;

    const int c = seg * kWave + lane;                      // 16-byte chunk of the row
    const bool active = c < p.H / 8;
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
    gather_all<true>(acc, reinterpret_cast<const u32x4*>(p.y) + (active ? c : 0), p.H / 8, cs, cw, nv, p.stream_min);
    if (!active) return;
    if (p.bias != nullptr) add8(acc, reinterpret_cast<const u32x4*>(p.bias + (int64_t)t * p.H)[c]);
    st_nt(reinterpret_cast<u32x4*>(p.out + (int64_t)t * p.H) + c, pack8(acc));
}

// Source-side reduce after the combine exchange ([DeepEP->MegaMoE] §2.5: the reduce epilogue adds the rows
// that come back from the ranks that held the token's experts; [MoE-comm] §一: plus the shared-expert bias).
// Item (t, s) = 1 KiB segment s of token t: lanes r < R read the token's window rows, the valid ones are
// compacted and gathered like combine's expert rows; fp32 sum of local, then ranks in ascending order, then
// bias; one RNE rounding.
struct ReduceParams {
    const uint16_t* partials;   // [R, T, H]
    const uint16_t* local;
    const uint16_t* bias;
    uint16_t* out;
    const int32_t* send_slot;   // [T, R] or nullptr (R == 1)
    int T, H, R, rank;
    int nseg;
    int64_t nitems;
    int stream_min;
};

__global__ __launch_bounds__(kBlock) void k_combine_reduce(ReduceParams p) {
    touch_kernargs<sizeof(ReduceParams)>();
    __shared__ int cs_lds[kWavesPerBlock][kWave];
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wv;
    if (item >= p.nitems) return;
    const int t = (int)(item / p.nseg), seg = (int)(item % p.nseg);
    int64_t row = -1;                                      // window row of token t for rank `lane`
    if (p.send_slot != nullptr && lane < p.R && lane != p.rank) {
        const int j = p.send_slot[(int64_t)t * p.R + lane];
        if (j >= 0) row = (int64_t)lane * p.T + j;
    }
    const uint64_t vm = ballot(row >= 0);
    const int nv = popc64(vm);
    if (row >= 0) cs_lds[wv][popc64(vm & lanemask_lt())] = (int)row;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int cs = lane < nv ? cs_lds[wv][lane] : 0;

    const int c = seg * kWave + lane;
    const bool active = c < p.H / 8;
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
    if (active && p.local != nullptr) add8(acc, reinterpret_cast<const u32x4*>(p.local + (int64_t)t * p.H)[c]);
    gather_all<false>(acc, reinterpret_cast<const u32x4*>(p.partials) + (active ? c : 0), p.H / 8, cs, 0.0f, nv,
                      p.stream_min);
    if (!active) return;
    if (p.bias != nullptr) add8(acc, reinterpret_cast<const u32x4*>(p.bias + (int64_t)t * p.H)[c]);
    st_nt(reinterpret_cast<u32x4*>(p.out + (int64_t)t * p.H) + c, pack8(acc));
}

}  // namespace

hipError_t launch_combine_reduce(const Handle& h, const ReduceArgs& a, hipStream_t stream) {
    if (h.T == 0) return hipSuccess;
    ReduceParams p;
    p.partials = static_cast<const uint16_t*>(a.partials);
    p.local = static_cast<const uint16_t*>(a.local);
    p.bias = static_cast<const uint16_t*>(a.bias);
    p.out = static_cast<uint16_t*>(a.out);
    p.send_slot = h.R > 1 ? h.ws.send_slot : nullptr;
    p.T = h.T;
    p.H = a.hidden;
    p.R = h.R;
    p.rank = h.rank;
    p.nseg = (a.hidden / 8 + kWave - 1) / kWave;
    p.nitems = (int64_t)h.T * p.nseg;
    p.stream_min = p.nitems >= kStreamMinWaves ? kReduceStreamRows : INT_MAX;
    const unsigned nblocks = (unsigned)((p.nitems + kWavesPerBlock - 1) / kWavesPerBlock);
    hipLaunchKernelGGL(k_combine_reduce, dim3(nblocks), dim3(kBlock), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_combine(const Handle& h, const CombineArgs& a, hipStream_t stream) {
    if (h.T == 0) return hipSuccess;
    Params p;
    p.y = static_cast<const uint16_t*>(a.y);
    p.w = a.topk_weights;
    p.bias = static_cast<const uint16_t*>(a.bias);
    p.out = static_cast<uint16_t*>(a.out);
    p.T = h.T;
    p.H = a.hidden;
    if (a.tokens) {               // one row per token: its row among this rank's tokens, unit weight
        p.slot = h.ws.send_slot + h.rank;
        p.stride = h.R;
        p.K = 1;
        p.w = nullptr;
    } else {
        p.slot = h.ws.slot;
        p.stride = h.K;
        p.K = h.K;
    }
    p.nseg = (a.hidden / 8 + kWave - 1) / kWave;
    p.nitems = (int64_t)h.T * p.nseg;
    p.stream_min = p.nitems >= kStreamMinWaves ? kCombineStreamRows : INT_MAX;
    const unsigned nblocks = (unsigned)((p.nitems + kWavesPerBlock - 1) / kWavesPerBlock);
    hipLaunchKernelGGL(k_combine, dim3(nblocks), dim3(kBlock), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ep
