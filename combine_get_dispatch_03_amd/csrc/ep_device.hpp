// ep_device.hpp -- wave64 and number-format helpers for the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ep {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ int popc64(uint64_t m) { return __builtin_popcountll(m); }

__device__ __forceinline__ int readlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

__device__ __forceinline__ float readlane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Lanes whose key equals this lane's key, among lanes with `active` set.  One ballot per key bit:
// wave64 has no match-any instruction, so peers are the lanes that agree on every bit.
__device__ __forceinline__ uint64_t match_peers(int key, bool active, int nbits) {
    uint64_t peers = ballot(active);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t m = ballot(bit);
        peers &= bit ? m : ~m;
    }
    return peers;
}

// Inclusive prefix sum over the 64 lanes.  Within each 16-lane row: four DPP row shifts (by 1, 2, 4, 8; lanes
// with no source read 0), each a VALU add; then rows 1..3 add the totals of the rows before them, read from
// lanes 15, 31 and 47.  No LDS round trip.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(v, 15);
    const int r1 = __builtin_amdgcn_readlane(v, 31);
    const int r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane_id() >> 4;
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// OR over the 64 lanes, the same in every lane: four DPP row shifts within each 16-lane row (lanes with no
// source read 0), then the four row results read back from lanes 15, 31, 47 and 63.
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
    int x = (int)v;
    x |= __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x |= __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x |= __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x |= __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    return (uint32_t)(__builtin_amdgcn_readlane(x, 15) | __builtin_amdgcn_readlane(x, 31) |
                      __builtin_amdgcn_readlane(x, 47) | __builtin_amdgcn_readlane(x, 63));
}

// Lane permutation within rows of 16 lanes by a DPP control (every lane has a source for the controls used here).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Max over groups of 8 consecutive lanes (lanes 8g..8g+7), in registers: swap neighbours (quad_perm 1,0,3,2),
// swap pairs (quad_perm 2,3,0,1), then each lane meets the other quad of its 8 through the half-row mirror
// (lane i <-> lane 7 - i within each 8).
__device__ __forceinline__ float group8_max(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));     // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_f<0x4E>(v));     // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_f<0x141>(v));    // row_half_mirror
    return v;
}

// bf16 pair (packed in a uint32, element 0 in the low half) -> two floats (exact).
__device__ __forceinline__ float bf16lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Four floats -> four OCP e4m3fn bytes (element 0 in the low byte), round to nearest even with
// saturation to +-448: the clamp to [-448, 448] first makes the hardware conversion (v_cvt_pk_fp8_f32,
// OCP format on gfx950) saturate instead of producing NaN; inside that range rounding is RNE.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
    d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// 16-byte vector of four 32-bit words (a native vector type, so it maps to dwordx4 loads and stores).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Reads one dword of every 64-byte line of the kernel's first `bytes` argument bytes, all issued before one wait.
// The compiler fetches argument fields on demand (it re-reads them rather than hold them in scalar registers),
// one wait each; a launch's arguments are new memory, so without this each wait on a line not yet read is a
// scalar-cache miss of its own.
template <int kBytes>
__device__ __forceinline__ void touch_kernargs() {
    typedef const __attribute__((address_space(4))) uint32_t* karg_ptr;
    const karg_ptr ka = (karg_ptr)__builtin_amdgcn_kernarg_segment_ptr();
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < (kBytes + 63) / 64; ++i) s ^= ka[16 * i];
    asm volatile("" ::"s"(s));
}

// Streaming 16-byte global accesses (non-temporal: the data is touched once).
__device__ __forceinline__ u32x4 ld_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

}  // namespace ep
