// ep_internal.hpp -- host-side internals shared by the library's translation units: the handle, the
// workspace carve-up and the kernel launchers.  Nothing here is part of the C ABI (include/ep.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "ep.h"

namespace ep {

constexpr int kLayoutTileTokens = 256;           // tokens per layout tile (one 1024-thread block)
constexpr int kMaxTopk = 32;
constexpr int kMaxExperts = 1024;
constexpr int kMaxRanks = 64;
constexpr int kMaxAlignment = 65536;
constexpr int kMaxHidden = 32768;
constexpr int kMaxRowBytes = 65536;

// Device arrays carved out of the caller's workspace.  All int32.
struct Workspace {
    int32_t* tile_hist;   // [ntiles, E + R + 1]  per tile: expert counts | token-in-rank counts | invalid
    int32_t* slot;        // [T, K]       expert-major row of each entry, -1 if not local
    int32_t* send_slot;   // [T, R]       rank of t among the tokens with an expert on r, else -1: its row in the
                          //              send window of r (r != rank) or in the token-major receive rows (r == rank)
    int32_t* cnt_local;   // [El]         routed entries of each local expert
    int32_t* psum;        // [El + 1]     aligned exclusive row starts of the local experts
    int32_t* pad_rows;    // [El * (A-1)] dense list of padding rows, expert by expert (A > 1 only)
    int32_t* pad_total;   // [1]          number of padding rows
    size_t bytes;         // total bytes used
};

// Offsets of the carve-up for the given sizes; with base == nullptr only `bytes` is meaningful.
Workspace carve_workspace(void* base, int T, int K, int E, int R, int A);

struct Handle {
    int T, K, E, R, rank, A;
    int El;        // local experts E / R
    int lo;        // first local expert rank * El
    int ntiles;    // ceil(T / kLayoutTileTokens)
    int64_t cap;   // receive capacity in rows
    const int64_t* topk_idx;
    Workspace ws;
};

// Opt `kernel` in to `bytes` of dynamic LDS (above the 64 KiB default; gfx950 has 160 KiB per CU) on the current
// device; the attribute is only ever raised, to the largest size asked for per (kernel, device); thread-safe.
hipError_t allow_dynamic_lds(const void* kernel, int bytes);

// ---- launchers (each enqueues on `stream` and returns hipGetLastError()) -----------------------------

struct LayoutOutputs {
    int32_t* num_tokens_per_rank;
    int32_t* num_tokens_per_expert;
    uint8_t* is_token_in_rank;
    int32_t* psum;
    int32_t* num_invalid;
};
hipError_t launch_layout(const Handle& h, const LayoutOutputs& out, hipStream_t stream);

struct DispatchArgs {
    enum Mode { kBf16, kFp8, kRows };
    Mode mode;
    const void* x;             // kBf16 / kFp8: bf16 [T, hidden]; kRows: [T, row_bytes] bytes
    const float* x_scales;     // kRows: [T, nscales] or nullptr
    int row_bytes;             // kRows only
    int nscales;               // kRows only
    const float* topk_weights;
    int hidden;
    bool zero_pad;
    bool expand;               // false: token-major receive rows (kBf16 / kFp8 only)
    ep_dispatch_out_t out;
};
hipError_t launch_dispatch(const Handle& h, const DispatchArgs& a, hipStream_t stream);

// Layout and dispatch of one routing table: one launch for <= 256 tokens (every block builds the layout in LDS),
// else launch_layout then launch_dispatch.  The handle's workspace ends up as launch_layout leaves it.
hipError_t launch_layout_dispatch(const Handle& h, const LayoutOutputs& lo, const DispatchArgs& a, hipStream_t stream);

struct ReduceArgs {
    const void* partials;      // bf16 [R, T, hidden]
    const void* local;         // bf16 [T, hidden] or nullptr
    const void* bias;          // bf16 [T, hidden] or nullptr
    void* out;                 // bf16 [T, hidden]
    int hidden;
};
hipError_t launch_combine_reduce(const Handle& h, const ReduceArgs& a, hipStream_t stream);

struct CombineArgs {
    const void* y;
    const float* topk_weights;
    const void* bias;
    void* out;
    int hidden;
    bool tokens;               // true: y holds the token-major rows (one per token, unit weight)
};
hipError_t launch_combine(const Handle& h, const CombineArgs& a, hipStream_t stream);

}  // namespace ep
