// ep_api.hip -- the C ABI of include/ep.h: argument validation, workspace carve-up, handle lifetime and the
// kernel launches.  Validation runs entirely on the host before anything is enqueued; nothing here
// allocates device memory or synchronises.
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <unordered_set>
#include <utility>

#include "ep_internal.hpp"

// Device scratch of ep_layout_dispatch_noalloc: the layout workspace of a caller that cannot allocate device
// memory.  One copy per GPU, for the life of the process.  In host code `scratch` names a host-side stand-in,
// not device memory: host code uses only the per-device address that hipGetSymbolAddress returns for it.
constexpr size_t kNoAllocScratchBytes = 4u << 20;   // 4 MiB
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace ep {
namespace {

thread_local char g_last_error[512] = "";

ep_status_t fail(ep_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

ep_status_t hip_fail(hipError_t e, const char* what) {
    return fail(EP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared shape checks of ep_get_layout / ep_layout_workspace_bytes / ep_recv_capacity.
const char* check_shape(int T, int K, int E, int R, int rank, int A) {
    if (T < 0) return "num_tokens must be >= 0";
    if (K < 1 || K > kMaxTopk) return "num_topk must be in [1, 32]";
    if (E < 1 || E > kMaxExperts) return "num_experts must be in [1, 1024]";
    if (R < 1 || R > kMaxRanks) return "num_ranks must be in [1, 64]";
    if (E % R != 0) return "num_experts must be a multiple of num_ranks";
    if (rank < 0 || rank >= R) return "rank must be in [0, num_ranks)";
    if (A < 1 || A > kMaxAlignment) return "expert_alignment must be in [1, 65536]";
    const int64_t cap = (int64_t)T * K + (int64_t)(E / R) * (A - 1);
    if (cap > INT32_MAX) return "receive capacity exceeds int32 rows";
    // send-window rows r * T + j are int32 in the kernels
    if ((int64_t)T * R > INT32_MAX) return "num_tokens * num_ranks exceeds int32 rows";
    return nullptr;
}

// Live handles.  A handle is looked up here before it is read, so a freed or foreign pointer is rejected without
// being dereferenced (a stale pointer that the allocator has since handed to a new handle is indistinguishable
// from that new handle).
// Both are created on first use and never destroyed, so calls made while the process exits (a binding's
// finaliser freeing its handle) still find them.
std::mutex& handles_mu() {
    static std::mutex* m = new std::mutex;
    return *m;
}
std::unordered_set<const Handle*>& live_handles() {
    static std::unordered_set<const Handle*>* s = new std::unordered_set<const Handle*>;
    return *s;
}

bool register_handle(const Handle* h) {
    std::lock_guard<std::mutex> lock(handles_mu());
    try {
        live_handles().insert(h);
    } catch (...) {
        return false;
    }
    return true;
}

// Removes h from the live set; false if it was not there.
bool unregister_handle(const Handle* h) {
    std::lock_guard<std::mutex> lock(handles_mu());
    return live_handles().erase(h) != 0;
}

// Per-device state of ep_layout_dispatch_noalloc: the device address of `scratch` (looked up once, with the
// device current) and the handle that the call returns, overwritten by each call on that device.  Host statics:
// nothing is allocated for them.
constexpr int kMaxDevices = 64;
struct NoAllocSlot {
    void* scratch = nullptr;   // device address of this device's copy of `scratch`
    bool ready = false;
    Handle handle;
};
std::mutex g_noalloc_mu;
NoAllocSlot g_noalloc[kMaxDevices];

// The slot index of a static handle, or -1.
int static_handle_index(const Handle* h) {
    for (int d = 0; d < kMaxDevices; ++d)
        if (h == &g_noalloc[d].handle) return d;
    return -1;
}

const Handle* check_handle(ep_handle_t h) {
    const Handle* hd = reinterpret_cast<const Handle*>(h);
    if (hd == nullptr) return nullptr;
    const int d = static_handle_index(hd);
    if (d >= 0) {
        std::lock_guard<std::mutex> lock(g_noalloc_mu);
        return g_noalloc[d].ready && g_noalloc[d].handle.T >= 0 ? hd : nullptr;
    }
    std::lock_guard<std::mutex> lock(handles_mu());
    return live_handles().count(hd) != 0 ? hd : nullptr;
}

}  // namespace

hipError_t allow_dynamic_lds(const void* kernel, int bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    // (kernel, device) -> largest size set; a fixed table, so that no call allocates host memory for it
    struct Entry {
        const void* kernel;
        int dev, bytes;
    };
    constexpr int kEntries = 256;
    static std::mutex mu;
    static Entry table[kEntries];
    static int used = 0;
    std::lock_guard<std::mutex> lock(mu);
    int i = 0;
    while (i < used && !(table[i].kernel == kernel && table[i].dev == dev)) ++i;
    if (i < used && table[i].bytes >= bytes) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    if (i == used && used < kEntries) table[used++] = Entry{kernel, dev, 0};
    if (i < used) table[i].bytes = bytes;   // (a full table only costs a repeated attribute call)
    return hipSuccess;
}

Workspace carve_workspace(void* base, int T, int K, int E, int R, int A) {
    const int ntiles = (T + kLayoutTileTokens - 1) / kLayoutTileTokens;
    const int El = E / R;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes, 256);
        return o;
    };
    const size_t o_hist = take(sizeof(int32_t) * (size_t)ntiles * (size_t)(E + R + 1));
    const size_t o_slot = take(sizeof(int32_t) * (size_t)T * K);
    const size_t o_send = take(sizeof(int32_t) * (size_t)T * R);
    const size_t o_cnt = take(sizeof(int32_t) * (size_t)El);
    const size_t o_psum = take(sizeof(int32_t) * (size_t)(El + 1));
    const size_t o_pad = take(sizeof(int32_t) * (size_t)El * (size_t)(A - 1));
    const size_t o_padn = take(sizeof(int32_t));
    Workspace w;
    char* b = static_cast<char*>(base);
    auto at = [&](size_t o) { return b ? reinterpret_cast<int32_t*>(b + o) : nullptr; };
    w.tile_hist = at(o_hist);
    w.slot = at(o_slot);
    w.send_slot = at(o_send);
    w.cnt_local = at(o_cnt);
    w.psum = at(o_psum);
    w.pad_rows = A > 1 ? at(o_pad) : nullptr;
    w.pad_total = at(o_padn);
    w.bytes = off;
    return w;
}

}  // namespace ep

using namespace ep;

extern "C" {

int64_t ep_recv_capacity(int num_tokens, int num_topk, int num_local_experts, int expert_alignment) {
    if (num_tokens < 0 || num_topk < 1 || num_topk > kMaxTopk || num_local_experts < 1 ||
        num_local_experts > kMaxExperts || expert_alignment < 1 || expert_alignment > kMaxAlignment)
        return -1;
    const int64_t cap = (int64_t)num_tokens * num_topk + (int64_t)num_local_experts * (expert_alignment - 1);
    return cap > INT32_MAX ? -1 : cap;
}

size_t ep_layout_workspace_bytes(int num_tokens, int num_topk, int num_experts, int num_ranks, int expert_alignment) {
    if (check_shape(num_tokens, num_topk, num_experts, num_ranks, 0, expert_alignment) != nullptr) return 0;
    return carve_workspace(nullptr, num_tokens, num_topk, num_experts, num_ranks, expert_alignment).bytes;
}

const char* ep_status_string(ep_status_t s) {
    switch (s) {
        case EP_OK: return "ok";
        case EP_ERR_INVALID_ARG: return "invalid argument";
        case EP_ERR_UNSUPPORTED: return "unsupported mode";
        case EP_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* ep_last_error(void) { return g_last_error; }

}  // extern "C"

namespace {

// Validation of ep_get_layout's arguments and the carve-up of its workspace (nothing is enqueued).
ep_status_t layout_args(const int64_t* topk_idx, int num_tokens, int num_topk, int num_experts, int num_ranks,
                        int rank, int expert_alignment, void* workspace, size_t workspace_bytes,
                        ep_handle_t* handle_out, Workspace* ws) {
    if (handle_out == nullptr) return fail(EP_ERR_INVALID_ARG, "handle_out is NULL");
    if (const char* why = check_shape(num_tokens, num_topk, num_experts, num_ranks, rank, expert_alignment))
        return fail(EP_ERR_INVALID_ARG, "%s", why);
    if (num_tokens > 0 && topk_idx == nullptr) return fail(EP_ERR_INVALID_ARG, "topk_idx is NULL");
    if (workspace == nullptr) return fail(EP_ERR_INVALID_ARG, "workspace is NULL");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(EP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    *ws = carve_workspace(workspace, num_tokens, num_topk, num_experts, num_ranks, expert_alignment);
    if (workspace_bytes < ws->bytes)
        return fail(EP_ERR_INVALID_ARG, "workspace_bytes %zu < required %zu", workspace_bytes, ws->bytes);
    return EP_OK;
}

void fill_handle(Handle* h, const int64_t* topk_idx, int num_tokens, int num_topk, int num_experts, int num_ranks,
                 int rank, int expert_alignment, const Workspace& ws) {
    h->T = num_tokens;
    h->K = num_topk;
    h->E = num_experts;
    h->R = num_ranks;
    h->rank = rank;
    h->A = expert_alignment;
    h->El = num_experts / num_ranks;
    h->lo = rank * h->El;
    h->ntiles = (num_tokens + kLayoutTileTokens - 1) / kLayoutTileTokens;
    h->cap = (int64_t)num_tokens * num_topk + (int64_t)h->El * (expert_alignment - 1);
    h->topk_idx = topk_idx;
    h->ws = ws;
}

// Validation and a new handle for ep_get_layout / ep_layout_dispatch (nothing is enqueued).
ep_status_t new_handle(const int64_t* topk_idx, int num_tokens, int num_topk, int num_experts, int num_ranks, int rank,
                       int expert_alignment, void* workspace, size_t workspace_bytes, ep_handle_t* handle_out,
                       Handle** h_out) {
    Workspace ws;
    const ep_status_t st = layout_args(topk_idx, num_tokens, num_topk, num_experts, num_ranks, rank,
                                       expert_alignment, workspace, workspace_bytes, handle_out, &ws);
    if (st != EP_OK) return st;
    Handle* h = new (std::nothrow) Handle;
    if (h == nullptr) return fail(EP_ERR_INVALID_ARG, "out of host memory for the handle");
    fill_handle(h, topk_idx, num_tokens, num_topk, num_experts, num_ranks, rank, expert_alignment, ws);
    *h_out = h;
    return EP_OK;
}

void drop_handle(Handle* h) {
    delete h;
}

// Makes a fully built handle visible to the other calls.
ep_status_t publish_handle(Handle* h, ep_handle_t* handle_out) {
    if (!register_handle(h)) {
        drop_handle(h);
        return fail(EP_ERR_INVALID_ARG, "out of host memory for the handle registry");
    }
    *handle_out = reinterpret_cast<ep_handle_t>(h);
    return EP_OK;
}

// Validation of ep_dispatch's arguments against a handle, and its launch arguments (nothing is enqueued).
ep_status_t dispatch_args(const Handle* h, const void* x, int hidden, const float* topk_weights, ep_dtype_t recv_dtype,
                          int do_expand, int do_zero_padding, const ep_dispatch_out_t* out, DispatchArgs* a) {
    if (recv_dtype != EP_DTYPE_BF16 && recv_dtype != EP_DTYPE_FP8_E4M3)
        return fail(EP_ERR_INVALID_ARG, "recv_dtype must be EP_DTYPE_BF16 or EP_DTYPE_FP8_E4M3");
    const bool fp8 = recv_dtype == EP_DTYPE_FP8_E4M3;
    if (hidden < 8 || hidden > kMaxHidden || hidden % 8 != 0)
        return fail(EP_ERR_INVALID_ARG, "hidden must be a multiple of 8 in [8, 32768]");
    if (fp8 && hidden % 128 != 0) return fail(EP_ERR_INVALID_ARG, "FP8 dispatch needs hidden % 128 == 0");
    if (out == nullptr) return fail(EP_ERR_INVALID_ARG, "out is NULL");
    if (h->T > 0) {
        if (x == nullptr || !aligned16(x)) return fail(EP_ERR_INVALID_ARG, "x must be non-NULL and 16-byte aligned");
        if (out->recv_x == nullptr || !aligned16(out->recv_x))
            return fail(EP_ERR_INVALID_ARG, "recv_x must be non-NULL and 16-byte aligned");
        const int64_t need = do_expand ? h->cap : (int64_t)h->T;
        if (out->recv_capacity < need)
            return fail(EP_ERR_INVALID_ARG, "recv_capacity %lld < required %lld", (long long)out->recv_capacity,
                        (long long)need);
        if (fp8 && out->recv_x_scales == nullptr) return fail(EP_ERR_INVALID_ARG, "FP8 needs recv_x_scales");
        if (h->R > 1) {
            if (out->send_x == nullptr || !aligned16(out->send_x))
                return fail(EP_ERR_INVALID_ARG, "num_ranks > 1 needs a 16-byte aligned send_x");
            if (fp8 && out->send_x_scales == nullptr)
                return fail(EP_ERR_INVALID_ARG, "num_ranks > 1 with FP8 needs send_x_scales");
        }
    }
    a->mode = fp8 ? DispatchArgs::kFp8 : DispatchArgs::kBf16;
    a->x = x;
    a->x_scales = nullptr;
    a->row_bytes = 0;
    a->nscales = 0;
    a->topk_weights = topk_weights;
    a->hidden = hidden;
    a->zero_pad = do_zero_padding != 0;
    a->expand = do_expand != 0;
    a->out = *out;
    if (!fp8) a->out.recv_x_scales = nullptr;
    if (a->expand) a->out.recv_topk_idx = nullptr;
    return EP_OK;
}

}  // namespace

extern "C" {

ep_status_t ep_get_layout(const int64_t* topk_idx, int num_tokens, int num_topk, int num_experts, int num_ranks,
                          int rank, int expert_alignment, void* workspace, size_t workspace_bytes,
                          int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                          int32_t* psum_num_recv_tokens_per_expert, int32_t* num_invalid_topk,
                          ep_handle_t* handle_out, void* stream) {
    g_last_error[0] = '\0';
    Handle* h = nullptr;
    const ep_status_t st = new_handle(topk_idx, num_tokens, num_topk, num_experts, num_ranks, rank, expert_alignment,
                                      workspace, workspace_bytes, handle_out, &h);
    if (st != EP_OK) return st;
    const LayoutOutputs out{num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank,
                            psum_num_recv_tokens_per_expert, num_invalid_topk};
    const hipError_t err = launch_layout(*h, out, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) {
        drop_handle(h);
        return hip_fail(err, "layout launch");
    }
    return publish_handle(h, handle_out);
}

ep_status_t ep_dispatch(ep_handle_t handle, const void* x, int hidden, const float* topk_weights,
                        ep_dtype_t recv_dtype, int do_expand, int do_zero_padding, const ep_dispatch_out_t* out,
                        void* stream) {
    g_last_error[0] = '\0';
    const Handle* h = check_handle(handle);
    if (h == nullptr) return fail(EP_ERR_INVALID_ARG, "invalid handle");
    DispatchArgs a;
    const ep_status_t st = dispatch_args(h, x, hidden, topk_weights, recv_dtype, do_expand, do_zero_padding, out, &a);
    if (st != EP_OK) return st;
    const hipError_t err = launch_dispatch(*h, a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "dispatch launch");
    return EP_OK;
}

ep_status_t ep_layout_dispatch(const int64_t* topk_idx, int num_tokens, int num_topk, int num_experts, int num_ranks,
                               int rank, int expert_alignment, void* workspace, size_t workspace_bytes,
                               int32_t* num_tokens_per_rank, int32_t* num_tokens_per_expert,
                               uint8_t* is_token_in_rank, int32_t* psum_num_recv_tokens_per_expert,
                               int32_t* num_invalid_topk, const void* x, int hidden, const float* topk_weights,
                               ep_dtype_t recv_dtype, int do_expand, int do_zero_padding,
                               const ep_dispatch_out_t* out, ep_handle_t* handle_out, void* stream) {
    g_last_error[0] = '\0';
    Handle* h = nullptr;
    ep_status_t st = new_handle(topk_idx, num_tokens, num_topk, num_experts, num_ranks, rank, expert_alignment,
                                workspace, workspace_bytes, handle_out, &h);
    if (st != EP_OK) return st;
    DispatchArgs a;
    st = dispatch_args(h, x, hidden, topk_weights, recv_dtype, do_expand, do_zero_padding, out, &a);
    if (st != EP_OK) {
        drop_handle(h);
        return st;
    }
    const LayoutOutputs lo{num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank,
                           psum_num_recv_tokens_per_expert, num_invalid_topk};
    const hipError_t err = launch_layout_dispatch(*h, lo, a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) {
        drop_handle(h);
        return hip_fail(err, "layout_dispatch launch");
    }
    return publish_handle(h, handle_out);
}

ep_status_t ep_layout_dispatch_noalloc(const int64_t* topk_idx, int num_tokens, int num_topk, int num_experts,
                                       int num_ranks, int rank, int expert_alignment, int32_t* num_tokens_per_rank,
                                       int32_t* num_tokens_per_expert, uint8_t* is_token_in_rank,
                                       int32_t* psum_num_recv_tokens_per_expert, int32_t* num_invalid_topk,
                                       const void* x, int hidden, const float* topk_weights, ep_dtype_t recv_dtype,
                                       int do_expand, int do_zero_padding, const ep_dispatch_out_t* out,
                                       ep_handle_t* handle_out, void* stream) {
    g_last_error[0] = '\0';
    if (handle_out == nullptr) return fail(EP_ERR_INVALID_ARG, "handle_out is NULL");
    if (const char* why = check_shape(num_tokens, num_topk, num_experts, num_ranks, rank, expert_alignment))
        return fail(EP_ERR_INVALID_ARG, "%s", why);
    const size_t need = carve_workspace(nullptr, num_tokens, num_topk, num_experts, num_ranks, expert_alignment).bytes;
    if (need > kNoAllocScratchBytes)
        return fail(EP_ERR_INVALID_ARG,
                    "ep_layout_dispatch_noalloc: these sizes need %zu bytes of layout workspace, more than its "
                    "static scratch of %zu bytes; call ep_layout_dispatch with a workspace instead",
                    need, kNoAllocScratchBytes);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(EP_ERR_INVALID_ARG, "ep_layout_dispatch_noalloc: device %d beyond the first %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    NoAllocSlot& slot = g_noalloc[dev];
    if (!slot.ready) {   // set-up, once per device, with that device current
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255u) != 0)
            return fail(EP_ERR_HIP, "hipGetSymbolAddress(scratch) returned an unusable address");
        slot.scratch = ptr;
        slot.handle.T = -1;   // no layout yet
        slot.ready = true;
    }
    Workspace ws;
    ep_status_t st = layout_args(topk_idx, num_tokens, num_topk, num_experts, num_ranks, rank, expert_alignment,
                                 slot.scratch, kNoAllocScratchBytes, handle_out, &ws);
    if (st != EP_OK) return st;
    Handle h;
    fill_handle(&h, topk_idx, num_tokens, num_topk, num_experts, num_ranks, rank, expert_alignment, ws);
    DispatchArgs a;
    st = dispatch_args(&h, x, hidden, topk_weights, recv_dtype, do_expand, do_zero_padding, out, &a);
    if (st != EP_OK) return st;
    const LayoutOutputs lo{num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank,
                           psum_num_recv_tokens_per_expert, num_invalid_topk};
    e = launch_layout_dispatch(h, lo, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "layout_dispatch_noalloc launch");
    slot.handle = h;
    *handle_out = reinterpret_cast<ep_handle_t>(&slot.handle);
    return EP_OK;
}

ep_status_t ep_dispatch_rows(ep_handle_t handle, const void* rows, int row_bytes, const float* row_scales,
                             int num_scales, const float* topk_weights, int do_zero_padding,
                             const ep_dispatch_out_t* out, void* stream) {
    g_last_error[0] = '\0';
    const Handle* h = check_handle(handle);
    if (h == nullptr) return fail(EP_ERR_INVALID_ARG, "invalid handle");
    if (row_bytes < 16 || row_bytes > kMaxRowBytes || row_bytes % 16 != 0)
        return fail(EP_ERR_INVALID_ARG, "row_bytes must be a multiple of 16 in [16, 65536]");
    if (num_scales < 0 || num_scales > kMaxHidden / 128)
        return fail(EP_ERR_INVALID_ARG, "num_scales must be in [0, 256]");
    if (out == nullptr) return fail(EP_ERR_INVALID_ARG, "out is NULL");
    if (h->T > 0) {
        if (rows == nullptr || !aligned16(rows)) return fail(EP_ERR_INVALID_ARG, "rows must be non-NULL and 16-byte aligned");
        if (num_scales > 0 && row_scales == nullptr) return fail(EP_ERR_INVALID_ARG, "num_scales > 0 needs row_scales");
        if (out->recv_x == nullptr || !aligned16(out->recv_x))
            return fail(EP_ERR_INVALID_ARG, "recv_x must be non-NULL and 16-byte aligned");
        if (out->recv_capacity < h->cap)
            return fail(EP_ERR_INVALID_ARG, "recv_capacity %lld < required %lld", (long long)out->recv_capacity,
                        (long long)h->cap);
        if (num_scales > 0 && out->recv_x_scales == nullptr)
            return fail(EP_ERR_INVALID_ARG, "num_scales > 0 needs recv_x_scales");
    }
    DispatchArgs a;
    a.mode = DispatchArgs::kRows;
    a.x = rows;
    a.x_scales = num_scales > 0 ? row_scales : nullptr;
    a.row_bytes = row_bytes;
    a.nscales = num_scales;
    a.topk_weights = topk_weights;
    a.hidden = 0;
    a.zero_pad = do_zero_padding != 0;
    a.expand = true;
    a.out = *out;
    a.out.recv_topk_idx = nullptr;
    if (num_scales == 0) a.out.recv_x_scales = nullptr;
    const hipError_t err = launch_dispatch(*h, a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "dispatch_rows launch");
    return EP_OK;
}

ep_status_t ep_combine_reduce(ep_handle_t handle, const void* partials, int hidden, const void* local,
                              const void* bias, void* out, void* stream) {
    g_last_error[0] = '\0';
    const Handle* h = check_handle(handle);
    if (h == nullptr) return fail(EP_ERR_INVALID_ARG, "invalid handle");
    if (hidden < 8 || hidden > kMaxHidden || hidden % 8 != 0)
        return fail(EP_ERR_INVALID_ARG, "hidden must be a multiple of 8 in [8, 32768]");
    if (h->T > 0) {
        if (h->R > 1 && (partials == nullptr || !aligned16(partials)))
            return fail(EP_ERR_INVALID_ARG, "partials must be non-NULL and 16-byte aligned");
        if (out == nullptr || !aligned16(out)) return fail(EP_ERR_INVALID_ARG, "out must be non-NULL and 16-byte aligned");
        if (local != nullptr && !aligned16(local)) return fail(EP_ERR_INVALID_ARG, "local must be 16-byte aligned");
        if (bias != nullptr && !aligned16(bias)) return fail(EP_ERR_INVALID_ARG, "bias must be 16-byte aligned");
    }
    ReduceArgs a;
    a.partials = partials;
    a.local = local;
    a.bias = bias;
    a.out = out;
    a.hidden = hidden;
    const hipError_t err = launch_combine_reduce(*h, a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "combine_reduce launch");
    return EP_OK;
}

ep_status_t ep_combine(ep_handle_t handle, const void* y, int hidden, int64_t y_rows, const float* topk_weights,
                       const void* bias, void* out, void* stream) {
    g_last_error[0] = '\0';
    const Handle* h = check_handle(handle);
    if (h == nullptr) return fail(EP_ERR_INVALID_ARG, "invalid handle");
    if (hidden < 8 || hidden > kMaxHidden || hidden % 8 != 0)
        return fail(EP_ERR_INVALID_ARG, "hidden must be a multiple of 8 in [8, 32768]");
    if (h->T > 0) {
        if (y == nullptr || !aligned16(y)) return fail(EP_ERR_INVALID_ARG, "y must be non-NULL and 16-byte aligned");
        if (y_rows < h->cap)
            return fail(EP_ERR_INVALID_ARG, "y_rows %lld < required %lld", (long long)y_rows, (long long)h->cap);
        if (out == nullptr || !aligned16(out)) return fail(EP_ERR_INVALID_ARG, "out must be non-NULL and 16-byte aligned");
        if (bias != nullptr && !aligned16(bias)) return fail(EP_ERR_INVALID_ARG, "bias must be 16-byte aligned");
    }
    CombineArgs a;
    a.y = y;
    a.topk_weights = topk_weights;
    a.bias = bias;
    a.out = out;
    a.hidden = hidden;
    a.tokens = false;
    const hipError_t err = launch_combine(*h, a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "combine launch");
    return EP_OK;
}

ep_status_t ep_combine_tokens(ep_handle_t handle, const void* y, int hidden, int64_t y_rows, const void* bias,
                              void* out, void* stream) {
    g_last_error[0] = '\0';
    const Handle* h = check_handle(handle);
    if (h == nullptr) return fail(EP_ERR_INVALID_ARG, "invalid handle");
    if (hidden < 8 || hidden > kMaxHidden || hidden % 8 != 0)
        return fail(EP_ERR_INVALID_ARG, "hidden must be a multiple of 8 in [8, 32768]");
    if (h->T > 0) {
        if (y == nullptr || !aligned16(y)) return fail(EP_ERR_INVALID_ARG, "y must be non-NULL and 16-byte aligned");
        if (y_rows < h->T)
            return fail(EP_ERR_INVALID_ARG, "y_rows %lld < num_tokens %d", (long long)y_rows, h->T);
        if (out == nullptr || !aligned16(out)) return fail(EP_ERR_INVALID_ARG, "out must be non-NULL and 16-byte aligned");
        if (bias != nullptr && !aligned16(bias)) return fail(EP_ERR_INVALID_ARG, "bias must be 16-byte aligned");
    }
    CombineArgs a;
    a.y = y;
    a.topk_weights = nullptr;
    a.bias = bias;
    a.out = out;
    a.hidden = hidden;
    a.tokens = true;
    const hipError_t err = launch_combine(*h, a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "combine_tokens launch");
    return EP_OK;
}

ep_status_t ep_handle_free(ep_handle_t handle) {
    Handle* h = reinterpret_cast<Handle*>(handle);
    if (h == nullptr) return EP_OK;
    if (static_handle_index(h) >= 0) return EP_OK;   // a device's ep_layout_dispatch_noalloc handle: never freed
    if (!unregister_handle(h)) return fail(EP_ERR_INVALID_ARG, "invalid handle (not live: freed twice or never created)");
    drop_handle(h);
    return EP_OK;
}

}  // extern "C"
