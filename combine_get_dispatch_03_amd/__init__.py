"""Python binding of libep_mi355x.so (include/ep.h): MoE expert-parallel layout, dispatch and combine on one
MI355X (gfx950) GPU.

The functions keep the C names (ep_get_layout, ep_dispatch, ep_layout_dispatch, ep_combine, ep_combine_tokens,
ep_dispatch_rows, ep_combine_reduce, ep_handle_free, ep_recv_capacity, ep_layout_workspace_bytes).  They only marshal arguments: tensors become device pointers, the stream is
torch's current HIP stream, and output tensors are allocated by torch when the caller does not pass them.
Every step of the path runs in the HIP kernels of the library; there is no other implementation, and if
the library is not built or cannot be loaded the import of this binding fails.

    h, lay = ep_get_layout(topk_idx, num_experts=256, expert_alignment=128)
    d = ep_dispatch(h, x, topk_weights, fp8=True, do_zero_padding=True)
    out = ep_combine(h, y, topk_weights, bias=None)
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libep_mi355x.so")

EP_OK = 0
EP_DTYPE_BF16 = 0
EP_DTYPE_FP8_E4M3 = 1


class EPError(RuntimeError):
    pass


class _DispatchOut(ctypes.Structure):
    _fields_ = [
        ("recv_x", ctypes.c_void_p), ("recv_x_scales", ctypes.c_void_p), ("recv_src_idx", ctypes.c_void_p),
        ("recv_topk_weights", ctypes.c_void_p), ("recv_topk_idx", ctypes.c_void_p),
        ("recv_capacity", ctypes.c_int64),
        ("send_x", ctypes.c_void_p), ("send_x_scales", ctypes.c_void_p), ("send_src_idx", ctypes.c_void_p),
        ("send_topk_idx", ctypes.c_void_p), ("send_topk_weights", ctypes.c_void_p),
    ]


def _load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libep_mi355x.so is not built: run `python -m combine_get_dispatch_03_amd.build` "
                          "(or __graft_entry__.build())")
    # torch is imported first, so the HIP runtime the library links (soname libamdhip64.so.7) resolves to the
    # one torch already loaded: streams and device pointers then belong to the same runtime.
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.ep_recv_capacity.restype = I64
    lib.ep_recv_capacity.argtypes = [I, I, I, I]
    lib.ep_layout_workspace_bytes.restype = SZ
    lib.ep_layout_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.ep_status_string.restype = ctypes.c_char_p
    lib.ep_status_string.argtypes = [I]
    lib.ep_last_error.restype = ctypes.c_char_p
    lib.ep_last_error.argtypes = []
    lib.ep_get_layout.restype = I
    lib.ep_get_layout.argtypes = [P, I, I, I, I, I, I, P, SZ, P, P, P, P, P, ctypes.POINTER(P), P]
    lib.ep_dispatch.restype = I
    lib.ep_dispatch.argtypes = [P, P, I, P, I, I, I, ctypes.POINTER(_DispatchOut), P]
    lib.ep_combine.restype = I
    lib.ep_combine.argtypes = [P, P, I, I64, P, P, P, P]
    lib.ep_handle_free.restype = I
    lib.ep_handle_free.argtypes = [P]
    lib.ep_dispatch_rows.restype = I
    lib.ep_dispatch_rows.argtypes = [P, P, I, P, I, P, I, ctypes.POINTER(_DispatchOut), P]
    lib.ep_combine_reduce.restype = I
    lib.ep_combine_reduce.argtypes = [P, P, I, P, P, P, P]
    lib.ep_combine_tokens.restype = I
    lib.ep_combine_tokens.argtypes = [P, P, I, I64, P, P, P]
    lib.ep_layout_dispatch_noalloc.restype = I
    lib.ep_layout_dispatch_noalloc.argtypes = [P, I, I, I, I, I, I, P, P, P, P, P, P, I, P, I, I, I,
                                               ctypes.POINTER(_DispatchOut), ctypes.POINTER(P), P]
    lib.ep_layout_dispatch.restype = I
    lib.ep_layout_dispatch.argtypes = [P, I, I, I, I, I, I, P, SZ, P, P, P, P, P, P, I, P, I, I, I,
                                       ctypes.POINTER(_DispatchOut), ctypes.POINTER(P), P]
    return lib


_lib = _load_library()


def hip_runtimes_loaded() -> list[str]:
    """Paths of the libamdhip64 copies mapped into this process (exactly one is expected)."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(line.split()[-1])
    return sorted(paths)


def _check(status: int, what: str):
    if status != EP_OK:
        msg = _lib.ep_last_error().decode(errors="replace")
        raise EPError("%s failed: %s (%s)" % (what, _lib.ep_status_string(status).decode(), msg))


def _ptr(t):
    # a plain int: the c_void_p argument types convert it (cheaper than building a c_void_p per pointer)
    return None if t is None else t.data_ptr()


# torch's current raw stream without building a Stream object (~0.2 us instead of ~2.5 us per call)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_cur_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream):
    """HIP stream handle: the given torch stream's, else torch's current stream on the current device."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None and _cur_device is not None:
        return _raw_stream(_cur_device())
    return torch.cuda.current_stream().cuda_stream


def _on_stream(stream, fn, *args, **kw):
    """Run an allocating helper with `stream` current, so that the tensors it makes belong to the stream the
    call's kernels write them on: torch's caching allocator hands a freed block to later work of the block's
    own stream only, which then is ordered after those kernels.  stream=None: torch's current stream, where
    the kernels run anyway."""
    if stream is None:
        return fn(*args, **kw)
    with torch.cuda.stream(stream):
        return fn(*args, **kw)


def _need(t, dtype, name, device=None, shape=None):
    """t must be a contiguous tensor of `dtype` and `shape` (when given) on `device` (when given; else on a GPU).
    The shape is checked before the placement, so the shape rules can be exercised without a GPU."""
    # one expression for the common (valid) case; the checks below only name what is wrong
    if (type(t) is torch.Tensor and t.dtype is dtype and (shape is None or t.shape == shape)
            and (t.device == device if device is not None else t.is_cuda) and t.is_contiguous()):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if device is not None:
        if t.device != device:
            raise ValueError("%s must be on %s, got %s" % (name, device, t.device))
    elif not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _opt(out, key, dtype, shape, device):
    """An optional output: absent/None, or exactly dtype/shape on device."""
    t = out.get(key)
    if t is not None:
        _need(t, dtype, key, device, shape)


def check_layout_outputs(outputs, T, E, R, device):
    """Caller-supplied layout outputs (any entry may be None): the sizes the library writes."""
    El = E // R
    _opt(outputs, "num_tokens_per_rank", torch.int32, (R,), device)
    _opt(outputs, "num_tokens_per_expert", torch.int32, (E,), device)
    _opt(outputs, "is_token_in_rank", torch.uint8, (T, R), device)
    _opt(outputs, "psum_num_recv_tokens_per_expert", torch.int32, (El + 1,), device)
    _opt(outputs, "num_invalid_topk", torch.int32, (1,), device)


def check_workspace(workspace, device):
    """A caller's workspace: one contiguous uint8 buffer on the device (its length is checked by the library)."""
    _need(workspace, torch.uint8, "workspace", device)
    if workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")


def check_dispatch_outputs(out, T, K, R, hidden, fp8, do_expand, device):
    """Every dispatch output the library will write, against the sizes it writes: recv_x [cap, hidden] (e4m3
    bytes or bf16) with every other recv array on the same cap rows, the send windows [R, T, ...].  Returns cap
    (the recv_capacity passed to the library, which checks it against the layout's bound)."""
    if not isinstance(out, dict) or out.get("recv_x") is None:
        raise ValueError("out must be a dict holding recv_x")
    rx = out["recv_x"]
    xdt = torch.uint8 if fp8 else torch.bfloat16
    if not isinstance(rx, torch.Tensor) or rx.dim() != 2:
        raise ValueError("recv_x must be a 2-D tensor [rows, hidden]")
    cap = rx.shape[0]
    _need(rx, xdt, "recv_x", device, (cap, hidden))
    if fp8:
        if out.get("recv_x_scales") is None:
            raise ValueError("FP8 dispatch needs recv_x_scales")
        _need(out["recv_x_scales"], torch.float32, "recv_x_scales", device, (cap, hidden // 128))
    _opt(out, "recv_src_idx", torch.int32, (cap,), device)
    _opt(out, "recv_topk_weights", torch.float32, (cap,) if do_expand else (T, K), device)
    if not do_expand:
        _opt(out, "recv_topk_idx", torch.int64, (T, K), device)
    if R > 1:
        if out.get("send_x") is None:
            raise ValueError("num_ranks > 1 needs send_x")
        _need(out["send_x"], xdt, "send_x", device, (R, T, hidden))
        if fp8:
            if out.get("send_x_scales") is None:
                raise ValueError("num_ranks > 1 with FP8 needs send_x_scales")
            _need(out["send_x_scales"], torch.float32, "send_x_scales", device, (R, T, hidden // 128))
        _opt(out, "send_src_idx", torch.int32, (R, T), device)
        _opt(out, "send_topk_idx", torch.int64, (R, T, K), device)
        _opt(out, "send_topk_weights", torch.float32, (R, T, K), device)
    return cap


def check_rows_outputs(out, row_dtype, row_elems, G, device):
    """Outputs of ep_dispatch_rows: recv_x [cap, row_elems] of the rows' dtype, scales [cap, G] when G > 0, and
    the optional per-row metadata on the same cap rows.  Returns cap."""
    if not isinstance(out, dict) or out.get("recv_x") is None:
        raise ValueError("out must be a dict holding recv_x")
    rx = out["recv_x"]
    if not isinstance(rx, torch.Tensor) or rx.dim() != 2:
        raise ValueError("recv_x must be a 2-D tensor [rows, row_elements]")
    cap = rx.shape[0]
    _need(rx, row_dtype, "recv_x", device, (cap, row_elems))
    if G > 0:
        if out.get("recv_x_scales") is None:
            raise ValueError("rows with scales need recv_x_scales")
        _need(out["recv_x_scales"], torch.float32, "recv_x_scales", device, (cap, G))
    _opt(out, "recv_src_idx", torch.int32, (cap,), device)
    _opt(out, "recv_topk_weights", torch.float32, (cap,), device)
    return cap


def ep_recv_capacity(num_tokens, num_topk, num_local_experts, expert_alignment) -> int:
    return int(_lib.ep_recv_capacity(num_tokens, num_topk, num_local_experts, expert_alignment))


def ep_layout_workspace_bytes(num_tokens, num_topk, num_experts, num_ranks=1, expert_alignment=1) -> int:
    return int(_lib.ep_layout_workspace_bytes(num_tokens, num_topk, num_experts, num_ranks, expert_alignment))


class Handle:
    """Owns an ep_handle_t plus references to the tensors it points into (topk_idx and the workspace)."""

    def __init__(self, ptr, topk_idx, workspace, num_tokens, num_topk, num_experts, num_ranks, rank,
                 expert_alignment):
        self._ptr = ptr
        self.topk_idx = topk_idx
        self.workspace = workspace
        self.num_tokens, self.num_topk, self.num_experts = num_tokens, num_topk, num_experts
        self.num_ranks, self.rank, self.expert_alignment = num_ranks, rank, expert_alignment
        self.num_local_experts = num_experts // num_ranks
        self._cap = None

    @property
    def recv_capacity(self):
        """Rows of the expert-major receive buffers (ep_recv_capacity of the handle's sizes)."""
        if self._cap is None:
            self._cap = ep_recv_capacity(self.num_tokens, self.num_topk, self.num_local_experts,
                                         self.expert_alignment)
        return self._cap

    @property
    def ptr(self):
        if self._ptr is None:
            raise EPError("handle already freed")
        return self._ptr

    def free(self):
        if self._ptr is not None and _lib is not None:
            _check(_lib.ep_handle_free(self._ptr), "ep_handle_free")
        self._ptr = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def _layout_prep(topk_idx, num_experts, num_ranks, expert_alignment, workspace, outputs):
    _need(topk_idx, torch.int64, "topk_idx")
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [num_tokens, num_topk]")
    T, K = topk_idx.shape
    dev = topk_idx.device
    if num_ranks < 1 or num_experts < 1 or num_experts % num_ranks != 0:
        raise ValueError("num_experts must be a positive multiple of num_ranks")
    if workspace is not None:   # its length is checked by the library call itself
        check_workspace(workspace, dev)
    else:
        nbytes = ep_layout_workspace_bytes(T, K, num_experts, num_ranks, expert_alignment)
        if nbytes == 0:
            raise EPError("ep_layout_workspace_bytes rejected the sizes (T=%d K=%d E=%d R=%d A=%d)"
                          % (T, K, num_experts, num_ranks, expert_alignment))
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    El = num_experts // num_ranks
    if outputs is not None:
        check_layout_outputs(outputs, T, num_experts, num_ranks, dev)
    else:
        outputs = dict(
            num_tokens_per_rank=torch.empty(num_ranks, dtype=torch.int32, device=dev),
            num_tokens_per_expert=torch.empty(num_experts, dtype=torch.int32, device=dev),
            is_token_in_rank=torch.empty((T, num_ranks), dtype=torch.uint8, device=dev),
            psum_num_recv_tokens_per_expert=torch.empty(El + 1, dtype=torch.int32, device=dev),
            num_invalid_topk=torch.empty(1, dtype=torch.int32, device=dev))
    return T, K, workspace, outputs


_LAYOUT_KEYS = ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank",
                "psum_num_recv_tokens_per_expert", "num_invalid_topk")


def _layout_ptrs(outputs):
    g = outputs.get
    return tuple(None if t is None else t.data_ptr() for t in (g(k) for k in _LAYOUT_KEYS))


def ep_get_layout(topk_idx, num_experts, num_ranks=1, rank=0, expert_alignment=1, workspace=None, outputs=None,
                  stream=None):
    """Layout of `topk_idx` (int64 [T, K] on the GPU).  Returns (Handle, dict) with the device outputs
    num_tokens_per_rank, num_tokens_per_expert, is_token_in_rank, psum_num_recv_tokens_per_expert and
    num_invalid_topk.  `outputs` may supply any of those tensors (or None entries to skip them)."""
    T, K, workspace, outputs = _on_stream(stream, _layout_prep, topk_idx, num_experts, num_ranks, expert_alignment,
                                          workspace, outputs)
    h = ctypes.c_void_p()
    _check(_lib.ep_get_layout(
        _ptr(topk_idx), T, K, num_experts, num_ranks, rank, expert_alignment, _ptr(workspace), workspace.numel(),
        *_layout_ptrs(outputs), ctypes.byref(h), _stream(stream)), "ep_get_layout")
    return Handle(h, topk_idx, workspace, T, K, num_experts, num_ranks, rank, expert_alignment), outputs


def alloc_dispatch_outputs(handle: Handle, hidden: int, fp8: bool, want_meta=True, want_send_meta=True,
                           device=None, recv_capacity=None, do_expand=True):
    """Allocate (uninitialised) dispatch output tensors for `handle` (token-major shapes when do_expand is
    False: num_tokens rows, recv_topk_weights and recv_topk_idx [T, K])."""
    dev = device if device is not None else handle.topk_idx.device
    T, K, R = handle.num_tokens, handle.num_topk, handle.num_ranks
    if recv_capacity is not None:
        cap = recv_capacity
    else:
        cap = handle.recv_capacity if do_expand else T
    G = hidden // 128
    o = {}
    if fp8:
        o["recv_x"] = torch.empty((cap, hidden), dtype=torch.uint8, device=dev)
        o["recv_x_scales"] = torch.empty((cap, G), dtype=torch.float32, device=dev)
    else:
        o["recv_x"] = torch.empty((cap, hidden), dtype=torch.bfloat16, device=dev)
        o["recv_x_scales"] = None
    o["recv_src_idx"] = torch.empty(cap, dtype=torch.int32, device=dev) if want_meta else None
    wshape = cap if do_expand else (T, K)
    o["recv_topk_weights"] = torch.empty(wshape, dtype=torch.float32, device=dev) if want_meta else None
    o["recv_topk_idx"] = torch.empty((T, K), dtype=torch.int64, device=dev) if (want_meta and not do_expand) else None
    if R > 1:
        o["send_x"] = torch.empty((R, T, hidden), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
        o["send_x_scales"] = torch.empty((R, T, G), dtype=torch.float32, device=dev) if fp8 else None
        o["send_src_idx"] = torch.empty((R, T), dtype=torch.int32, device=dev) if want_send_meta else None
        o["send_topk_idx"] = torch.empty((R, T, K), dtype=torch.int64, device=dev) if want_send_meta else None
        o["send_topk_weights"] = torch.empty((R, T, K), dtype=torch.float32, device=dev) if want_send_meta else None
    else:
        for k in ("send_x", "send_x_scales", "send_src_idx", "send_topk_idx", "send_topk_weights"):
            o[k] = None
    return o


_RECV_KEYS = ("recv_x", "recv_x_scales", "recv_src_idx", "recv_topk_weights", "recv_topk_idx")
_SEND_KEYS = ("send_x", "send_x_scales", "send_src_idx", "send_topk_idx", "send_topk_weights")


def _dispatch_struct(out, cap, keys=_RECV_KEYS + _SEND_KEYS):
    s = _DispatchOut()   # zeroed: absent tensors stay NULL
    for k in keys:
        t = out.get(k)
        if t is not None:
            setattr(s, k, t.data_ptr())
    s.recv_capacity = cap
    return s


def ep_dispatch(handle: Handle, x, topk_weights=None, fp8=True, do_expand=True, do_zero_padding=False, out=None,
                want_meta=True, want_send_meta=True, stream=None):
    """Dispatch `x` (bf16 [T, H]) through `handle`.  Returns the dict of output tensors (allocated here unless
    `out` is given; rows that the call does not write keep whatever the tensors held)."""
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2 or x.shape[0] != handle.num_tokens:
        raise ValueError("x must be [num_tokens, hidden]")
    H = x.shape[1]
    dev = x.device
    if topk_weights is not None:
        _need(topk_weights, torch.float32, "topk_weights", dev, (handle.num_tokens, handle.num_topk))
    if out is None:
        out = _on_stream(stream, alloc_dispatch_outputs, handle, H, fp8, want_meta, want_send_meta,
                         device=dev, do_expand=do_expand)
        cap = out["recv_x"].shape[0]
    else:
        cap = check_dispatch_outputs(out, handle.num_tokens, handle.num_topk, handle.num_ranks, H, fp8,
                                     do_expand, dev)
    s = _dispatch_struct(out, cap)
    _check(_lib.ep_dispatch(handle.ptr, _ptr(x), H, _ptr(topk_weights),
                            EP_DTYPE_FP8_E4M3 if fp8 else EP_DTYPE_BF16, int(bool(do_expand)),
                            int(bool(do_zero_padding)), ctypes.byref(s), _stream(stream)), "ep_dispatch")
    return out


def ep_layout_dispatch(topk_idx, x, num_experts, num_ranks=1, rank=0, expert_alignment=1, topk_weights=None,
                       fp8=True, do_expand=True, do_zero_padding=False, out=None, workspace=None, outputs=None,
                       want_meta=True, want_send_meta=True, stream=None):
    """ep_get_layout + ep_dispatch in one call (one kernel launch for <= 256 tokens).  Returns (Handle, layout
    outputs dict, dispatch outputs dict), the same as the two calls would."""
    T, K, workspace, outputs = _on_stream(stream, _layout_prep, topk_idx, num_experts, num_ranks, expert_alignment,
                                          workspace, outputs)
    dev = topk_idx.device
    _need(x, torch.bfloat16, "x", dev)
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [num_tokens, hidden]")
    H = x.shape[1]
    if topk_weights is not None:
        _need(topk_weights, torch.float32, "topk_weights", dev, (T, K))
    if out is None:
        tmp = Handle(None, topk_idx, workspace, T, K, num_experts, num_ranks, rank, expert_alignment)
        out = _on_stream(stream, alloc_dispatch_outputs, tmp, H, fp8, want_meta, want_send_meta, device=dev,
                         do_expand=do_expand)
        cap = out["recv_x"].shape[0]
    else:
        cap = check_dispatch_outputs(out, T, K, num_ranks, H, fp8, do_expand, dev)
    s = _dispatch_struct(out, cap)
    h = ctypes.c_void_p()
    _check(_lib.ep_layout_dispatch(
        _ptr(topk_idx), T, K, num_experts, num_ranks, rank, expert_alignment, _ptr(workspace), workspace.numel(),
        *_layout_ptrs(outputs), _ptr(x), H, _ptr(topk_weights), EP_DTYPE_FP8_E4M3 if fp8 else EP_DTYPE_BF16,
        int(bool(do_expand)), int(bool(do_zero_padding)), ctypes.byref(s), ctypes.byref(h), _stream(stream)),
        "ep_layout_dispatch")
    return Handle(h, topk_idx, workspace, T, K, num_experts, num_ranks, rank, expert_alignment), outputs, out


def ep_layout_dispatch_noalloc(topk_idx, x, num_experts, out, num_ranks=1, rank=0, expert_alignment=1,
                               topk_weights=None, fp8=True, do_expand=True, do_zero_padding=False, outputs=None,
                               stream=None):
    """ep_layout_dispatch for callers that cannot allocate: no workspace (the library's static per-GPU scratch
    serves as one), caller-supplied dispatch outputs `out`, and optional layout `outputs` (None: not written).
    Nothing is allocated here either.  The returned Handle wraps the GPU's static handle: valid until the next
    call of this function on the same GPU, which overwrites it; freeing it is a no-op.  Returns (Handle,
    outputs, out)."""
    _need(topk_idx, torch.int64, "topk_idx")
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [num_tokens, num_topk]")
    T, K = topk_idx.shape
    dev = topk_idx.device
    if num_ranks < 1 or num_experts < 1 or num_experts % num_ranks != 0:
        raise ValueError("num_experts must be a positive multiple of num_ranks")
    _need(x, torch.bfloat16, "x", dev)
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [num_tokens, hidden]")
    H = x.shape[1]
    if topk_weights is not None:
        _need(topk_weights, torch.float32, "topk_weights", dev, (T, K))
    if out is None:
        raise ValueError("ep_layout_dispatch_noalloc needs caller-allocated dispatch outputs (out)")
    cap = check_dispatch_outputs(out, T, K, num_ranks, H, fp8, do_expand, dev)
    if outputs is None:
        outputs = {}
    else:
        check_layout_outputs(outputs, T, num_experts, num_ranks, dev)
    s = _dispatch_struct(out, cap)
    h = ctypes.c_void_p()
    _check(_lib.ep_layout_dispatch_noalloc(
        _ptr(topk_idx), T, K, num_experts, num_ranks, rank, expert_alignment, *_layout_ptrs(outputs), _ptr(x), H,
        _ptr(topk_weights), EP_DTYPE_FP8_E4M3 if fp8 else EP_DTYPE_BF16, int(bool(do_expand)),
        int(bool(do_zero_padding)), ctypes.byref(s), ctypes.byref(h), _stream(stream)),
        "ep_layout_dispatch_noalloc")
    return Handle(h, topk_idx, None, T, K, num_experts, num_ranks, rank, expert_alignment), outputs, out


def ep_combine(handle: Handle, y, topk_weights=None, bias=None, out=None, stream=None):
    """Combine expert outputs `y` (bf16 [>= recv_capacity, H]) back to token order.  Returns out [T, H] bf16."""
    _need(y, torch.bfloat16, "y")
    if y.dim() != 2:
        raise ValueError("y must be [rows, hidden]")
    H = y.shape[1]
    T = handle.num_tokens
    dev = y.device
    if topk_weights is not None:
        _need(topk_weights, torch.float32, "topk_weights", dev, (T, handle.num_topk))
    if bias is not None:
        _need(bias, torch.bfloat16, "bias", dev, (T, H))
    if out is None:
        out = _on_stream(stream, torch.empty, (T, H), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, torch.bfloat16, "out", dev, (T, H))
    _check(_lib.ep_combine(handle.ptr, _ptr(y), H, y.shape[0], _ptr(topk_weights), _ptr(bias), _ptr(out),
                           _stream(stream)), "ep_combine")
    return out


def ep_combine_tokens(handle: Handle, y, bias=None, out=None, stream=None):
    """Combine for the token-major rows (dispatch with do_expand=False): out[t] = y[row of t] + bias, where
    y (bf16 [>= T, H]) holds one row per token of this rank in dispatch order.  Returns out [T, H] bf16."""
    _need(y, torch.bfloat16, "y")
    if y.dim() != 2:
        raise ValueError("y must be [rows, hidden]")
    H = y.shape[1]
    T = handle.num_tokens
    dev = y.device
    if bias is not None:
        _need(bias, torch.bfloat16, "bias", dev, (T, H))
    if out is None:
        out = _on_stream(stream, torch.empty, (T, H), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, torch.bfloat16, "out", dev, (T, H))
    _check(_lib.ep_combine_tokens(handle.ptr, _ptr(y), H, y.shape[0], _ptr(bias), _ptr(out), _stream(stream)),
           "ep_combine_tokens")
    return out


def ep_dispatch_rows(handle: Handle, rows, scales=None, topk_weights=None, do_zero_padding=False, out=None,
                     stream=None):
    """Place received rows (uint8 [N, row_bytes] or bf16 [N, H]) expert-major through `handle` (a layout over
    the rows' local expert ids).  scales: fp32 [N, G] travelling with the rows.  Returns the output dict."""
    if not isinstance(rows, torch.Tensor) or rows.dtype not in (torch.uint8, torch.bfloat16):
        raise TypeError("rows must be a uint8 or bfloat16 tensor")
    _need(rows, rows.dtype, "rows")
    if rows.dim() != 2 or rows.shape[0] != handle.num_tokens:
        raise ValueError("rows must be [num_received_rows, row_elements]")
    dev = rows.device
    N = handle.num_tokens
    row_bytes = rows.shape[1] * rows.element_size()
    G = 0
    if scales is not None:
        if not isinstance(scales, torch.Tensor) or scales.dim() != 2:
            raise ValueError("scales must be a 2-D tensor [num_received_rows, num_scales]")
        G = scales.shape[1]
        _need(scales, torch.float32, "scales", dev, (N, G))
    if topk_weights is not None:
        _need(topk_weights, torch.float32, "topk_weights", dev, (N, handle.num_topk))
    cap = handle.recv_capacity
    if out is None:
        out = _on_stream(stream, lambda: dict(
            recv_x=torch.empty((cap, rows.shape[1]), dtype=rows.dtype, device=dev),
            recv_x_scales=torch.empty((cap, G), dtype=torch.float32, device=dev) if G else None,
            recv_src_idx=torch.empty(cap, dtype=torch.int32, device=dev),
            recv_topk_weights=torch.empty(cap, dtype=torch.float32, device=dev)))
    cap = check_rows_outputs(out, rows.dtype, rows.shape[1], G, dev)
    s = _dispatch_struct(out, cap, _RECV_KEYS[:4])   # the library reads the recv fields only
    _check(_lib.ep_dispatch_rows(handle.ptr, _ptr(rows), row_bytes, _ptr(scales), G, _ptr(topk_weights),
                                 int(bool(do_zero_padding)), ctypes.byref(s), _stream(stream)), "ep_dispatch_rows")
    return out


def ep_combine_reduce(handle: Handle, partials=None, local=None, bias=None, out=None, hidden=None, stream=None):
    """Sum the combine partials returned by the other ranks (bf16 [R, T, H], window r from rank r) with this
    rank's local combine output and the bias.  Returns out [T, H] bf16."""
    T = handle.num_tokens
    ref = next((t for t in (partials, local, bias, out) if t is not None), None)
    if ref is None:
        raise ValueError("ep_combine_reduce needs at least one of partials, local, bias, out")
    _need(ref, torch.bfloat16, "partials/local/bias/out")
    H = ref.shape[-1] if hidden is None else hidden
    dev = ref.device
    if partials is not None:
        _need(partials, torch.bfloat16, "partials", dev, (handle.num_ranks, T, H))
    if local is not None:
        _need(local, torch.bfloat16, "local", dev, (T, H))
    if bias is not None:
        _need(bias, torch.bfloat16, "bias", dev, (T, H))
    if out is None:
        out = _on_stream(stream, torch.empty, (T, H), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, torch.bfloat16, "out", dev, (T, H))
    _check(_lib.ep_combine_reduce(handle.ptr, _ptr(partials), H, _ptr(local), _ptr(bias), _ptr(out),
                                  _stream(stream)), "ep_combine_reduce")
    return out


def ep_handle_free(handle: Handle):
    handle.free()


__all__ = ["ep_get_layout", "ep_dispatch", "ep_layout_dispatch", "ep_layout_dispatch_noalloc", "ep_combine", "ep_combine_tokens", "ep_handle_free", "ep_recv_capacity",
           "ep_dispatch_rows", "ep_combine_reduce",
           "ep_layout_workspace_bytes", "alloc_dispatch_outputs", "Handle", "EPError", "LIB_PATH",
           "hip_runtimes_loaded"]
