"""CPU checks of the C ABI: the library loads, exports every function include/ep.h declares, and its host-only
helpers and pre-launch validation behave as documented.  Nothing here launches a kernel."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep.h")
LIB = os.path.join(ROOT, "combine_get_dispatch_03_amd", "libep_mi355x.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import combine_get_dispatch_03_amd.build as b
        b.build()
    L = ctypes.CDLL(LIB)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    L.ep_recv_capacity.restype = I64
    L.ep_recv_capacity.argtypes = [I, I, I, I]
    L.ep_layout_workspace_bytes.restype = SZ
    L.ep_layout_workspace_bytes.argtypes = [I, I, I, I, I]
    L.ep_status_string.restype = ctypes.c_char_p
    L.ep_last_error.restype = ctypes.c_char_p
    L.ep_get_layout.restype = I
    L.ep_get_layout.argtypes = [P, I, I, I, I, I, I, P, SZ, P, P, P, P, P, ctypes.POINTER(P), P]
    L.ep_dispatch.restype = I
    L.ep_dispatch.argtypes = [P, P, I, P, I, I, I, P, P]
    L.ep_combine.restype = I
    L.ep_combine.argtypes = [P, P, I, I64, P, P, P, P]
    L.ep_handle_free.restype = I
    L.ep_handle_free.argtypes = [P]
    L.ep_combine_tokens.restype = I
    L.ep_combine_tokens.argtypes = [P, P, I, I64, P, P, P]
    return L


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("ep_get_layout", "ep_dispatch", "ep_combine", "ep_handle_free", "ep_recv_capacity",
              "ep_layout_workspace_bytes", "ep_status_string", "ep_last_error", "ep_dispatch_rows",
              "ep_combine_reduce", "ep_combine_tokens"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in _declared():
        assert hasattr(lib, n), n


def test_recv_capacity(lib):
    assert lib.ep_recv_capacity(4096, 8, 256, 128) == 4096 * 8 + 256 * 127
    assert lib.ep_recv_capacity(128, 8, 256, 128) == 33536
    assert lib.ep_recv_capacity(4096, 8, 256, 1) == 32768
    assert lib.ep_recv_capacity(0, 8, 8, 16) == 8 * 15
    assert lib.ep_recv_capacity(-1, 8, 8, 16) == -1
    assert lib.ep_recv_capacity(1 << 30, 32, 1, 1) == -1     # beyond int32 rows


def test_workspace_bytes(lib):
    n = lib.ep_layout_workspace_bytes(4096, 8, 256, 1, 128)
    assert n >= 4096 * 8 * 4 + 16 * 256 * 4
    assert lib.ep_layout_workspace_bytes(0, 8, 256, 1, 128) > 0
    assert lib.ep_layout_workspace_bytes(4096, 8, 256, 3, 128) == 0   # 256 % 3 != 0
    assert lib.ep_layout_workspace_bytes(4096, 33, 256, 1, 128) == 0  # K > 32
    assert lib.ep_layout_workspace_bytes(4096, 8, 2048, 1, 128) == 0  # E > 1024
    assert lib.ep_layout_workspace_bytes(4096, 8, 256, 128, 128) == 0 # R > 64
    # the per-rank token rows ([T, R] int32) grow with R (the per-local-expert arrays shrink a little)
    assert lib.ep_layout_workspace_bytes(4096, 8, 256, 8, 1) - lib.ep_layout_workspace_bytes(4096, 8, 256, 1, 1) \
        >= 4096 * 7 * 4 - 2 * 256 * 4 - 512


def test_status_strings(lib):
    assert lib.ep_status_string(0) == b"ok"
    assert lib.ep_status_string(1) == b"invalid argument"
    assert lib.ep_status_string(2) == b"unsupported mode"
    assert lib.ep_status_string(3) == b"HIP error"


@pytest.mark.parametrize("T,K,E,R,rank,A,ws_ok,why", [
    (16, 0, 8, 1, 0, 1, True, b"num_topk"),
    (16, 4, 0, 1, 0, 1, True, b"num_experts"),
    (16, 4, 8, 3, 0, 1, True, b"multiple of num_ranks"),
    (16, 4, 8, 2, 2, 1, True, b"rank"),
    (16, 4, 8, 1, 0, 0, True, b"expert_alignment"),
    (-1, 4, 8, 1, 0, 1, True, b"num_tokens"),
    (16, 4, 8, 1, 0, 1, False, b"workspace_bytes"),
])
def test_layout_validation_before_launch(lib, T, K, E, R, rank, A, ws_ok, why):
    h = ctypes.c_void_p()
    fake_dev = ctypes.c_void_p(0x10000)     # never dereferenced: validation fails first
    ws = ctypes.c_void_p(0x100000)
    rc = lib.ep_get_layout(fake_dev, T, K, E, R, rank, A, ws, 1 << 30 if ws_ok else 16, None, None, None, None,
                           None, ctypes.byref(h), None)
    assert rc == 1
    assert why in lib.ep_last_error()
    assert h.value is None


def test_layout_rejects_null_and_misaligned(lib):
    h = ctypes.c_void_p()
    rc = lib.ep_get_layout(None, 16, 4, 8, 1, 0, 1, ctypes.c_void_p(0x100000), 1 << 20, None, None, None, None,
                           None, ctypes.byref(h), None)
    assert rc == 1 and b"topk_idx" in lib.ep_last_error()
    rc = lib.ep_get_layout(ctypes.c_void_p(0x10000), 16, 4, 8, 1, 0, 1, ctypes.c_void_p(0x100010), 1 << 20, None,
                           None, None, None, None, ctypes.byref(h), None)
    assert rc == 1 and b"256-byte" in lib.ep_last_error()
    rc = lib.ep_get_layout(ctypes.c_void_p(0x10000), 16, 4, 8, 1, 0, 1, ctypes.c_void_p(0x100000), 1 << 20, None,
                           None, None, None, None, None, None)
    assert rc == 1 and b"handle_out" in lib.ep_last_error()


def test_dispatch_combine_reject_bad_handles(lib):
    assert lib.ep_dispatch(None, None, 128, None, 1, 1, 0, None, None) == 1
    assert b"handle" in lib.ep_last_error()
    assert lib.ep_combine(None, None, 128, 0, None, None, None, None) == 1
    bogus = (ctypes.c_uint32 * 64)()                       # a host block that is not a handle
    assert lib.ep_dispatch(ctypes.cast(bogus, ctypes.c_void_p), None, 128, None, 1, 1, 0, None, None) == 1
    assert lib.ep_handle_free(None) == 0
    assert lib.ep_combine_tokens(None, None, 128, 0, None, None, None) == 1
    assert b"handle" in lib.ep_last_error()


def test_handle_lookup_never_dereferences(lib):
    """A pointer that is not a live handle is rejected without being read: addresses that are not mapped at all
    (reading them would crash the process) and a host block whose bytes look like anything."""
    for addr in (0x10, 0x1000, 0x7FFF0000DEAD0):
        p = ctypes.c_void_p(addr)
        assert lib.ep_handle_free(p) == 1
        assert b"not live" in lib.ep_last_error()
        assert lib.ep_dispatch(p, None, 128, None, 1, 1, 0, None, None) == 1
        assert lib.ep_combine(p, None, 128, 0, None, None, None, None) == 1
        assert lib.ep_combine_tokens(p, None, 128, 0, None, None, None) == 1
    junk = (ctypes.c_uint8 * 4096)(*([0xFF] * 4096))
    assert lib.ep_handle_free(ctypes.cast(junk, ctypes.c_void_p)) == 1


def test_limit_on_window_rows(lib):
    """num_tokens * num_ranks must fit in int32 (send-window rows are int32 in the kernels)."""
    h = ctypes.c_void_p()
    T = (1 << 31) // 64 + 1                                # T * 64 > INT32_MAX, T * K and the capacity fit
    rc = lib.ep_get_layout(ctypes.c_void_p(0x10000), T, 1, 64, 64, 0, 1, ctypes.c_void_p(0x100000), 1 << 40,
                           None, None, None, None, None, ctypes.byref(h), None)
    assert rc == 1 and b"num_ranks" in lib.ep_last_error()
    assert lib.ep_layout_workspace_bytes(T, 1, 64, 64, 1) == 0
    assert lib.ep_layout_workspace_bytes(T, 1, 64, 32, 1) > 0


def test_noalloc_rejects_oversize_before_anything(lib):
    """ep_layout_dispatch_noalloc rejects sizes whose layout workspace exceeds its 4 MiB static scratch, on the host,
    before it looks up a device (so this runs without a GPU; the pointers are never read)."""
    P, I = ctypes.c_void_p, ctypes.c_int
    f = lib.ep_layout_dispatch_noalloc
    f.restype = I
    f.argtypes = [P, I, I, I, I, I, I, P, P, P, P, P, P, I, P, I, I, I, P, ctypes.POINTER(P), P]
    ws = lib.ep_layout_workspace_bytes
    assert ws(110000, 8, 256, 1, 128) > 4 << 20 >= ws(100000, 8, 256, 1, 128)
    h = ctypes.c_void_p()
    rc = f(P(0x10000), 110000, 8, 256, 1, 0, 128, None, None, None, None, None, P(0x20000), 128, None, 1, 1, 0,
           None, ctypes.byref(h), None)
    assert rc == 1 and b"static scratch" in lib.ep_last_error()
    assert h.value is None
    rc = f(P(0x10000), 100, 8, 256, 1, 0, 128, None, None, None, None, None, P(0x20000), 128, None, 1, 1, 0,
           None, None, None)
    assert rc == 1 and b"handle_out" in lib.ep_last_error()


_OUT_FIELDS = ("recv_x", "recv_x_scales", "recv_src_idx", "recv_topk_weights", "recv_topk_idx", "recv_capacity",
               "send_x", "send_x_scales", "send_src_idx", "send_topk_idx", "send_topk_weights")


def test_dispatch_out_struct_matches_header(tmp_path):
    """The binding's ctypes mirror of ep_dispatch_out_t has the C struct's size and field offsets (gcc compiles a
    probe against include/ep.h and prints them)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "probe.c"
    body = "".join('    printf("%%s %%zu\\n", "%s", offsetof(ep_dispatch_out_t, %s));\n' % (f, f) for f in _OUT_FIELDS)
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "ep.h"\nint main(void) {\n'
                   '    printf("sizeof %zu\\n", sizeof(ep_dispatch_out_t));\n' + body + '    return 0;\n}\n')
    exe = tmp_path / "probe"
    subprocess.run([cc, "-std=c11", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], check=True, capture_output=True,
                                                       text=True).stdout.splitlines())
    import combine_get_dispatch_03_amd as ep
    D = ep._DispatchOut
    assert [f[0] for f in D._fields_] == list(_OUT_FIELDS)
    assert int(got["sizeof"]) == ctypes.sizeof(D)
    for f in _OUT_FIELDS:
        assert int(got[f]) == getattr(D, f).offset, f


def test_dispatch_struct_from_tensors():
    """The binding fills the struct from whichever output tensors are present, NULL for the rest, and takes
    recv_capacity from recv_x's rows (host tensors stand in: only their addresses are read)."""
    import torch
    import combine_get_dispatch_03_amd as ep
    out = dict(recv_x=torch.empty((37, 16), dtype=torch.uint8), recv_x_scales=torch.empty((37, 1)),
               recv_src_idx=None, recv_topk_weights=torch.empty(37), send_x=torch.empty((2, 5, 16), dtype=torch.uint8))
    s = ep._dispatch_struct(out, 37)
    assert s.recv_capacity == 37
    for f in _OUT_FIELDS:
        if f == "recv_capacity":
            continue
        t = out.get(f)
        assert getattr(s, f) == (t.data_ptr() if t is not None else None), f
