"""CPU checks of bench.py's contract: the algorithmic byte model on the prefill shape against figures worked out
by hand from the per-row sizes, and the one-GPU guard of --gpus."""
import os
import subprocess
import sys

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_byte_model_prefill_by_hand():
    """Prefill: T = 4096, H = 7168, K = 8, one rank, FP8 rows of 7168 + 56 * 4 = 7392 bytes, zero padding.
    With V = 32768 routed rows and P = 15104 padding rows:
      dispatch = x 4096 * 14336 (58,720,256) + slot map and weights 4096 * 8 * 8 (262,144)
               + routed rows 32768 * (7392 + 8) (242,483,200) + padding metadata 15104 * 8 (120,832)
               + padding rows 15104 * 7392 (111,648,768)                                  = 413,235,200
      combine  = y rows 32768 * 14336 (469,762,048) + slots and weights 262,144 + out 58,720,256 = 528,744,448"""
    cfg = W.CONFIGS["prefill"]
    bm = bench.bytes_model(cfg, dict(V=32768, P=15104, N_send=0))
    assert bm["row_bytes"] == 7392
    assert bm["dispatch"] == 413_235_200
    assert bm["combine"] == 528_744_448


def test_byte_model_send_windows_and_bias():
    """ep8-like rank: send rows carry the row, the source index (4 B) and K int64 ids + K fp32 weights; a bias
    adds one more [T, 2H] read to combine; no zero padding means padding rows cost only their metadata."""
    cfg = W.Config("t", 4, 256, 16, 2, "uniform", 4, False, True, num_ranks=2, rank=0, bias=True)
    bm = bench.bytes_model(cfg, dict(V=3, P=5, N_send=2))
    row_b = 256 + 4 * 2
    assert bm["dispatch"] == 4 * 512 + 4 * 2 * 8 + 4 * 2 * 4 + 3 * (row_b + 8) + 5 * 8 + 2 * (row_b + 4 + 2 * 12)
    assert bm["combine"] == 3 * 512 + 4 * 2 * 8 + 4 * 512 + 4 * 512


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_all_cores_leg_computes_the_oracle():
    """The all-cores CPU leg (the oracle's C dispatch and combine over token ranges, one thread each) writes the
    same dispatch outputs, byte for byte, and the same combine as the single-threaded oracle calls."""
    import numpy as np
    import torch

    import oracle as O

    cfg = W.Config("t", 300, 1024, 32, 4, "uniform", 16, True, True, bias=True, bias_std=0.1)
    inp = W.make_inputs(cfg, seed=5)
    idx = np.ascontiguousarray(inp["topk_idx"].numpy())
    w = np.ascontiguousarray(inp["topk_weights"].numpy())
    x = np.ascontiguousarray(W.bf16_bits(inp["x"]))
    bias = W.bf16_bits(inp["bias"])
    lay = O.layout(idx, cfg.num_experts, 1, 0, cfg.expert_alignment)
    y = W.bf16_bits(W.normal_bf16((lay["cap"], cfg.hidden), torch.Generator().manual_seed(2)))
    ref = O.dispatch(x, idx, w, lay, cfg.num_experts, 1, 0, cfg.expert_alignment, fp8=True, zero_pad=True,
                     recv_fill=(0, 0.0))
    ref_out = O.combine(y, lay["slot"], w, bias)
    for ncores in (1, 3, 7):
        got, _ = bench.oracle_token_ranges(x, idx, w, y, bias, cfg, ncores)
        used = int(lay["psum"][-1])
        assert np.array_equal(got["recv_x"][:used], ref["recv_x"][:used])
        assert np.array_equal(got["recv_scales"][:used].view(np.uint32), ref["recv_scales"][:used].view(np.uint32))
        assert np.array_equal(got["recv_src"][:used], ref["recv_src"][:used])
        assert np.array_equal(got["recv_w"][:used].view(np.uint32), ref["recv_w"][:used].view(np.uint32))
        assert np.array_equal(got["out"], ref_out)


def test_local_rows_by_token_inverts_the_source_index():
    """The write probes' destination map: every row in use whose source index is a token goes to that token's
    list, in row order, and the others are the padding rows."""
    import numpy as np

    rng = np.random.default_rng(3)
    T, K, cap, used = 40, 6, 400, 360
    src = np.full(cap, -1, np.int64)
    rows = rng.choice(used, 150, replace=False)
    src[rows] = rng.integers(0, T, rows.size)
    src[used + 5] = 7                                    # past the rows in use: ignored
    token_rows, V, pads = bench.local_rows_by_token(src, used, T, K * 8)
    assert V == int((src[:used] >= 0).sum())
    assert pads.tolist() == [i for i in range(used) if src[i] < 0]
    for t in range(T):
        mine = [r for r in range(used) if src[r] == t]
        assert token_rows[t, :len(mine)].tolist() == mine
        assert (token_rows[t, len(mine):] == -1).all()


def test_probe_library_exports_what_bench_calls():
    """libbench_probe.so (built by __graft_entry__.build()) exports every probe bench.py declares: the Probe class
    sets argtypes on each of them, so a missing symbol would only surface on the GPU machine."""
    import ctypes
    import re

    import pytest

    if not os.path.exists(bench.PROBE_LIB):
        pytest.skip("libbench_probe.so is not built")
    lib = ctypes.CDLL(bench.PROBE_LIB)
    src = open(os.path.join(ROOT, "bench.py")).read()
    names = sorted(set(re.findall(r"self\.lib\.(probe_\w+)\.argtypes", src)))
    assert {"probe_combine_gathers", "probe_row_writes", "probe_dispatch_writes", "probe_flush"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
