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
