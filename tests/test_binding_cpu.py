"""CPU checks of the Python binding's argument validation: every output tensor a caller hands in is checked
against the dtype and exact shape the library writes, before any library call, so a tensor that is too short or
of the wrong type is rejected instead of being written past its end.  Host tensors stand in for device tensors
(the checks take the expected device as an argument); nothing here calls into the library."""
import pytest
import torch

import combine_get_dispatch_03_amd as ep

CPU = torch.device("cpu")
T, K, R, H = 40, 4, 4, 256
G = H // 128
CAP = 200


def _fp8_out(R=R, do_expand=True):
    o = dict(recv_x=torch.empty((CAP, H), dtype=torch.uint8), recv_x_scales=torch.empty((CAP, G)),
             recv_src_idx=torch.empty(CAP, dtype=torch.int32),
             recv_topk_weights=torch.empty(CAP) if do_expand else torch.empty((T, K)))
    if not do_expand:
        o["recv_topk_idx"] = torch.empty((T, K), dtype=torch.int64)
    if R > 1:
        o.update(send_x=torch.empty((R, T, H), dtype=torch.uint8), send_x_scales=torch.empty((R, T, G)),
                 send_src_idx=torch.empty((R, T), dtype=torch.int32),
                 send_topk_idx=torch.empty((R, T, K), dtype=torch.int64), send_topk_weights=torch.empty((R, T, K)))
    return o


def test_valid_outputs_pass():
    assert ep.check_dispatch_outputs(_fp8_out(), T, K, R, H, True, True, CPU) == CAP
    assert ep.check_dispatch_outputs(_fp8_out(do_expand=False), T, K, R, H, True, False, CPU) == CAP
    bf = dict(recv_x=torch.empty((CAP, H), dtype=torch.bfloat16), recv_src_idx=None, recv_topk_weights=None)
    assert ep.check_dispatch_outputs(bf, T, K, 1, H, False, True, CPU) == CAP


@pytest.mark.parametrize("key,bad,err,match", [
    ("recv_x", torch.empty((CAP, H), dtype=torch.bfloat16), TypeError, "recv_x"),      # uint8 expected (FP8)
    ("recv_x", torch.empty((CAP, H // 2), dtype=torch.uint8), ValueError, "recv_x"),   # row too short
    ("recv_x_scales", torch.empty((CAP - 1, G)), ValueError, "recv_x_scales"),        # one row short
    ("recv_x_scales", torch.empty((CAP, G), dtype=torch.float64), TypeError, "recv_x_scales"),
    ("recv_x_scales", None, ValueError, "recv_x_scales"),                               # required for FP8
    ("recv_src_idx", torch.empty(CAP - 1, dtype=torch.int32), ValueError, "recv_src_idx"),
    ("recv_src_idx", torch.empty(CAP, dtype=torch.int64), TypeError, "recv_src_idx"),
    ("recv_topk_weights", torch.empty(CAP // 2), ValueError, "recv_topk_weights"),
    ("send_x", torch.empty((R, T - 1, H), dtype=torch.uint8), ValueError, "send_x"),
    ("send_x", None, ValueError, "send_x"),
    ("send_x_scales", torch.empty((R, T, G - 1)), ValueError, "send_x_scales"),
    ("send_src_idx", torch.empty((R - 1, T), dtype=torch.int32), ValueError, "send_src_idx"),
    ("send_topk_idx", torch.empty((R, T, K), dtype=torch.int32), TypeError, "send_topk_idx"),
    ("send_topk_weights", torch.empty((R, T, K - 1)), ValueError, "send_topk_weights"),
    ("recv_x", torch.empty((2 * CAP, H), dtype=torch.uint8)[::2], ValueError, "contiguous"),
])
def test_dispatch_output_rejections(key, bad, err, match):
    o = _fp8_out()
    o[key] = bad
    with pytest.raises(err, match=match):
        ep.check_dispatch_outputs(o, T, K, R, H, True, True, CPU)


def test_token_major_shapes():
    o = _fp8_out(do_expand=False)
    o["recv_topk_idx"] = torch.empty((T, K - 1), dtype=torch.int64)
    with pytest.raises(ValueError, match="recv_topk_idx"):
        ep.check_dispatch_outputs(o, T, K, R, H, True, False, CPU)
    o = _fp8_out(do_expand=False)
    o["recv_topk_weights"] = torch.empty(CAP)                   # expert-major shape in token-major mode
    with pytest.raises(ValueError, match="recv_topk_weights"):
        ep.check_dispatch_outputs(o, T, K, R, H, True, False, CPU)


def test_wrong_device_rejected():
    o = _fp8_out()
    with pytest.raises(ValueError, match="must be on"):
        ep.check_dispatch_outputs(o, T, K, R, H, True, True, torch.device("cuda", 0))


def test_rows_outputs():
    o = dict(recv_x=torch.empty((CAP, 80), dtype=torch.uint8), recv_x_scales=torch.empty((CAP, 3)),
             recv_src_idx=torch.empty(CAP, dtype=torch.int32), recv_topk_weights=torch.empty(CAP))
    assert ep.check_rows_outputs(o, torch.uint8, 80, 3, CPU) == CAP
    with pytest.raises(TypeError, match="recv_x"):
        ep.check_rows_outputs(o, torch.bfloat16, 40, 3, CPU)          # rows are bf16, recv_x uint8
    with pytest.raises(ValueError, match="recv_x_scales"):
        ep.check_rows_outputs(o, torch.uint8, 80, 4, CPU)
    o["recv_src_idx"] = torch.empty(CAP - 5, dtype=torch.int32)
    with pytest.raises(ValueError, match="recv_src_idx"):
        ep.check_rows_outputs(o, torch.uint8, 80, 3, CPU)


def test_layout_outputs_and_workspace():
    E = 16
    good = dict(num_tokens_per_rank=torch.empty(R, dtype=torch.int32), num_tokens_per_expert=None,
                is_token_in_rank=torch.empty((T, R), dtype=torch.uint8),
                psum_num_recv_tokens_per_expert=torch.empty(E // R + 1, dtype=torch.int32), num_invalid_topk=None)
    ep.check_layout_outputs(good, T, E, R, CPU)
    for key, bad in (("num_tokens_per_expert", torch.empty(E - 1, dtype=torch.int32)),
                     ("is_token_in_rank", torch.empty((T, R), dtype=torch.int32)),
                     ("psum_num_recv_tokens_per_expert", torch.empty(E // R, dtype=torch.int32)),
                     ("num_invalid_topk", torch.empty(2, dtype=torch.int32))):
        o = dict(good)
        o[key] = bad
        with pytest.raises((TypeError, ValueError), match=key):
            ep.check_layout_outputs(o, T, E, R, CPU)
    ep.check_workspace(torch.empty(4096, dtype=torch.uint8), CPU)
    with pytest.raises(TypeError, match="workspace"):
        ep.check_workspace(torch.empty(1024, dtype=torch.int32), CPU)   # numel would not be its byte length
    with pytest.raises(ValueError, match="1-D"):
        ep.check_workspace(torch.empty((64, 64), dtype=torch.uint8), CPU)
