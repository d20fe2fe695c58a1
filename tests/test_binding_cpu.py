"""The Python binding refuses host (CPU) tensors and non-tensors before any
pointer reaches the library (checked without a GPU)."""
import pytest
import torch

m = pytest.importorskip("moe_expert_ffn_router_amd")


def test_host_tensors_are_refused():
    logits = torch.zeros((4, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="device"):
        m.route_topk(logits, 2)
    with pytest.raises(ValueError, match="device"):
        m.route_align(logits, 2, 16)
    with pytest.raises(ValueError, match="device"):
        m.align_block(torch.zeros((4, 2), dtype=torch.int32), 8, 16)
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    w1 = torch.zeros((8, 256, 128), dtype=torch.bfloat16)
    w2 = torch.zeros((8, 128, 128), dtype=torch.bfloat16)
    ids = torch.zeros((4, 2), dtype=torch.int32)
    wts = torch.zeros((4, 2), dtype=torch.float32)
    sid = torch.zeros(256, dtype=torch.int32)
    be = torch.zeros(16, dtype=torch.int32)
    npad = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(ValueError, match="device"):
        m.ffn_bf16(x, w1, w2, ids, wts, sid, be, npad, 16)
    with pytest.raises(ValueError, match="device"):
        m.forward_small(logits, x, w1, w2, 2)
    with pytest.raises(ValueError, match="device"):
        m.forward_small_static(logits, x, w1, w2, 2)


def test_non_tensors_and_wrong_ranks_are_refused():
    with pytest.raises(TypeError):
        m.route_topk([[0.0, 1.0]], 1)
    with pytest.raises(ValueError, match="dimensions"):
        m.route_topk(torch.zeros(8), 1)
    with pytest.raises(ValueError, match="dimensions"):
        m.align_block(torch.zeros(8, dtype=torch.int32), 8, 16)
