"""Host-side checks of the PyTorch entry points (no GPU): layout and gate-mode
inference and argument validation, which run before any library call."""

from __future__ import annotations

import pytest
import torch

from bwd_block_map_amd.torch_api import block_sparse_attn, dims, gate_mode_of


def test_dims_bhsd_and_bshd():
    q = torch.empty(2, 3, 512, 128)
    k = torch.empty(2, 1, 768, 128)
    assert dims(q, k, "bhsd") == (2, 3, 1, 512, 768, 128)
    qs, ks = q.transpose(1, 2), k.transpose(1, 2)
    assert dims(qs, ks, "bshd") == (2, 3, 1, 512, 768, 128)


def test_dims_rejects_bad_input():
    with pytest.raises(ValueError):
        dims(torch.empty(2, 512, 128), torch.empty(2, 512, 128), "bhsd")
    with pytest.raises(ValueError):
        dims(torch.empty(1, 2, 64, 128), torch.empty(1, 2, 64, 128), "tnd")
    with pytest.raises(ValueError):
        dims(torch.empty(1, 2, 64, 128), torch.empty(2, 2, 64, 128), "bhsd")


def test_gate_mode_inference():
    q = torch.empty(1, 4, 256, 128)
    assert gate_mode_of(None, q, "bhsd") == "none"
    assert gate_mode_of(torch.empty_like(q), q, "bhsd") == "per_element"
    assert gate_mode_of(torch.empty(1, 4, 256), q, "bhsd") == "per_token"
    with pytest.raises(ValueError):
        gate_mode_of(torch.empty(1, 4, 128), q, "bhsd")


def test_block_sparse_attn_checks_the_map_before_any_launch():
    q = torch.empty(1, 2, 512, 128, dtype=torch.bfloat16)
    bad_blocks = torch.ones(1, 2, 3, 2, dtype=torch.uint8)  # 512 rows do not split into 3 blocks
    with pytest.raises(ValueError):
        block_sparse_attn(q, q, q, bad_blocks)
    bad_heads = torch.ones(1, 3, 2, 2, dtype=torch.uint8)
    with pytest.raises(ValueError):
        block_sparse_attn(q, q, q, bad_heads)


def test_tnd_entry_checks_lengths_and_map_before_any_launch():
    from bwd_block_map_amd.torch_api import block_sparse_attn_tnd
    q = torch.empty(100, 4, 128, dtype=torch.bfloat16)
    k = torch.empty(150, 2, 128, dtype=torch.bfloat16)
    good = torch.ones(2, 4, 1, 1, dtype=torch.uint8)
    with pytest.raises(ValueError, match="sum to"):  # 60 + 30 != 100 query tokens
        block_sparse_attn_tnd(q, k, k, good, (128, 128), [60, 30], [100, 50])
    with pytest.raises(ValueError, match="one entry per sequence"):
        block_sparse_attn_tnd(q, k, k, good, (128, 128), [60, 40], [150])
    with pytest.raises(ValueError, match="block_map must be"):  # 2 KV blocks of 64 for 100 keys
        block_sparse_attn_tnd(q, k, k, good, (128, 64), [60, 40], [100, 50])
    with pytest.raises(ValueError, match="3-D"):
        block_sparse_attn_tnd(q[None], k, k, good, (128, 128), [60, 40], [100, 50])
