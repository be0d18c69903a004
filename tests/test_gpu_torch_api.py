"""GPU checks of the PyTorch entry points: autograd through the C ABI gives
exactly what direct vsa_fwd / vsa_bwd calls give (same kernels, same inputs),
the BSHD twin equals the BHSD entry on transposed tensors, the no-grad path
equals the training forward, and the block-map entry matches the oracle.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import GRAD_TOL, OUT_TOL, check
from workloads.synth import make_case

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.gpu_run import run_case  # noqa: E402
import bwd_block_map_amd as vsa  # noqa: E402


def _leaf(t):
    return t.detach().clone().cuda().requires_grad_(True)


def _video_autograd(case, layout, gate_grad=False):
    """out and grads through video_sparse_attn[_bshd] with loss sum(out * dO)."""
    q, k, v = (_leaf(t) for t in (case.q, case.k, case.v))
    gate = None
    if case.gate is not None:
        gate = _leaf(case.gate) if gate_grad else case.gate.cuda()
    fn = vsa.video_sparse_attn if layout == "bhsd" else vsa.video_sparse_attn_bshd
    out = fn(q, k, v, case.kv_var, case.q_var, case.topk, block_size=(4, 8, 8),
             compress_attn_weight=gate, scale=case.scale)
    (out * case.dout.cuda()).sum().backward()
    return out.detach(), q.grad, k.grad, v.grad, (gate.grad if gate_grad else None)


def _transposed(t):
    return None if t is None else t.transpose(1, 2).contiguous()


def test_video_entry_matches_the_c_abi_bit_for_bit():
    case = make_case("p1_gated", device="cuda")  # q_var / kv_var, top-k 2, per-element gate
    ref = run_case(case, keep_device=True)
    out, dq, dk, dv, _ = _video_autograd(case, "bhsd")
    for name, a, b in (("out", out, ref["out"]), ("dq", dq, ref["dq"]), ("dk", dk, ref["dk"]),
                       ("dv", dv, ref["dv"])):
        assert torch.equal(a, b), f"{name} differs from the direct C-ABI run"


def test_gate_gradient_matches_the_c_abi():
    case = make_case("p1_gated", device="cuda")
    ref = run_case(case, keep_device=True)
    *_, dgate = _video_autograd(case, "bhsd", gate_grad=True)
    assert torch.equal(dgate, ref["dgate"])


def test_bshd_entry_equals_bhsd_entry():
    case = make_case("p1_gated", device="cuda")
    a = _video_autograd(case, "bhsd")
    import copy
    cb = copy.copy(case)
    for n in ("q", "k", "v", "dout", "gate"):
        setattr(cb, n, _transposed(getattr(case, n)))
    b = _video_autograd(cb, "bshd")
    for name, x, y in zip(("out", "dq", "dk", "dv"), a[:4], b[:4]):
        assert torch.equal(x, y.transpose(1, 2)), f"{name}: BSHD != BHSD"


def test_no_grad_path_equals_training_forward():
    case = make_case("p1_infer", device="cuda")
    q, k, v = (_leaf(t) for t in (case.q, case.k, case.v))
    train = vsa.video_sparse_attn(q, k, v, case.kv_var, case.q_var, case.topk, scale=case.scale)
    with torch.no_grad():
        infer = vsa.video_sparse_attn(q, k, v, case.kv_var, case.q_var, case.topk,
                                      scale=case.scale)
    assert not infer.requires_grad
    assert torch.equal(train.detach(), infer)


def test_block_map_entry_against_the_oracle():
    case = make_case("c1_vsa256_tiny", layout="bhsd", device="cuda")
    q, k, v = (_leaf(t) for t in (case.q, case.k, case.v))
    out, lse = vsa.block_sparse_attn(q, k, v, case.block_map.cuda(), kv_valid=case.kv_var,
                                     q_valid=case.q_var, layout="bhsd", scale=case.scale)
    assert not lse.requires_grad
    (out * case.dout.cuda()).sum().backward()
    orc = oracle.Oracle(case, np.float64, threads=8)
    o_ref, _, l_ref = orc.fwd()
    dq_r, dk_r, dv_r = orc.bwd()[:3]
    check("out", o_ref, out.detach().float().cpu().numpy(), OUT_TOL)
    check("lse", l_ref, lse.float().cpu().numpy(), OUT_TOL)
    check("dq", dq_r, q.grad.float().cpu().numpy(), GRAD_TOL)
    check("dk", dk_r, k.grad.float().cpu().numpy(), GRAD_TOL)
    check("dv", dv_r, v.grad.float().cpu().numpy(), GRAD_TOL)
