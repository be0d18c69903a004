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
from workloads.synth import build_case, make_case

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


def test_vsa128_video_entries_against_the_oracle():
    """VSA-128: (2, 8, 8) video tiles of 128 tokens through video_sparse_attn and
    its BSHD twin, with partial q_var / kv_var, pooled-score top-k and a signed
    q-shaped gate, autograd through q, k, v and the gate, against the oracle."""
    from tests.test_gpu_parity import _topk_agreement
    case = build_case("vsa128", dtype="bf16", layout="bhsd", B=1, Hq=2, D=128, q_block=128,
                      kv_block=128, q_var=[128, 77, 128, 40], kv_var=[128, 128, 33, 128, 90],
                      topk=3, map_kind="none", gate_mode="per_element", gate_kind="scaled",
                      pad_dout=False, seed=43, device="cuda")
    orc = oracle.Oracle(case, np.float64, threads=8)
    o_ref, _, _ = orc.fwd()
    dq_r, dk_r, dv_r, dg_r = orc.bwd()
    for layout in ("bhsd", "bshd"):
        c = case
        if layout == "bshd":
            import copy
            c = copy.copy(case)
            for n in ("q", "k", "v", "dout", "gate"):
                setattr(c, n, _transposed(getattr(case, n)))
        q, k, v, g = (_leaf(getattr(c, n)) for n in ("q", "k", "v", "gate"))
        fn = vsa.video_sparse_attn if layout == "bhsd" else vsa.video_sparse_attn_bshd
        out = fn(q, k, v, c.kv_var, c.q_var, c.topk, block_size=(2, 8, 8),
                 compress_attn_weight=g, scale=c.scale)
        (out * c.dout.cuda()).sum().backward()
        back = (lambda t: t.transpose(1, 2)) if layout == "bshd" else (lambda t: t)
        # the selection the library made must be the oracle's (no near-ties here)
        p = vsa.make_problem(dtype=q.dtype, layout=layout, B=1, Hq=2, Hkv=2, Sq=c.Sq,
                             Skv=c.Skv, D=128, q_block=128, kv_block=128,
                             q_valid=torch.as_tensor(c.q_var, dtype=torch.int32, device="cuda"),
                             kv_valid=torch.as_tensor(c.kv_var, dtype=torch.int32, device="cuda"),
                             scale=c.scale, topk=c.topk, gate_mode="per_element")
        buf = vsa.Buffers(p, q.detach(), training=False)
        vsa.vsa_fwd(p, q.detach(), k.detach(), v.detach(), buf.map, g.detach(), buf.out, buf.lse,
                    None, buf.ws_fwd)
        torch.cuda.synchronize()
        assert _topk_agreement(orc, buf.map.cpu().numpy()).all()
        print(f"[vsa128 {layout}]")
        check("out", o_ref, back(out.detach()).float().cpu().numpy(), OUT_TOL)
        for name, ref, t in (("dq", dq_r, q), ("dk", dk_r, k), ("dv", dv_r, v), ("dgate", dg_r, g)):
            check(name, ref, back(t.grad).float().cpu().numpy(), GRAD_TOL)


def test_projected_gate_through_autograd():
    """video_sparse_attn with gate_proj = (w, b): autograd returns exactly the
    C ABI's dq, dk, dv and its [dw | db] split into w.grad and b.grad."""
    case = build_case("proj_api", dtype="bf16", layout="bshd", B=1, Hq=4, Hkv=2, D=128,
                      q_var=[256, 90, 256], kv_var=[256, 256, 0, 140], topk=2, map_kind="none",
                      gate_mode="projected", seed=54, device="cuda")
    ref = run_case(case, keep_device=True)
    Hq, D = case.Hq, case.D
    w = case.gate[:Hq * D].reshape(Hq, D).clone().requires_grad_(True)
    b = case.gate[Hq * D:].clone().requires_grad_(True)
    q, k, v = (_leaf(t) for t in (case.q, case.k, case.v))
    out = vsa.video_sparse_attn_bshd(q, k, v, case.kv_var, case.q_var, case.topk,
                                     block_size=(4, 8, 8), scale=case.scale, gate_proj=(w, b))
    (out * case.dout.cuda()).sum().backward()
    for name, a, r in (("out", out.detach(), ref["out"]), ("dq", q.grad, ref["dq"]),
                       ("dk", k.grad, ref["dk"]), ("dv", v.grad, ref["dv"])):
        assert torch.equal(a, r), f"{name} differs from the direct C-ABI run"
    assert torch.equal(w.grad.reshape(-1), ref["dgate"][:Hq * D])
    assert torch.equal(b.grad, ref["dgate"][Hq * D:])
    with pytest.raises(ValueError):
        vsa.video_sparse_attn_bshd(q, k, v, case.kv_var, case.q_var, case.topk,
                                   gate_proj=(w[:, :64], b))


def test_per_video_counts_through_the_video_entry():
    """video_sparse_attn with [B, tiles] counts (one row per video) gives
    exactly the C ABI's outputs and gradients for the same problem."""
    case = build_case("per_video", dtype="bf16", layout="bhsd", B=2, Hq=2, D=128,
                      q_var=[[256, 90, 256], [256, 256, 40]],
                      kv_var=[[256, 256, 0, 140], [70, 256, 256, 256]], topk=2, map_kind="none",
                      gate_mode="per_token", seed=73, device="cuda")
    ref = run_case(case, keep_device=True)
    out, dq, dk, dv, dgate = _video_autograd(case, "bhsd", gate_grad=True)
    for name, a, b in (("out", out, ref["out"]), ("dq", dq, ref["dq"]), ("dk", dk, ref["dk"]),
                       ("dv", dv, ref["dv"]), ("dgate", dgate, ref["dgate"])):
        assert torch.equal(a, b), f"{name} differs from the direct C-ABI run"


def test_tnd_entry_matches_the_c_abi_and_the_oracle():
    """block_sparse_attn_tnd (packed sequences, per-sequence lengths, GQA) gives
    exactly the C ABI's out, lse and gradients for the same problem, and the
    oracle's within the bars."""
    case = make_case("c3_tnd_gqa_page", device="cuda")
    ref = run_case(case, keep_device=True)
    q, k, v = (_leaf(t) for t in (case.q, case.k, case.v))
    out, lse = vsa.block_sparse_attn_tnd(q, k, v, case.block_map.cuda(),
                                         (case.q_block, case.kv_block), case.q_lens,
                                         case.kv_lens, scale=case.scale)
    (out * case.dout.cuda()).sum().backward()
    for name, a, b in (("out", out.detach(), ref["out"]), ("lse", lse, ref["lse"]),
                       ("dq", q.grad, ref["dq"]), ("dk", k.grad, ref["dk"]),
                       ("dv", v.grad, ref["dv"])):
        assert torch.equal(a, b), f"{name} differs from the direct C-ABI run"
    orc = oracle.Oracle(case, np.float64, threads=8)
    o_ref, _, l_ref = orc.fwd()
    check("out", o_ref, out.detach().float().cpu().numpy(), OUT_TOL)
    dq_r, dk_r, dv_r = orc.bwd()[:3]
    check("dk", dk_r, k.grad.float().cpu().numpy(), GRAD_TOL)
