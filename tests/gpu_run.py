"""Run a workload case through the C-ABI library (test-side glue).

Copies the seeded inputs to the GPU, fills a vsa_problem and calls vsa_fwd /
vsa_bwd / block_map_to_index through the Python binding. Nothing here
computes attention; the results come back as numpy arrays.
"""

from __future__ import annotations

import numpy as np
import torch

import bwd_block_map_amd as vsa


def device_inputs(case, device="cuda"):
    d = {n: (getattr(case, n).to(device) if getattr(case, n) is not None else None)
         for n in ("q", "k", "v", "dout", "gate")}
    d["q_valid"] = torch.as_tensor(case.q_var, dtype=torch.int32, device=device) \
        if case.q_var is not None else None
    d["kv_valid"] = torch.as_tensor(case.kv_var, dtype=torch.int32, device=device) \
        if case.kv_var is not None else None
    if case.layout == "tnd":
        d["cu_q"] = torch.as_tensor(np.concatenate([[0], np.cumsum(case.q_lens)]),
                                    dtype=torch.int32, device=device)
        d["cu_kv"] = torch.as_tensor(np.concatenate([[0], np.cumsum(case.kv_lens)]),
                                     dtype=torch.int32, device=device)
    else:
        d["cu_q"] = d["cu_kv"] = None
    d["map"] = case.block_map.to(device).contiguous() if case.block_map is not None else None
    return d


def problem_for(case, d, map_batch_stride=None, atomic_dq=False, persistent=None):
    proj = case.gate_mode == "projected"
    return vsa.make_problem(
        dtype=case.torch_dtype, layout=case.layout, B=case.B, Hq=case.Hq, Hkv=case.Hkv,
        Sq=case.Sq, Skv=case.Skv, D=case.D, q_block=case.q_block, kv_block=case.kv_block,
        q_valid=d["q_valid"], kv_valid=d["kv_valid"], cu_seqlens_q=d["cu_q"],
        cu_seqlens_kv=d["cu_kv"],
        max_seqlen_q=max(case.q_lens) if case.q_lens else 0,
        max_seqlen_kv=max(case.kv_lens) if case.kv_lens else 0,
        scale=case.scale, topk=case.topk, gate_mode=case.gate_mode,
        map_batch_stride=map_batch_stride, atomic_dq=atomic_dq, persistent=persistent,
        gate_proj=d["gate"] if proj else None)


def run_case(case, training=True, backward=True, dout_none=False, device="cuda", d=None,
             keep_device=False, atomic_dq=False, persistent=None):
    d = device_inputs(case, device) if d is None else d
    p = problem_for(case, d, atomic_dq=atomic_dq, persistent=persistent)
    buf = vsa.Buffers(p, d["q"], training=training or backward)
    bmap = d["map"] if case.topk == 0 else buf.map
    proj = case.gate_mode == "projected"
    # a projected gate: its parameters go into the problem, `gate` receives
    # the per-token gate values the forward computes
    gate = d["gate"]
    if proj:
        shape = (case.B, case.Hq, case.Sq) if case.layout == "bhsd" else (case.B, case.Sq, case.Hq)
        gate = torch.full(shape, float("nan"), dtype=case.torch_dtype, device=device)
    vsa.vsa_fwd(p, d["q"], d["k"], d["v"], bmap, gate, buf.out, buf.lse,
                buf.saved if training or backward else None, buf.ws_fwd)
    res = dict(out=buf.out, lse=buf.lse, map=bmap)
    if proj:
        res["gate_vals"] = gate
    if backward:
        dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
        if proj:
            dg = torch.full((case.Hq * case.D + case.Hq,), float("nan"), dtype=torch.float32,
                            device=device)
        else:
            dg = torch.empty_like(d["gate"]) if d["gate"] is not None else None
        vsa.vsa_bwd(p, d["q"], d["k"], d["v"], None if proj else d["gate"],
                    None if dout_none else d["dout"], buf.out, buf.lse, buf.saved, dq, dk, dv, dg,
                    buf.ws_bwd)
        res.update(dq=dq, dk=dk, dv=dv, dgate=dg)
    torch.cuda.synchronize()
    if keep_device:
        return res
    return {k: (v.float().cpu().numpy() if v is not None and v.dtype != torch.uint8
                else (v.cpu().numpy() if v is not None else None)) for k, v in res.items()}
