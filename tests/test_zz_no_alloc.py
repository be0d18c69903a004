"""vsa_fwd_noalloc (the forward whose workspace is the library's own device
scratch) against vsa_fwd with a caller workspace, through the C ABI: two calls
in a row, the second on a smaller problem, each bit-identical to vsa_fwd (out,
lse, the top-k map), and a backward from the no-alloc forward's saved state
identical to one from vsa_fwd's."""

from __future__ import annotations

import pytest
import torch

from workloads.synth import build_case, make_case

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.gpu_run import device_inputs, problem_for  # noqa: E402
import bwd_block_map_amd as vsa  # noqa: E402


def _both(case, training):
    d = device_inputs(case)
    p = problem_for(case, d)
    assert vsa.vsa_sizes(p)["ws_fwd"] <= vsa.NOALLOC_SCRATCH_BYTES
    ref = vsa.Buffers(p, d["q"], training=training)
    new = vsa.Buffers(p, d["q"], training=training)
    # poison the outputs of the call under test so stale values cannot pass
    new.out.fill_(float("nan"))
    new.lse.fill_(float("nan"))
    if new.map is not None:
        new.map.fill_(7)
    rmap = d["map"] if case.topk == 0 else ref.map
    nmap = d["map"] if case.topk == 0 else new.map
    vsa.vsa_fwd(p, d["q"], d["k"], d["v"], rmap, d["gate"], ref.out, ref.lse,
                ref.saved if training else None, ref.ws_fwd)
    vsa.vsa_fwd_noalloc(p, d["q"], d["k"], d["v"], nmap, d["gate"], new.out, new.lse,
                        new.saved if training else None)
    torch.cuda.synchronize()
    assert torch.equal(ref.out, new.out), case.name
    assert torch.equal(ref.lse, new.lse), case.name
    assert torch.equal(rmap, nmap), case.name
    return d, p, ref, new


def _grads(case, d, p, buf):
    dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
    dg = torch.empty_like(d["gate"]) if d["gate"] is not None else None
    vsa.vsa_bwd(p, d["q"], d["k"], d["v"], d["gate"], d["dout"], buf.out, buf.lse, buf.saved,
                dq, dk, dv, dg, buf.ws_bwd)
    torch.cuda.synchronize()
    return dq, dk, dv, dg


def test_noalloc_forward_equals_vsa_fwd_on_two_calls():
    # first call: video tiles, top-k, gate, training (saved state written)
    big = build_case("noalloc_big", dtype="bf16", layout="bshd", B=1, Hq=4, Hkv=2, D=128,
                     q_var=[256] * 5 + [100], kv_var=[256, 64, 256, 256, 173, 256, 16],
                     topk=3, map_kind="none", gate_mode="per_token", seed=51)
    print(f"[{big.name}] Hq={big.Hq} Sq={big.Sq} Skv={big.Skv}", flush=True)
    d, p, ref, new = _both(big, training=True)
    for a, b in zip(_grads(big, d, p, ref), _grads(big, d, p, new)):
        assert torch.equal(a, b)
    # second call, smaller: a caller map, inference (no saved state)
    small = make_case("c1_vsa256_tiny", layout="bhsd")
    print(f"[{small.name}] Hq={small.Hq} Sq={small.Sq} Skv={small.Skv}", flush=True)
    _both(small, training=False)
