"""The forward without allocation (vsa_fwd_noalloc) and the backward captured
in one HIP graph (torch.cuda.graph) and replayed: every replay, with eager
work and synchronisations between replays, must equal the eager calls bit for
bit. The library clears its counters and accumulators with fill kernels, so
nothing it records into a graph is a memset node."""

from __future__ import annotations

import pytest
import torch

from workloads.synth import build_case

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.gpu_run import device_inputs, problem_for  # noqa: E402
import bwd_block_map_amd as vsa  # noqa: E402


def _step(p, d, buf, outs, stream=None):
    out, lse, dq, dk, dv, dg = outs
    bmap = buf.map if buf.map is not None else d["map"]
    vsa.vsa_fwd_noalloc(p, d["q"], d["k"], d["v"], bmap, d["gate"], out, lse, buf.saved,
                        stream=stream)
    vsa.vsa_bwd(p, d["q"], d["k"], d["v"], d["gate"], d["dout"], out, lse, buf.saved, dq, dk, dv,
                dg, buf.ws_bwd, stream=stream)


@pytest.mark.parametrize("persistent,atomic_dq", [(True, False), (False, True)],
                         ids=["persistent_dkdv", "atomic_dq"])
def test_forward_and_backward_replay_from_a_graph(persistent, atomic_dq):
    """Top-k, the per-token gate and GQA, with the persistent dK/dV grid (its
    item counter cleared inside the graph) or the atomic-dQ backward (its
    float accumulator cleared inside the graph)."""
    case = build_case("graph", dtype="bf16", layout="bshd", B=1, Hq=4, Hkv=2, D=128,
                      q_var=[256, 100, 256], kv_var=[256, 64, 256, 16, 256], topk=3,
                      map_kind="none", gate_mode="per_token", seed=91)
    d = device_inputs(case)
    p = problem_for(case, d, atomic_dq=atomic_dq, persistent=persistent)
    buf = vsa.Buffers(p, d["q"], training=True)

    def fresh():
        return (torch.empty_like(d["q"]), torch.empty(buf.lse.shape, dtype=torch.float32,
                                                      device="cuda"),
                torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"]),
                torch.empty_like(d["gate"]))

    ref = fresh()
    _step(p, d, buf, ref)  # eager (also looks up the scratch address)
    torch.cuda.synchronize()
    got = fresh()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(p, d, buf, got, stream=s.cuda_stream)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _step(p, d, buf, got, stream=torch.cuda.current_stream().cuda_stream)
    names = ("out", "lse", "dq", "dk", "dv", "dgate")
    for replay in range(3):
        for t in got:
            t.fill_(float("nan"))  # stale values cannot pass
        x = torch.randn(512, 512, device="cuda") @ torch.randn(512, 512, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, a, b in zip(names, ref, got):
            if n == "dq" and atomic_dq:  # float atomics: the order of the adds varies
                assert torch.allclose(a.float(), b.float(), rtol=2e-2, atol=2e-3), (replay, n)
            else:
                assert torch.equal(a, b), (replay, n)
        del x
