"""The C-ABI library on the host: it loads, exports every entry point that
include/vsa.h declares, and its host-only calls (argument checks, buffer
sizes) behave as documented. No compute entry point is called here."""

from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

import bwd_block_map_amd as vsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "vsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_entry_point():
    names = _declared()
    assert {"vsa_fwd", "vsa_bwd", "block_map_to_index", "vsa_sizes", "vsa_validate"} <= set(names)
    lib = ctypes.CDLL(vsa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    assert set(vsa.EXPORTS) == set(names)
    assert vsa.vsa_abi_version() == vsa.ABI_VERSION


def _prob(**kw):
    base = dict(dtype=torch.bfloat16, layout="bhsd", B=1, Hq=2, Hkv=2, Sq=768, Skv=1024, D=128,
                q_block=256, kv_block=256)
    base.update(kw)
    return vsa.make_problem(**base)


def test_validate_accepts_the_workload_shapes():
    vsa.vsa_validate(_prob())
    vsa.vsa_validate(_prob(layout="bshd", Hq=40, Hkv=40, Sq=368640, Skv=368640, topk=144,
                           gate_mode="per_token"))
    vsa.vsa_validate(_prob(dtype=torch.float16, B=2, Hq=8, Hkv=8, Sq=4096, Skv=4096,
                           q_block=128, kv_block=128))
    # the Ascend page's [8, 128] block shape, and [16, 128]
    vsa.vsa_validate(_prob(Sq=256, Skv=256, q_block=8, kv_block=128))
    vsa.vsa_validate(_prob(Sq=256, Skv=256, q_block=16, kv_block=128))
    # KV blocks of any multiple of 64 keys, Q blocks of any multiple of 32 rows
    for qb, kb in [(64, 64), (96, 192), (32, 320), (128, 512)]:
        vsa.vsa_validate(_prob(Sq=1024, Skv=1024, q_block=qb, kv_block=kb))


def _code(p):
    with pytest.raises(vsa.VsaError) as e:
        vsa.vsa_validate(p)
    return e.value.code, e.value.msg


def test_validate_rejects_bad_problems_with_messages():
    fake = torch.zeros(4, dtype=torch.int32)  # host tensor: only its address is recorded
    c, m = _code(_prob(layout="tnd", Sq=30, Skv=40, max_seqlen_q=30, max_seqlen_kv=40,
                       q_block=128, kv_block=128, cu_seqlens_kv=fake))
    assert c == vsa.ERR_INVALID_ARG and m == "actual_seq_lengths must be specified"
    c, m = _code(_prob(layout="tnd", Sq=30, Skv=40, max_seqlen_q=30, max_seqlen_kv=40,
                       q_block=128, kv_block=128, cu_seqlens_q=fake))
    assert c == vsa.ERR_INVALID_ARG and m == "actual_seq_lengths_kv must be specified"
    assert _code(_prob(Hq=3, Hkv=2))[0] == vsa.ERR_INVALID_ARG
    # 24-bit row offsets of the tile loads: token-major rows of 65536 heads are too long
    c, m = _code(_prob(layout="bshd", Hq=65536, Hkv=65536, Sq=256, Skv=256))
    assert c == vsa.ERR_UNSUPPORTED and "65536 heads" in m
    assert _code(_prob(D=256))[0] == vsa.ERR_UNSUPPORTED
    assert _code(_prob(D=0, scale=1.0))[0] == vsa.ERR_INVALID_ARG
    assert _code(_prob(q_block=48))[0] == vsa.ERR_UNSUPPORTED
    assert _code(_prob(Sq=240, q_block=24))[0] == vsa.ERR_UNSUPPORTED
    assert _code(_prob(scale=float("nan")))[0] == vsa.ERR_INVALID_ARG
    assert _code(_prob(scale=-1.0))[0] == vsa.ERR_INVALID_ARG
    assert _code(_prob(topk=-1))[0] == vsa.ERR_INVALID_ARG
    p = _prob()
    p.struct.Qb = 4
    assert _code(p)[0] == vsa.ERR_INVALID_ARG
    p = _prob()
    p.struct.abi_version = 99
    assert _code(p)[0] == vsa.ERR_INVALID_ARG
    c, _ = _code(_prob(layout="tnd", Sq=30, Skv=40, max_seqlen_q=30, max_seqlen_kv=40,
                       q_block=128, kv_block=128, cu_seqlens_q=fake, cu_seqlens_kv=fake, topk=2))
    assert c == vsa.ERR_UNSUPPORTED
    # the coarse kernels keep one score row of every KV tile in LDS: 39000 tiles
    # do not fit even with one Q tile per work-group (38000 do)
    vsa.vsa_validate(_prob(B=1, Hq=1, Hkv=1, Sq=256, Skv=38000 * 64, kv_block=64, topk=1))
    c, m = _code(_prob(B=1, Hq=1, Hkv=1, Sq=256, Skv=39000 * 64, kv_block=64, topk=1))
    assert c == vsa.ERR_UNSUPPORTED and "too large for the coarse kernels" in m


def test_sizes_cover_index_and_state():
    s = vsa.vsa_sizes(_prob(topk=2, gate_mode="per_token"))
    assert s["nnz_capacity"] == 1 * 2 * 3 * 2
    # saved holds both CSR directions, the pooled/coarse state and O_sel
    assert s["saved"] >= 2 * 768 * 128 * 2 + 2 * (1 * 2 * 3 + 1) * 4
    s2 = vsa.vsa_sizes(_prob())
    assert s2["nnz_capacity"] == 1 * 2 * 3 * 4
    assert s2["saved"] < s["saved"]
    big = vsa.vsa_sizes(_prob(layout="bshd", Hq=40, Hkv=40, Sq=368640, Skv=368640, topk=144,
                              gate_mode="per_token"))
    assert big["nnz_capacity"] == 40 * 1440 * 144


def test_compute_calls_reject_bad_arguments_before_launching():
    # no GPU is needed: the checks run on the host and return before any launch
    p = _prob()
    with pytest.raises(vsa.VsaError) as e:
        vsa.vsa_fwd(p, None, None, None, None, None, None, None, None, None)
    assert e.value.code == vsa.ERR_INVALID_ARG
    with pytest.raises(vsa.VsaError) as e:
        vsa.vsa_bwd(p, None, None, None, None, None, None, None, None, None, None, None, None, None)
    assert e.value.code == vsa.ERR_INVALID_ARG


def test_noalloc_forward_refuses_a_workspace_beyond_its_scratch():
    """vsa_fwd_noalloc checks the problem's forward workspace against its fixed
    scratch on the host, before it looks at any pointer or device: the 720p
    video problem (top-k map, pooled tiles, coarse output: > 64 MiB) is refused
    with VSA_ERR_WORKSPACE. The pointers are placeholders that are never read."""
    import ctypes as C
    p = _prob(layout="bshd", Hq=40, Hkv=40, Sq=368640, Skv=368640, topk=144,
              gate_mode="per_token")
    assert vsa.vsa_sizes(p)["ws_fwd"] > vsa.NOALLOC_SCRATCH_BYTES
    fake = C.c_void_p(256)
    rc = vsa.lib().vsa_fwd_noalloc(p.ref, fake, fake, fake, fake, fake, fake, fake, None,
                                   C.c_size_t(0), None)
    assert rc == vsa.ERR_WORKSPACE
    assert "scratch" in vsa.vsa_last_error()


def test_backward_flags_are_checked():
    """Unknown flag bits, and the two dK/dV grid choices together, are
    INVALID_ARG; each flag alone is accepted and only the persistent grid's
    span list adds to the backward workspace."""
    ok = [_prob(atomic_dq=a, persistent=pb) for a in (False, True) for pb in (None, True, False)]
    for p in ok:
        vsa.vsa_validate(p)
    p = _prob()
    p.struct.flags = vsa.FLAG_PERSISTENT | vsa.FLAG_NO_PERSISTENT
    assert _code(p)[0] == vsa.ERR_INVALID_ARG
    p.struct.flags = 64
    assert _code(p)[0] == vsa.ERR_INVALID_ARG
    auto, span = vsa.vsa_sizes(_prob())["ws_bwd"], vsa.vsa_sizes(_prob(persistent=False))["ws_bwd"]
    assert auto > span
    atomic = vsa.vsa_sizes(_prob(atomic_dq=True, persistent=False))["ws_bwd"]
    assert atomic >= span + 768 * 2 * 128 * 4  # the float dQ accumulator


def test_projected_gate_problem_is_checked():
    """VSA_GATE_PROJECTED needs gate_proj (16-byte aligned, [Hq*D + Hq] fp32)
    and BHSD/BSHD; gate_proj with any other gate mode is INVALID_ARG; the
    backward workspace grows by the per-row dL/dz and the per-Q-block
    partial sums of dw and db."""
    theta = torch.zeros(2 * 128 + 2, dtype=torch.float32)
    vsa.vsa_validate(_prob(gate_mode="projected", gate_proj=theta))
    vsa.vsa_validate(_prob(layout="bshd", gate_mode="projected", gate_proj=theta, topk=2))
    p = _prob(gate_mode="projected", gate_proj=theta)
    p.struct.gate_proj = None
    assert _code(p)[0] == vsa.ERR_INVALID_ARG
    p.struct.gate_proj = theta.data_ptr() + 4
    c, m = _code(p)
    assert c == vsa.ERR_INVALID_ARG and "aligned" in m
    p = _prob(gate_mode="per_token")
    p.struct.gate_proj = theta.data_ptr()
    assert _code(p)[0] == vsa.ERR_INVALID_ARG
    p = _prob(gate_mode="projected", gate_proj=theta)
    p.struct.gate_mode = 4
    assert _code(p)[0] == vsa.ERR_INVALID_ARG
    with pytest.raises(ValueError):
        _prob(gate_mode="projected", gate_proj=theta[:-1])
    tok = vsa.vsa_sizes(_prob(gate_mode="per_token"))["ws_bwd"]
    proj = vsa.vsa_sizes(_prob(gate_mode="projected", gate_proj=theta))["ws_bwd"]
    rows, blocks = 2 * 768, 2 * 3
    assert proj - tok >= 4 * (rows + blocks * 128 + blocks)


def test_per_entry_valid_counts_are_checked():
    """[B, tiles] counts set the batch strides to Qb / KVb; a stride below the
    tile count, a negative one, or one without its counts is INVALID_ARG."""
    qv = torch.full((1, 3), 256, dtype=torch.int32)
    kv = torch.full((1, 4), 256, dtype=torch.int32)
    p = _prob(q_valid=qv, kv_valid=kv)
    assert (p.struct.q_valid_batch_stride, p.struct.kv_valid_batch_stride) == (3, 4)
    vsa.vsa_validate(p)
    assert _prob(q_valid=qv[0], kv_valid=kv[0]).struct.q_valid_batch_stride == 0
    p.struct.q_valid_batch_stride = 2
    assert _code(p)[0] == vsa.ERR_INVALID_ARG
    p.struct.q_valid_batch_stride = -3
    assert _code(p)[0] == vsa.ERR_INVALID_ARG
    p = _prob()
    p.struct.kv_valid_batch_stride = 4
    c, m = _code(p)
    assert c == vsa.ERR_INVALID_ARG and "needs the counts" in m
    with pytest.raises(ValueError):
        _prob(B=2, q_valid=torch.full((3, 3), 256, dtype=torch.int32))


def test_head_dimensions_up_to_128():
    """D in 1 .. 128 is accepted (the Ascend operator takes head_dim <= 128),
    D = 129 is UNSUPPORTED; a D < 128 problem needs the D = 128 problem's
    workspaces plus room for its widened copies, and the same saved state."""
    for D in (1, 8, 64, 96, 128):
        vsa.vsa_validate(_prob(D=D))
    assert _code(_prob(D=129))[0] == vsa.ERR_UNSUPPORTED
    full = vsa.vsa_sizes(_prob(D=128, topk=2, gate_mode="per_element"))
    half = vsa.vsa_sizes(_prob(D=64, topk=2, gate_mode="per_element"))
    assert half["saved"] == full["saved"]
    q_rows, kv_rows = 1 * 768 * 2, 1 * 1024 * 2
    copies_fwd = 2 * 128 * (3 * q_rows + 2 * kv_rows)  # q, out, gate; k, v
    assert half["ws_fwd"] >= full["ws_fwd"] + copies_fwd
    assert half["ws_bwd"] >= full["ws_bwd"] + copies_fwd + 2 * 128 * (3 * q_rows + 2 * kv_rows)
