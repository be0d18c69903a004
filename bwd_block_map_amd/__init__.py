"""Python binding of libvsa.so, the gfx950 block-sparse attention library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/vsa.h. PyTorch provides device
memory and the current stream. Importing works without a GPU; calling a
compute entry point without the built library raises (there is no fallback).

Entry points (same names as the C ABI): vsa_validate, vsa_sizes,
block_map_to_index, vsa_fwd, vsa_fwd_noalloc, vsa_bwd, vsa_last_error,
vsa_abi_version.
"""

from __future__ import annotations

import ctypes as C
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvsa.so")

BF16, FP16 = 0, 1
BHSD, BSHD, TND = 0, 1, 2
GATE_NONE, GATE_PER_TOKEN, GATE_PER_ELEMENT, GATE_PROJECTED = 0, 1, 2, 3
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
ABI_VERSION = 4
FLAG_ATOMIC_DQ = 1
FLAG_PERSISTENT = 2
FLAG_NO_PERSISTENT = 4

EXPORTS = ("vsa_last_error", "vsa_abi_version", "vsa_validate", "vsa_sizes",
           "block_map_to_index", "vsa_fwd", "vsa_fwd_noalloc", "vsa_bwd", "vsa_profile_begin",
           "vsa_profile_end")
NOALLOC_SCRATCH_BYTES = 64 << 20  # VSA_NOALLOC_SCRATCH_BYTES
KERNELS = ("index", "pool", "coarse_fwd", "sparse_fwd", "bwd_pre", "coarse_bwd", "sparse_dkdv",
           "sparse_dq", "dq_atomic_aux", "dkdv_order", "pad")

_DTYPES = {torch.bfloat16: BF16, torch.float16: FP16}
_LAYOUTS = {"bhsd": BHSD, "bshd": BSHD, "tnd": TND}
_GATES = {"none": GATE_NONE, "per_token": GATE_PER_TOKEN, "per_element": GATE_PER_ELEMENT,
          "projected": GATE_PROJECTED}


class VsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"vsa error {code}: {msg}")
        self.code = code
        self.msg = msg


class VsaProblem(C.Structure):
    _fields_ = [
        ("abi_version", C.c_int32), ("dtype", C.c_int32), ("layout", C.c_int32),
        ("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32),
        ("Sq", C.c_int32), ("Skv", C.c_int32), ("D", C.c_int32),
        ("q_block", C.c_int32), ("kv_block", C.c_int32), ("Qb", C.c_int32), ("KVb", C.c_int32),
        ("q_valid", C.c_void_p), ("kv_valid", C.c_void_p),
        ("cu_seqlens_q", C.c_void_p), ("cu_seqlens_kv", C.c_void_p),
        ("max_seqlen_q", C.c_int32), ("max_seqlen_kv", C.c_int32),
        ("scale", C.c_float), ("topk", C.c_int32), ("gate_mode", C.c_int32),
        ("map_batch_stride", C.c_int64), ("flags", C.c_int32), ("gate_proj", C.c_void_p),
        ("q_valid_batch_stride", C.c_int64), ("kv_valid_batch_stride", C.c_int64),
    ]


_LIB = None


def lib():
    """The loaded library; raises when it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bwd_block_map_amd.build` (no CPU fallback exists)")
        L = C.CDLL(LIB_PATH)
        L.vsa_last_error.restype = C.c_char_p
        for name in ("vsa_abi_version", "vsa_validate", "vsa_sizes", "block_map_to_index",
                     "vsa_fwd", "vsa_fwd_noalloc", "vsa_bwd", "vsa_profile_begin",
                     "vsa_profile_end"):
            getattr(L, name).restype = C.c_int
        _LIB = L
    return _LIB


def vsa_last_error() -> str:
    return lib().vsa_last_error().decode()


def vsa_abi_version() -> int:
    return lib().vsa_abi_version()


def _check(rc: int):
    if rc != OK:
        raise VsaError(rc, vsa_last_error())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return C.c_void_p(stream)
    if torch.cuda.is_available():
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return None


@dataclass
class Problem:
    """A vsa_problem plus the device tensors it points to (kept alive)."""
    struct: VsaProblem
    keep: tuple = ()

    @property
    def ref(self):
        return C.byref(self.struct)

    def __getattr__(self, name):
        return getattr(self.struct, name)


def make_problem(*, dtype: torch.dtype, layout: str, B: int, Hq: int, Hkv: int, Sq: int,
                 Skv: int, D: int = 128, q_block: int, kv_block: int,
                 q_valid: Optional[torch.Tensor] = None, kv_valid: Optional[torch.Tensor] = None,
                 cu_seqlens_q: Optional[torch.Tensor] = None,
                 cu_seqlens_kv: Optional[torch.Tensor] = None, max_seqlen_q: int = 0,
                 max_seqlen_kv: int = 0, scale: Optional[float] = None, topk: int = 0,
                 gate_mode: str = "none", map_batch_stride: Optional[int] = None,
                 atomic_dq: bool = False, persistent: Optional[bool] = None,
                 gate_proj: Optional[torch.Tensor] = None) -> Problem:
    """Fill a vsa_problem. q_valid / kv_valid / cu_seqlens are int32 device tensors;
    q_valid / kv_valid are [Qb] / [KVb] (one set for every batch entry) or
    [B, Qb] / [B, KVb] (per entry).
    gate_proj (gate_mode "projected"): the gate's parameters, a contiguous
    float32 device tensor [w (Hq x D) | b (Hq)].
    atomic_dq selects the backward that adds dQ inside the KV-owned pass
    (VSA_FLAG_ATOMIC_DQ). persistent: None lets the library choose the
    dK/dV grid, True forces the persistent longest-first grid
    (VSA_FLAG_PERSISTENT), False one work-group per span
    (VSA_FLAG_NO_PERSISTENT)."""
    lay = _LAYOUTS[layout]
    if lay == TND:
        Qb = -(-max_seqlen_q // q_block)
        KVb = -(-max_seqlen_kv // kv_block)
    else:
        Qb = -(-Sq // q_block)
        KVb = -(-Skv // kv_block)
    if map_batch_stride is None:
        map_batch_stride = Hq * Qb * KVb
    keep = tuple(t for t in (q_valid, kv_valid, cu_seqlens_q, cu_seqlens_kv) if t is not None)
    for t in keep:
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("valid counts and cu_seqlens must be contiguous int32 tensors")
    if gate_proj is not None:
        if gate_proj.dtype != torch.float32 or not gate_proj.is_contiguous() \
                or gate_proj.numel() != Hq * D + Hq:
            raise ValueError(f"gate_proj must be a contiguous float32 tensor of Hq*D+Hq = "
                             f"{Hq * D + Hq} elements")
        keep = keep + (gate_proj,)
    strides = []
    for t, n, name in ((q_valid, Qb, "q_valid"), (kv_valid, KVb, "kv_valid")):
        if t is not None and t.dim() == 2:
            if tuple(t.shape) != (B, n):
                raise ValueError(f"{name} must be [{n}] or [{B}, {n}], got {tuple(t.shape)}")
            strides.append(n)
            continue
        if t is not None and t.numel() != n:
            raise ValueError(f"{name} needs {n} entries, got {t.numel()}")
        strides.append(0)
    for t, total, mx, name in ((cu_seqlens_q, Sq, max_seqlen_q, "cu_seqlens_q"),
                               (cu_seqlens_kv, Skv, max_seqlen_kv, "cu_seqlens_kv")):
        if t is not None and lay == TND and t.is_cuda:
            # the kernels index packed rows through these offsets: check them once here
            c = t.cpu()
            if c.numel() != B + 1 or int(c[0]) != 0 or int(c[-1]) != total:
                raise ValueError(f"{name} must be [B+1] offsets from 0 to {total}")
            lens = c[1:] - c[:-1]
            if bool((lens < 0).any()) or int(lens.max()) > mx:
                raise ValueError(f"{name}: lengths must be in [0, max_seqlen={mx}]")
    s = VsaProblem(
        abi_version=ABI_VERSION, dtype=_DTYPES[dtype], layout=lay, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq,
        Skv=Skv, D=D, q_block=q_block, kv_block=kv_block, Qb=Qb, KVb=KVb,
        q_valid=None if q_valid is None else q_valid.data_ptr(),
        kv_valid=None if kv_valid is None else kv_valid.data_ptr(),
        cu_seqlens_q=None if cu_seqlens_q is None else cu_seqlens_q.data_ptr(),
        cu_seqlens_kv=None if cu_seqlens_kv is None else cu_seqlens_kv.data_ptr(),
        max_seqlen_q=max_seqlen_q, max_seqlen_kv=max_seqlen_kv,
        scale=1.0 / math.sqrt(D) if scale is None else float(scale), topk=topk,
        gate_mode=_GATES[gate_mode], map_batch_stride=map_batch_stride,
        flags=(FLAG_ATOMIC_DQ if atomic_dq else 0)
        | {None: 0, True: FLAG_PERSISTENT, False: FLAG_NO_PERSISTENT}[persistent],
        gate_proj=None if gate_proj is None else gate_proj.data_ptr(),
        q_valid_batch_stride=strides[0], kv_valid_batch_stride=strides[1])
    return Problem(s, keep)


def vsa_validate(p: Problem) -> None:
    _check(lib().vsa_validate(p.ref))


def vsa_sizes(p: Problem) -> dict:
    f, b, s = C.c_size_t(), C.c_size_t(), C.c_size_t()
    n = C.c_int64()
    _check(lib().vsa_sizes(p.ref, C.byref(f), C.byref(b), C.byref(s), C.byref(n)))
    return {"ws_fwd": f.value, "ws_bwd": b.value, "saved": s.value, "nnz_capacity": n.value}


def block_map_to_index(p: Problem, block_map: torch.Tensor, kv_owned: bool, row_ptr: torch.Tensor,
                       col_idx: torch.Tensor, col_capacity: int, ws: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    if block_map is not None:
        n = (p.Hq * p.Qb * p.KVb) * (1 if p.map_batch_stride == 0 else p.B)
        _expect(block_map, n, "block_map", torch.uint8)
        _expect(row_ptr, p.B * p.Hq * (p.KVb if kv_owned else p.Qb) + 1, "row_ptr", torch.int32)
        if col_idx is None or col_idx.numel() < col_capacity or col_idx.dtype != torch.int32:
            raise ValueError("col_idx must be an int32 tensor of at least col_capacity elements")
    _check(lib().block_map_to_index(
        p.ref, _ptr(block_map), C.c_int(1 if kv_owned else 0), _ptr(row_ptr), _ptr(col_idx),
        C.c_int64(col_capacity), _ptr(ws), C.c_size_t(0 if ws is None else ws.numel()),
        _stream(stream)))


def _numel_q(p):
    return (p.Sq if p.layout == TND else p.B * p.Sq) * p.Hq * p.D


def _numel_kv(p):
    return (p.Skv if p.layout == TND else p.B * p.Skv) * p.Hkv * p.D


def _expect(t, n, name, dtype=None):
    """Host-side size check: a buffer that does not match the problem never
    reaches a kernel."""
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.numel() != n:
        raise ValueError(f"{name} has {t.numel()} elements, the problem needs {n}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _check_tensors(p, q, k, v, gate, qlike=(), kvlike=(), lse=None, block_map=None):
    for t in p.keep:
        if not t.is_cuda:
            raise ValueError("valid counts, cu_seqlens and gate_proj must be device tensors")
    dt = torch.bfloat16 if p.dtype == BF16 else torch.float16
    nq, nk = _numel_q(p), _numel_kv(p)
    _expect(q, nq, "q", dt)
    _expect(k, nk, "k", dt)
    _expect(v, nk, "v", dt)
    for name, t in qlike:
        _expect(t, nq, name, dt)
    for name, t in kvlike:
        _expect(t, nk, name, dt)
    if gate is not None:
        per_tok = p.gate_mode in (GATE_PER_TOKEN, GATE_PROJECTED)
        _expect(gate, nq // p.D if per_tok else nq, "gate", dt)
    if lse is not None:
        _expect(lse, (p.Sq if p.layout == TND else p.B * p.Sq) * p.Hq, "lse", torch.float32)
    if block_map is not None:
        n = (p.Hq * p.Qb * p.KVb) * (1 if p.map_batch_stride == 0 else p.B)
        _expect(block_map, n, "block_map", torch.uint8)


def vsa_fwd(p: Problem, q, k, v, block_map, gate, out, lse, saved, ws, stream=None) -> None:
    if q is not None:
        _check_tensors(p, q, k, v, gate, qlike=(("out", out),), lse=lse, block_map=block_map)
    _check(lib().vsa_fwd(
        p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(block_map), _ptr(gate), _ptr(out), _ptr(lse),
        _ptr(saved), C.c_size_t(0 if saved is None else saved.numel() * saved.element_size()),
        _ptr(ws), C.c_size_t(0 if ws is None else ws.numel() * ws.element_size()),
        _stream(stream)))


def vsa_fwd_noalloc(p: Problem, q, k, v, block_map, gate, out, lse, saved, stream=None) -> None:
    """vsa_fwd with the library's own device scratch as the forward workspace
    (no allocation in the call; problems whose workspace exceeds
    NOALLOC_SCRATCH_BYTES are refused with ERR_WORKSPACE)."""
    if q is not None:
        _check_tensors(p, q, k, v, gate, qlike=(("out", out),), lse=lse, block_map=block_map)
    _check(lib().vsa_fwd_noalloc(
        p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(block_map), _ptr(gate), _ptr(out), _ptr(lse),
        _ptr(saved), C.c_size_t(0 if saved is None else saved.numel() * saved.element_size()),
        _stream(stream)))


def vsa_bwd(p: Problem, q, k, v, gate, dout, out, lse, saved, dq, dk, dv, dgate, ws,
            stream=None) -> None:
    if q is not None:
        _check_tensors(p, q, k, v, gate, qlike=(("dout", dout), ("out", out), ("dq", dq)),
                       kvlike=(("dk", dk), ("dv", dv)), lse=lse)
        if dgate is not None and p.gate_mode == GATE_PROJECTED:
            _expect(dgate, p.Hq * p.D + p.Hq, "dgate", torch.float32)
        elif dgate is not None:
            if gate is None:
                raise ValueError("dgate needs the gate it is the gradient of")
            _expect(dgate, gate.numel(), "dgate", gate.dtype)
    _check(lib().vsa_bwd(
        p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(dout), _ptr(out), _ptr(lse),
        _ptr(saved), C.c_size_t(0 if saved is None else saved.numel() * saved.element_size()),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgate),
        _ptr(ws), C.c_size_t(0 if ws is None else ws.numel() * ws.element_size()),
        _stream(stream)))


def vsa_profile_begin() -> None:
    _check(lib().vsa_profile_begin())


def vsa_profile_end() -> dict:
    """{kernel name: (total ms, launches)} of the launches since vsa_profile_begin."""
    n = len(KERNELS)
    ms = (C.c_double * n)()
    cnt = (C.c_int64 * n)()
    _check(lib().vsa_profile_end(ms, cnt, C.c_int(n)))
    return {KERNELS[i]: (ms[i], cnt[i]) for i in range(n)}


# ---------------------------------------------------------------------------
# Buffer allocation with torch (device memory only; no computation)
# ---------------------------------------------------------------------------

class Buffers:
    """Caller-owned buffers of one problem: out, lse, saved and workspaces."""

    def __init__(self, p: Problem, q: torch.Tensor, training: bool = True,
                 gate: Optional[torch.Tensor] = None):
        sz = vsa_sizes(p)
        dev = q.device
        self.sizes = sz
        self.out = torch.empty_like(q)
        lse_shape = (p.Hq, p.Sq) if p.layout == TND else (p.B, p.Hq, p.Sq)
        self.lse = torch.empty(lse_shape, dtype=torch.float32, device=dev)
        self.ws_fwd = torch.empty(max(sz["ws_fwd"], 1), dtype=torch.uint8, device=dev)
        self.ws_bwd = torch.empty(max(sz["ws_bwd"], 1), dtype=torch.uint8, device=dev)
        self.saved = torch.empty(max(sz["saved"], 1), dtype=torch.uint8, device=dev) \
            if training else None
        self.map = None
        if p.topk > 0:
            self.map = torch.empty((p.B, p.Hq, p.Qb, p.KVb), dtype=torch.uint8, device=dev)


# PyTorch entry points (autograd over vsa_fwd / vsa_bwd)
from .torch_api import (attention, block_sparse_attn, block_sparse_attn_tnd,  # noqa: E402
                        video_sparse_attn, video_sparse_attn_bshd)
