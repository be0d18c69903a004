"""CPU oracle for block-sparse attention: TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The GPU library never calls it and shares no code with it.

`oracle.cpp` holds the arithmetic (plain loops, float or double); this module
only builds it with g++, marshals arguments with ctypes and converts the seeded
workload tensors (exact bf16/fp16 values) to numpy arrays.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "oracle.cpp")
_LIB_PATH = os.path.join(_DIR, "liboracle.so")
# ORACLE_LIB names another build of oracle.cpp to load instead (the mutation
# test points it at copies with a planted mistake); it is never rebuilt here.
_LIB_OVERRIDE = os.environ.get("ORACLE_LIB")
_LIB = None

_LAYOUT = {"bhsd": 0, "bshd": 1, "tnd": 2}
_GATE = {"none": 0, "per_token": 1, "per_element": 2, "projected": 3}


class OracleProblem(C.Structure):
    _fields_ = [
        ("layout", C.c_int32), ("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32),
        ("Sq", C.c_int32), ("Skv", C.c_int32), ("D", C.c_int32),
        ("q_block", C.c_int32), ("kv_block", C.c_int32), ("Qb", C.c_int32), ("KVb", C.c_int32),
        ("q_var", C.POINTER(C.c_int32)), ("kv_var", C.POINTER(C.c_int32)),
        ("q_lens", C.POINTER(C.c_int32)), ("kv_lens", C.POINTER(C.c_int32)),
        ("scale", C.c_double), ("gate_mode", C.c_int32), ("threads", C.c_int32),
        ("q_var_bstride", C.c_int64), ("kv_var_bstride", C.c_int64),
    ]


def build(verbose: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile liboracle.so (plain g++, OpenMP, no target-specific flags so the
    binary runs on any x86-64 host). src / out let a test build a copy."""
    cmd = ["g++", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c++17", src, "-o", out + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + r.stderr)
    os.replace(out + ".tmp", out)
    if verbose:
        print(" ".join(cmd))
    return out


def lib():
    global _LIB
    if _LIB is None and _LIB_OVERRIDE:
        _LIB = C.CDLL(_LIB_OVERRIDE)
    if _LIB is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _LIB = C.CDLL(_LIB_PATH)
    return _LIB


def _ptr(a: Optional[np.ndarray], ct):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.POINTER(ct))


def _bstride(var) -> int:
    return 0 if var is None or np.ndim(var) < 2 else int(np.shape(var)[1])


class Prob:
    """ctypes problem for a workload case, keeping its int arrays alive."""

    def __init__(self, case, threads: int = 0):
        self.case = case
        self.keep = []

        def arr(x):
            if x is None:
                return None
            a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
            self.keep.append(a)
            return a.ctypes.data_as(C.POINTER(C.c_int32))

        self.s = OracleProblem(
            layout=_LAYOUT[case.layout], B=case.B, Hq=case.Hq, Hkv=case.Hkv, Sq=case.Sq,
            Skv=case.Skv, D=case.D, q_block=case.q_block, kv_block=case.kv_block, Qb=case.Qb,
            KVb=case.KVb, q_var=arr(case.q_var), kv_var=arr(case.kv_var), q_lens=arr(case.q_lens),
            kv_lens=arr(case.kv_lens), scale=float(case.scale), gate_mode=_GATE[case.gate_mode],
            threads=int(threads),
            # [B, tiles] counts: one row per batch entry
            q_var_bstride=_bstride(case.q_var), kv_var_bstride=_bstride(case.kv_var))

    @property
    def ref(self):
        return C.byref(self.s)


def _np(t, dt):
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return np.ascontiguousarray(t.astype(dt))
    return np.ascontiguousarray(t.detach().float().cpu().numpy().astype(dt))


def _sfx(dt):
    return "f64" if dt == np.float64 else "f32"


def _ct(dt):
    return C.c_double if dt == np.float64 else C.c_float


class Oracle:
    """Oracle evaluation of one workload case in float32 or float64."""

    def __init__(self, case, dtype=np.float64, threads: int = 0, tensors=None):
        self.case = case
        self.dt = dtype
        self.P = Prob(case, threads)
        self.L = lib()
        src = tensors if tensors is not None else dict(
            q=case.q, k=case.k, v=case.v, dout=case.dout, gate=case.gate)
        self.q = _np(src["q"], dtype)
        self.k = _np(src["k"], dtype)
        self.v = _np(src["v"], dtype)
        self.dout = _np(src["dout"], dtype)
        self.gate = _np(src.get("gate"), dtype)
        self._map = None
        self._pooled = None
        self._coarse = None

    # -- helpers -------------------------------------------------------------
    def _f(self, name):
        return getattr(self.L, f"oracle_{name}_{_sfx(self.dt)}")

    def _p(self, a):
        return _ptr(a, _ct(self.dt))

    # -- pooling / top-k / compression ----------------------------------------
    def pooled(self):
        if self._pooled is None:
            c = self.case
            qc = np.zeros((c.B, c.Hq, c.Qb, c.D), self.dt)
            kc = np.zeros((c.B, c.Hkv, c.KVb, c.D), self.dt)
            vc = np.zeros((c.B, c.Hkv, c.KVb, c.D), self.dt)
            self._f("pool")(self.P.ref, self._p(self.q), self._p(self.k), self._p(self.v),
                            self._p(qc), self._p(kc), self._p(vc))
            self._pooled = (qc, kc, vc)
        return self._pooled

    def coarse_scores(self):
        c = self.case
        qc, kc, _ = self.pooled()
        out = np.zeros((c.B, c.Hq, c.Qb, c.KVb), self.dt)
        self._f("coarse_scores")(self.P.ref, self._p(qc), self._p(kc), self._p(out))
        return out

    def topk_map(self, topk: Optional[int] = None):
        c = self.case
        qc, kc, _ = self.pooled()
        m = np.zeros((c.B, c.Hq, c.Qb, c.KVb), np.uint8)
        self._f("topk")(self.P.ref, self._p(qc), self._p(kc), int(c.topk if topk is None else topk),
                        _ptr(m, C.c_uint8))
        return m

    def coarse(self):
        if self._coarse is None:
            c = self.case
            qc, kc, vc = self.pooled()
            oc = np.zeros((c.B, c.Hq, c.Qb, c.D), self.dt)
            lc = np.zeros((c.B, c.Hq, c.Qb), self.dt)
            self._f("coarse_fwd")(self.P.ref, self._p(qc), self._p(kc), self._p(vc), self._p(oc),
                                  self._p(lc))
            self._coarse = (oc, lc)
        return self._coarse

    def block_map(self) -> np.ndarray:
        """The selection: the case's map, or the oracle's own pooled-score top-k."""
        if self._map is None:
            c = self.case
            if c.topk > 0:
                self._map = self.topk_map()
            else:
                self._map = np.ascontiguousarray(c.block_map.numpy().astype(np.uint8))
        return self._map

    def set_map(self, m: np.ndarray):
        self._map = np.ascontiguousarray(m.astype(np.uint8))

    # -- attention -------------------------------------------------------------
    def lse_shape(self):
        c = self.case
        return (c.Hq, c.Sq) if c.layout == "tnd" else (c.B, c.Hq, c.Sq)

    def fwd(self, heads: Optional[Sequence] = None):
        """out, O_sel and lse (natural log) for all heads, or for the listed
        (b, h) heads (other entries stay zero)."""
        c = self.case
        m = self.block_map()
        oc = self.coarse()[0] if c.gate_mode != "none" else None
        hm = None
        if heads is not None:
            hm = np.zeros(c.B * c.Hq, np.uint8)
            for b, h in heads:
                hm[b * c.Hq + h] = 1
        out = np.zeros(self.q.shape, self.dt)
        osel = np.zeros(self.q.shape, self.dt)
        lse = np.zeros(self.lse_shape(), self.dt)
        self._f("fwd")(self.P.ref, self._p(self.q), self._p(self.k), self._p(self.v),
                       self._p(self.gate), _ptr(m, C.c_uint8), self._p(oc), _ptr(hm, C.c_uint8),
                       self._p(out), self._p(osel), self._p(lse))
        return out, osel, lse

    def gate_values(self):
        """The projected gate of every token, in the per-token gate layout
        ([B, Hq, S] for BHSD, [B, S, Hq] for BSHD)."""
        c = self.case
        assert c.gate_mode == "projected"
        shape = (c.B, c.Hq, c.Sq) if c.layout == "bhsd" else (c.B, c.Sq, c.Hq)
        out = np.zeros(shape, self.dt)
        self._f("gate_values")(self.P.ref, self._p(self.q), self._p(self.gate), self._p(out))
        return out

    def fwd_rows(self, rows: np.ndarray):
        """rows: int32 [n, 3] of (b, h, s). Returns out [n, D], lse [n]."""
        c = self.case
        rows = np.ascontiguousarray(rows.astype(np.int32))
        m = self.block_map()
        oc = self.coarse()[0] if c.gate_mode != "none" else None
        out = np.zeros((len(rows), c.D), self.dt)
        lse = np.zeros((len(rows),), self.dt)
        self._f("fwd_rows")(self.P.ref, self._p(self.q), self._p(self.k), self._p(self.v),
                            self._p(self.gate), _ptr(m, C.c_uint8), self._p(oc),
                            C.c_int64(len(rows)), _ptr(rows, C.c_int32), self._p(out), self._p(lse))
        return out, lse

    def bwd(self, groups: Optional[Sequence] = None):
        """dq, dk, dv, dgate of L = sum(out * dO), for all heads or for the
        listed (b, kv_head) groups."""
        c = self.case
        m = self.block_map()
        gm = None
        if groups is not None:
            gm = np.zeros(c.B * c.Hkv, np.uint8)
            for b, hk in groups:
                gm[b * c.Hkv + hk] = 1
        dq = np.zeros(self.q.shape, self.dt)
        dk = np.zeros(self.k.shape, self.dt)
        dv = np.zeros(self.v.shape, self.dt)
        dg = np.zeros(self.gate.shape, self.dt) if self.gate is not None else None
        self._f("bwd")(self.P.ref, self._p(self.q), self._p(self.k), self._p(self.v),
                       self._p(self.gate), self._p(self.dout), _ptr(m, C.c_uint8),
                       _ptr(gm, C.c_uint8), self._p(dq), self._p(dk), self._p(dv), self._p(dg))
        return dq, dk, dv, dg

    def dq_rows(self, rows: np.ndarray):
        c = self.case
        rows = np.ascontiguousarray(rows.astype(np.int32))
        m = self.block_map()
        out = np.zeros((len(rows), c.D), self.dt)
        self._f("dq_rows")(self.P.ref, self._p(self.q), self._p(self.k), self._p(self.v),
                           self._p(self.gate), self._p(self.dout), _ptr(m, C.c_uint8),
                           C.c_int64(len(rows)), _ptr(rows, C.c_int32), self._p(out))
        return out


def _dkdv_tiles(self, tiles: np.ndarray):
    """dk, dv [n, kv_block, D] of sampled KV tiles, rows of (b, kv_head, j)."""
    c = self.case
    tiles = np.ascontiguousarray(np.asarray(tiles, np.int32).reshape(-1, 3))
    m = self.block_map()
    dk = np.zeros((len(tiles), c.kv_block, c.D), self.dt)
    dv = np.zeros((len(tiles), c.kv_block, c.D), self.dt)
    self._f("dkdv_tiles")(self.P.ref, self._p(self.q), self._p(self.k), self._p(self.v),
                          self._p(self.gate), self._p(self.dout), _ptr(m, C.c_uint8),
                          C.c_int64(len(tiles)), _ptr(tiles, C.c_int32), self._p(dk), self._p(dv))
    return dk, dv


Oracle.dkdv_tiles = _dkdv_tiles


def block_index(case, block_map: np.ndarray, kv_owned: bool):
    """Brute-force CSR of the live blocks: (row_ptr int32, col int32)."""
    P = Prob(case)
    rows = case.B * case.Hq * (case.KVb if kv_owned else case.Qb)
    cap = case.B * case.Hq * case.Qb * case.KVb
    rp = np.zeros(rows + 1, np.int32)
    col = np.zeros(max(cap, 1), np.int32)
    m = np.ascontiguousarray(block_map.astype(np.uint8))
    fn = lib().oracle_block_index
    fn.restype = C.c_int64
    nnz = fn(P.ref, _ptr(m, C.c_uint8), C.c_int32(1 if kv_owned else 0), _ptr(rp, C.c_int32),
             _ptr(col, C.c_int32), C.c_int64(cap))
    assert nnz >= 0
    return rp, col[:nnz].copy()
