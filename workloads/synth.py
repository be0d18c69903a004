"""Seeded synthetic workloads for block-sparse attention.

Every tensor is drawn from a torch generator seeded per case, in a fixed
order (q, k, v, dO, gate, then the block map and lengths), rounded to the
case's dtype, and (for the video tiles) zeroed in the padded tail slots of
each tile, because callers scatter tokens into a zeroed tile buffer
(FastVideo test_vsa256_backward.py page, `_zero_pad_tail`).

The shapes follow the source pages:
  * VSA-256 parity cases of the FastVideo test page (B=1, H=2, D=128, bf16,
    256-token tiles with per-tile valid counts `q_var` / `kv_var`);
  * the Ascend op-plugin test page's BNSD and TND cases (fp16/bf16, D=128,
    [128,128] blocks, GQA, variable lengths, its deterministic sparse mask);
  * the video-shaped workloads: latent grids cut into (4,8,8) tiles of 256
    tokens, the last temporal / spatial tiles partial.

Nothing here evaluates attention, pooling, top-k or the block index; the
valid-count arrays of the video cases are input geometry (how many latent
tokens fall in each tile), not results of the method.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np
import torch

_DT = {"bf16": torch.bfloat16, "fp16": torch.float16}


@dataclass
class Case:
    name: str
    dtype: str                 # "bf16" | "fp16"
    layout: str                # "bhsd" | "bshd" | "tnd"
    B: int
    Hq: int
    Hkv: int
    Sq: int                    # rows per batch (TND: total packed q tokens)
    Skv: int                   # keys per batch (TND: total packed kv tokens)
    D: int
    q_block: int
    kv_block: int
    Qb: int                    # Q blocks per batch (TND: of the longest sequence)
    KVb: int
    scale: float
    topk: int = 0              # 0: the block map below is the selection
    gate_mode: str = "none"    # "none" | "per_token" | "per_element" | "projected"
    q_var: Optional[np.ndarray] = None    # int32 [Qb] (or [B, Qb]) valid tokens per Q tile
    kv_var: Optional[np.ndarray] = None   # int32 [KVb] (or [B, KVb]) valid tokens per KV tile
    q_lens: Optional[List[int]] = None    # TND per-sequence lengths
    kv_lens: Optional[List[int]] = None
    block_map: Optional[torch.Tensor] = None  # uint8 [B, Hq, Qb, KVb], CPU
    q: torch.Tensor = None
    k: torch.Tensor = None
    v: torch.Tensor = None
    dout: torch.Tensor = None
    gate: Optional[torch.Tensor] = None
    meta: Dict[str, object] = field(default_factory=dict)

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DT[self.dtype]


def _ceil(a: int, b: int) -> int:
    return (a + b - 1) // b


def vsa_tile_counts(latent: Sequence[int], tile: Sequence[int] = (4, 8, 8)) -> np.ndarray:
    """Tokens of a (T, H, W) latent grid that land in each (4, 8, 8) tile.

    Tiles are ordered (t, h, w) row-major; edge tiles hold fewer tokens.
    """
    grid = [_ceil(n, t) for n, t in zip(latent, tile)]
    per_axis = []
    for n, t, g in zip(latent, tile, grid):
        per_axis.append(np.array([min(t, n - i * t) for i in range(g)], dtype=np.int64))
    counts = per_axis[0][:, None, None] * per_axis[1][None, :, None] * per_axis[2][None, None, :]
    return counts.reshape(-1).astype(np.int32)


def _randn(gen: torch.Generator, shape, dtype: torch.dtype, device) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(dtype)


def _tile_valid_mask(var: np.ndarray, block: int, layout: str, device) -> torch.Tensor:
    """1 where a slot of the tile buffer holds a token, broadcastable to the
    tensor layout ([B,H,S,D] or [B,S,H,D]); var is [tiles] or [B, tiles]."""
    cnt = torch.as_tensor(var, device=device).to(torch.int64)
    cnt = cnt.view(1, -1) if cnt.dim() == 1 else cnt
    idx = torch.arange(block, device=device).view(1, 1, -1)
    valid = (idx < cnt.unsqueeze(-1)).reshape(cnt.shape[0], -1)
    if layout == "bhsd":
        return valid.view(cnt.shape[0], 1, -1, 1)
    return valid.view(cnt.shape[0], -1, 1, 1)


def build_case(
    name: str,
    *,
    dtype: str = "bf16",
    layout: str = "bhsd",
    B: int = 1,
    Hq: int = 2,
    Hkv: Optional[int] = None,
    D: int = 128,
    q_block: int = 256,
    kv_block: int = 256,
    Sq: Optional[int] = None,
    Skv: Optional[int] = None,
    q_var: Optional[Sequence[int]] = None,
    kv_var: Optional[Sequence[int]] = None,
    q_lens: Optional[Sequence[int]] = None,
    kv_lens: Optional[Sequence[int]] = None,
    topk: int = 0,
    map_kind: str = "bernoulli",
    map_p: float = 0.5,
    map_per_row: int = 2,
    map_fn: Optional[Callable] = None,
    gate_mode: str = "none",
    gate_kind: str = "sigmoid",
    pad_inputs: bool = True,
    pad_dout: bool = True,
    scale: Optional[float] = None,
    seed: int = 42,
    device="cpu",
) -> Case:
    """Draw one case. Exactly one of (Sq/Skv, q_var/kv_var, q_lens/kv_lens)
    describes the sequence geometry:
      * q_var / kv_var: video tiles, Sq = tiles * q_block (tile buffer); one
        count per tile ([tiles]) or per batch entry and tile ([B, tiles]);
      * q_lens / kv_lens: packed TND sequences;
      * Sq / Skv: plain BHSD/BSHD sequences (the last block may be partial).
    map_kind: "bernoulli" (p = map_p, at least one block per Q block),
    "per_row" (map_per_row distinct blocks per Q block, uniform), "ones",
    "custom" (map_fn(case) -> uint8 [B,Hq,Qb,KVb]) or "none" (topk > 0).
    """
    Hkv = Hq if Hkv is None else Hkv
    tdt = _DT[dtype]
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    if q_lens is not None:
        assert layout == "tnd"
        q_lens = [int(x) for x in q_lens]
        kv_lens = [int(x) for x in kv_lens]
        B = len(q_lens)
        Sq, Skv = sum(q_lens), sum(kv_lens)
        Qb, KVb = _ceil(max(q_lens), q_block), _ceil(max(kv_lens), kv_block)
    elif q_var is not None:
        q_var = np.asarray(q_var, dtype=np.int32)
        kv_var = np.asarray(kv_var, dtype=np.int32)
        for var in (q_var, kv_var):
            assert var.ndim == 1 or var.shape[0] == B, "per-entry counts need one row per batch entry"
        Qb, KVb = q_var.shape[-1], kv_var.shape[-1]
        Sq, Skv = Qb * q_block, KVb * kv_block
    else:
        Skv = Sq if Skv is None else Skv
        Qb, KVb = _ceil(Sq, q_block), _ceil(Skv, kv_block)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)

    if layout == "bhsd":
        qs, ks = (B, Hq, Sq, D), (B, Hkv, Skv, D)
    elif layout == "bshd":
        qs, ks = (B, Sq, Hq, D), (B, Skv, Hkv, D)
    else:
        qs, ks = (Sq, Hq, D), (Skv, Hkv, D)
    q = _randn(gen, qs, tdt, device)
    k = _randn(gen, ks, tdt, device)
    v = _randn(gen, ks, tdt, device)
    dout = _randn(gen, qs, tdt, device)
    gate = None
    if gate_mode == "projected":
        # parameters of the projected gate sigmoid(<q, w_h> + b_h), fp32
        # [w (Hq x D) | b (Hq)]; w ~ N(0, 1/D) keeps <q, w_h> near N(0, 1)
        w = torch.randn(Hq, D, generator=gen, device=device, dtype=torch.float32) / math.sqrt(D)
        bias = torch.randn(Hq, generator=gen, device=device, dtype=torch.float32)
        gate = torch.cat([w.reshape(-1), bias])
    elif gate_mode != "none":
        if gate_mode == "per_token":
            gs = (B, Hq, Sq) if layout == "bhsd" else (B, Sq, Hq)
        else:
            gs = qs
        g = torch.randn(*gs, generator=gen, device=device, dtype=torch.float32)
        g = torch.sigmoid(g) if gate_kind == "sigmoid" else g * 0.1
        gate = g.to(tdt)

    if q_var is not None and pad_inputs:
        qm = _tile_valid_mask(q_var, q_block, layout, device)
        km = _tile_valid_mask(kv_var, kv_block, layout, device)
        q = q * qm.to(tdt)
        k = k * km.to(tdt)
        v = v * km.to(tdt)
        if pad_dout:
            dout = dout * qm.to(tdt)
            if gate is not None and gate_mode != "projected":
                gm = qm if gate.dim() == 4 else qm.squeeze(-1)
                gate = gate * gm.to(tdt)

    case = Case(name=name, dtype=dtype, layout=layout, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Skv=Skv, D=D,
                q_block=q_block, kv_block=kv_block, Qb=Qb, KVb=KVb, scale=scale, topk=topk,
                gate_mode=gate_mode, q_var=q_var, kv_var=kv_var,
                q_lens=list(q_lens) if q_lens is not None else None,
                kv_lens=list(kv_lens) if kv_lens is not None else None,
                q=q.contiguous(), k=k.contiguous(), v=v.contiguous(), dout=dout.contiguous(),
                gate=None if gate is None else gate.contiguous())
    case.block_map = _draw_map(case, gen, device, map_kind, map_p, map_per_row, map_fn)
    return case


def _seq_blocks(case: Case, b: int):
    """Number of Q and KV blocks that sequence b actually covers."""
    if case.q_lens is not None:
        return _ceil(case.q_lens[b], case.q_block), _ceil(case.kv_lens[b], case.kv_block)
    return case.Qb, case.KVb


def _draw_map(case: Case, gen, device, kind, p, per_row, fn) -> Optional[torch.Tensor]:
    shape = (case.B, case.Hq, case.Qb, case.KVb)
    if kind == "none":
        return None
    if kind == "ones":
        return torch.ones(shape, dtype=torch.uint8)
    if kind == "custom":
        return fn(case).to(torch.uint8).cpu().contiguous()
    if kind == "bernoulli":
        m = (torch.rand(*shape, generator=gen, device=device) < p).to(torch.uint8).cpu()
        # force at least one selected block inside each sequence's own grid
        fill = torch.randint(0, 1 << 30, shape[:3], generator=gen, device=device).cpu()
        for b in range(case.B):
            nq, nk = _seq_blocks(case, b)
            own = m[b, :, :nq, :nk]
            empty = own.sum(-1) == 0
            if empty.any():
                hs, qs = torch.nonzero(empty, as_tuple=True)
                js = fill[b, hs, qs] % nk
                m[b, hs, qs, js] = 1
        return m.contiguous()
    if kind == "per_row":
        keys = torch.rand(*shape, generator=gen, device=device).cpu()
        m = torch.zeros(shape, dtype=torch.uint8)
        for b in range(case.B):
            nq, nk = _seq_blocks(case, b)
            order = torch.argsort(keys[b, :, :nq, :nk], dim=-1)[..., :min(per_row, nk)]
            m[b, :, :nq].scatter_(-1, order, 1)
        return m.contiguous()
    raise ValueError(kind)


# ---------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------

def _c1(seed=42, device="cpu", layout="bhsd", **kw):
    """VSA-256 tiny: 3 Q tiles, 4 KV tiles with valid counts [256,173,79,256];
    2 KV tiles per (head, Q tile) drawn at random."""
    return build_case("c1_vsa256_tiny", dtype="bf16", layout=layout, B=1, Hq=2, D=128,
                      q_var=[256] * 3, kv_var=[256, 173, 79, 256], map_kind="per_row",
                      map_per_row=2, seed=seed, device=device, **kw)


def _c2(seed=42, device="cpu", **kw):
    """BNSD MHA: B=2, 8 heads, S=4096, fp16, [128,128] blocks, Bernoulli(0.25)."""
    return build_case("c2_bnsd_mha", dtype="fp16", layout="bhsd", B=2, Hq=8, Hkv=8, D=128,
                      q_block=128, kv_block=128, Sq=4096, Skv=4096, map_kind="bernoulli",
                      map_p=0.25, seed=seed, device=device, **kw)


def _c3(seed=42, device="cpu", **kw):
    """TND varlen GQA: 13 sequences, q_len ~ U{7..360}, kv_len = q_len + U{4..180},
    12 Q heads / 3 KV heads, fp16, [128,128] blocks, Bernoulli(0.5)."""
    g = torch.Generator().manual_seed(seed + 1000)
    ql = torch.randint(7, 361, (13,), generator=g).tolist()
    kl = [a + b for a, b in zip(ql, torch.randint(4, 181, (13,), generator=g).tolist())]
    return build_case("c3_tnd_gqa", dtype="fp16", layout="tnd", Hq=12, Hkv=3, D=128,
                      q_block=128, kv_block=128, q_lens=ql, kv_lens=kl, map_kind="bernoulli",
                      map_p=0.5, seed=seed, device=device, **kw)


def _page_tnd_mask(case: Case) -> torch.Tensor:
    """The Ascend test page's deterministic sparse TND mask: each Q block of
    sequence b / head n selects KV block (q+b+n) mod nkv, and also the next
    one when (q+n) is even and the sequence has more than one KV block."""
    m = torch.zeros(case.B, case.Hq, case.Qb, case.KVb, dtype=torch.uint8)
    for b in range(case.B):
        nk = _ceil(case.kv_lens[b], case.kv_block)
        for n in range(case.Hq):
            for qb in range(case.Qb):
                m[b, n, qb, (qb + b + n) % nk] = 1
                if nk > 1 and (qb + n) % 2 == 0:
                    m[b, n, qb, (qb + b + n + 1) % nk] = 1
    return m


_PAGE_Q_LENS = [355, 17, 41, 83, 129, 211, 7, 53, 97, 151, 233, 301, 19]
_PAGE_KV_LENS = [533, 23, 67, 101, 173, 257, 11, 89, 137, 199, 281, 349, 31]


def _c3_page(seed=42, device="cpu", full=False, **kw):
    """The Ascend page's fixed TND GQA case (13 sequences, 12/3 heads)."""
    return build_case("c3_tnd_gqa_page", dtype="fp16", layout="tnd", Hq=12, Hkv=3, D=128,
                      q_block=128, kv_block=128, q_lens=_PAGE_Q_LENS, kv_lens=_PAGE_KV_LENS,
                      map_kind="ones" if full else "custom", map_fn=_page_tnd_mask,
                      seed=seed, device=device, **kw)


def _c4(seed=42, device="cpu", **kw):
    """VSA-256 video: latent 21x48x80 in (4,8,8) tiles -> 360 tiles, B=1, H=12,
    bf16, BSHD, topk=36 by pooled score."""
    var = vsa_tile_counts((21, 48, 80))
    return build_case("c4_vsa256_video", dtype="bf16", layout="bshd", B=1, Hq=12, D=128,
                      q_var=var, kv_var=var, topk=36, map_kind="none", seed=seed,
                      device=device, **kw)


def _c5(seed=42, device="cpu", gate_mode="per_token", **kw):
    """VSA-256 720p with the compression gate: latent 21x90x160 in (4,8,8)
    tiles -> 1440 tiles, B=1, H=40, bf16, BSHD, topk=144, per-token per-head
    gate sigmoid(N(0,1)) (gate_mode selects another gate form for measuring
    it at this shape)."""
    var = vsa_tile_counts((21, 90, 160))
    return build_case("c5_vsa256_720p_gate", dtype="bf16", layout="bshd", B=1, Hq=40, D=128,
                      q_var=var, kv_var=var, topk=144, map_kind="none", gate_mode=gate_mode,
                      gate_kind="sigmoid", seed=seed, device=device, **kw)


def _c5_vsa128(seed=42, device="cpu", **kw):
    """The 720p latent in VSA-128 tiles: 21x90x160 in (2,8,8) tiles -> 11 x 12
    x 20 = 2640 tiles of 128 tokens, B=1, H=40, bf16, BSHD, topk=288 (the same
    tenth of the tiles as the 256-token workload), per-token gate."""
    var = vsa_tile_counts((21, 90, 160), tile=(2, 8, 8))
    return build_case("c5_vsa128_720p_gate", dtype="bf16", layout="bshd", B=1, Hq=40, D=128,
                      q_block=128, kv_block=128, q_var=var, kv_var=var, topk=288, map_kind="none",
                      gate_mode="per_token", gate_kind="sigmoid", seed=seed, device=device, **kw)


def _p1(name, kv_var, q_var, topk, seed, gate=False):
    """The FastVideo VSA-256 parity tests: bf16 N(0,1) q/k/v zero-padded by
    their tile counts, grad_out left unpadded, pooled-score top-k."""
    def make(seed=seed, device="cpu", layout="bhsd", **kw):
        return build_case(name, dtype="bf16", layout=layout, B=1, Hq=2, D=128, q_var=q_var,
                          kv_var=kv_var, topk=topk, map_kind="none",
                          gate_mode="per_element" if gate else "none", gate_kind="scaled",
                          pad_dout=False, seed=seed, device=device, **kw)
    return make


def _p3_bnsd(name, dtype, S, block, sparse):
    def mask_fn(case):
        m = torch.zeros(case.B, case.Hq, case.Qb, case.KVb, dtype=torch.uint8)
        for i in range(case.Qb):
            m[:, :, i, i % case.KVb] = 1
        return m

    def make(seed=42, device="cpu", **kw):
        return build_case(name, dtype=dtype, layout="bhsd", B=2, Hq=8, Hkv=8, D=128,
                          q_block=block[0], kv_block=block[1], Sq=S, Skv=S,
                          map_kind="custom" if sparse else "ones", map_fn=mask_fn,
                          seed=seed, device=device, **kw)
    return make


def _p3_tnd(name, hq, hkv, ql, kl, block=(128, 128), full=False):
    def make(seed=42, device="cpu", **kw):
        return build_case(name, dtype="fp16", layout="tnd", Hq=hq, Hkv=hkv, D=128,
                          q_block=block[0], kv_block=block[1], q_lens=ql, kv_lens=kl,
                          map_kind="ones" if full else "custom", map_fn=_page_tnd_mask,
                          seed=seed, device=device, **kw)
    return make


CASES: Dict[str, Callable[..., Case]] = {
    "c1_vsa256_tiny": _c1,
    "c2_bnsd_mha": _c2,
    "c3_tnd_gqa": _c3,
    "c3_tnd_gqa_page": _c3_page,
    "c4_vsa256_video": _c4,
    "c5_vsa256_720p_gate": _c5,
    "c5_vsa128_720p_gate": _c5_vsa128,
    "p1_fwd_bwd": _p1("p1_fwd_bwd", [256, 173, 79, 256], [256] * 3, 2, 42),
    "p1_gated": _p1("p1_gated", [256, 200, 256, 91], [256] * 3, 2, 7, gate=True),
    "p1_partial_q": _p1("p1_partial_q", [256, 128, 256], [256, 61, 199], 2, 11),
    "p1_cross": _p1("p1_cross", [256, 143, 256, 256, 88], [256] * 2, 3, 13),
    "p1_infer": _p1("p1_infer", [256, 173, 79, 256], [256] * 3, 2, 5),
    "p3_bnsd_fp16": _p3_bnsd("p3_bnsd_fp16", "fp16", 32, (128, 128), False),
    "p3_bnsd_bf16": _p3_bnsd("p3_bnsd_bf16", "bf16", 32, (128, 128), False),
    "p3_bnsd_sparse32": _p3_bnsd("p3_bnsd_sparse32", "fp16", 256, (32, 128), True),
    # the Ascend page's multi-block sparse scenario, block_shape [8, 128], and [16, 128]
    "p3_bnsd_q8": _p3_bnsd("p3_bnsd_q8", "fp16", 256, (8, 128), True),
    "p3_bnsd_q16": _p3_bnsd("p3_bnsd_q16", "bf16", 256, (16, 128), True),
    "p3_tnd_full": _p3_tnd("p3_tnd_full", 12, 3, _PAGE_Q_LENS, _PAGE_KV_LENS, full=True),
    "p3_tnd_sparse": _p3_tnd("p3_tnd_sparse", 12, 3, _PAGE_Q_LENS, _PAGE_KV_LENS),
    "p3_tnd_single": _p3_tnd("p3_tnd_single", 4, 2, [127], [191], full=True),
    "p3_tnd_uneven": _p3_tnd("p3_tnd_uneven", 4, 2, [1, 64, 129, 17], [128, 3, 257, 65]),
    "p3_tnd_group4": _p3_tnd("p3_tnd_group4", 8, 2, [96, 137], [111, 259]),
    "p3_tnd_mqa": _p3_tnd("p3_tnd_mqa", 8, 1, [65, 130], [129, 33]),
    "p3_tnd_tail64": _p3_tnd("p3_tnd_tail64", 4, 2, [65, 127, 3], [129, 11, 64], block=(64, 128)),
    "p3_tnd_q8": _p3_tnd("p3_tnd_q8", 4, 2, [65, 127, 3, 30], [129, 11, 64, 200], block=(8, 128)),
    # KV blocks other than 128 / 256: one 64-key chunk per block; 192 keys with
    # 96-row Q blocks (three 32-row waves per block); 320 keys (a dK/dV span of
    # 256 keys plus one of 64); 512 keys (two full spans)
    "p3_bnsd_kv64": _p3_bnsd("p3_bnsd_kv64", "bf16", 512, (64, 64), True),
    "p3_tnd_kv192": _p3_tnd("p3_tnd_kv192", 4, 2, [65, 300, 7], [129, 500, 400], block=(96, 192)),
    "p3_tnd_kv320": _p3_tnd("p3_tnd_kv320", 4, 1, [33, 250, 700], [321, 640, 650], block=(32, 320)),
    "p3_bnsd_kv512": _p3_bnsd("p3_bnsd_kv512", "fp16", 1024, (128, 512), False),
}


def make_case(name: str, **kw) -> Case:
    return CASES[name](**kw)
