"""PyTorch entry points over the C ABI: an autograd Function and the
video-tile wrappers.

Semantics follow the FastVideo adapter page (`block_sparse_attn_cute_fwd.py`,
its autograd bridge and BHSD / BSHD entry points) and the FastVideo VSA-256
test page (`video_sparse_attn` / `video_sparse_attn_bshd` usage):

- the forward returns `out` and a natural-log `lse` of shape [B, H, S]; the lse
  is not differentiable;
- when no input needs a gradient the call takes the inference path (no
  backward index, no saved state); its output equals the training forward;
- a missing output gradient in the backward counts as zeros;
- BSHD is the native layout of the video path; BHSD goes through the same
  kernels with its own strides (no transposes);
- the video wrappers build the tile map by pooled-score top-k inside the
  library and add the gated compression branch when a gate is given;
- a projected gate (weights w [H, D] and bias b [H]) has the library compute
  each token's gate as sigmoid(<q, w_h> + b_h) and return dw, db;
- packed variable-length sequences ([T, H, D], the Ascend operator's TND
  layout with per-sequence actual lengths) go through block_sparse_attn_tnd.

Everything here is argument marshalling: every step of the computation runs in
the library's HIP kernels.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Sequence, Tuple, Union

import torch

from . import Buffers, make_problem, vsa_bwd, vsa_fwd

Counts = Optional[Union[torch.Tensor, Sequence[int]]]


def _counts(x: Counts, device) -> Optional[torch.Tensor]:
    """Per-tile valid counts as a contiguous int32 tensor on `device`: [tiles]
    (shared by the batch) or [B, tiles] (per batch entry)."""
    if x is None:
        return None
    t = torch.as_tensor(x, dtype=torch.int32)
    t = t.to(device).contiguous()
    return t if t.dim() == 2 else t.view(-1)


def gate_mode_of(gate: Optional[torch.Tensor], q: torch.Tensor, layout: str) -> str:
    """'none', 'per_element' (gate shaped like q) or 'per_token' (q's shape
    without the head dimension D)."""
    if gate is None:
        return "none"
    if tuple(gate.shape) == tuple(q.shape):
        return "per_element"
    if tuple(gate.shape) == tuple(q.shape[:-1]):
        return "per_token"
    raise ValueError(f"gate shape {tuple(gate.shape)} matches neither q {tuple(q.shape)} "
                     f"(per element) nor {tuple(q.shape[:-1])} (per token)")


def dims(q: torch.Tensor, k: torch.Tensor, layout: str) -> Tuple[int, int, int, int, int, int]:
    """(B, Hq, Hkv, Sq, Skv, D) of BHSD [B,H,S,D] or BSHD [B,S,H,D] tensors."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError(f"{layout} tensors are 4-D, got q {tuple(q.shape)} and k {tuple(k.shape)}")
    if layout == "bhsd":
        B, Hq, Sq, D = q.shape
        Hkv, Skv = k.shape[1], k.shape[2]
    elif layout == "bshd":
        B, Sq, Hq, D = q.shape
        Skv, Hkv = k.shape[1], k.shape[2]
    else:
        raise ValueError(f"layout must be 'bhsd' or 'bshd', got {layout!r}")
    if k.shape[0] != B or k.shape[-1] != D:
        raise ValueError("q and k disagree on the batch or head size")
    return int(B), int(Hq), int(Hkv), int(Sq), int(Skv), int(D)


@dataclass(frozen=True)
class Spec:
    """Everything besides the tensors that defines one attention call."""
    layout: str
    q_block: int
    kv_block: int
    topk: int = 0
    scale: Optional[float] = None
    q_valid: Optional[torch.Tensor] = None
    kv_valid: Optional[torch.Tensor] = None
    # False: the backward adds dQ inside the KV-owned pass with float atomics
    # (faster or not, per workload; dq then varies in its last bits run to run)
    deterministic: bool = True
    # True: the gate slot holds the projected gate's parameters [w | b] (fp32)
    projected: bool = False
    # packed layout ("tnd"): [B+1] int32 offsets of the sequences and the
    # longest lengths
    cu_q: Optional[torch.Tensor] = None
    cu_kv: Optional[torch.Tensor] = None
    max_q: int = 0
    max_kv: int = 0

    def problem(self, q, k, gate):
        if self.layout == "tnd":
            Sq, Hq, D = (int(x) for x in q.shape)
            Skv, Hkv = int(k.shape[0]), int(k.shape[1])
            return make_problem(dtype=q.dtype, layout="tnd", B=int(self.cu_q.numel()) - 1, Hq=Hq,
                                Hkv=Hkv, Sq=Sq, Skv=Skv, D=D, q_block=self.q_block,
                                kv_block=self.kv_block, cu_seqlens_q=self.cu_q,
                                cu_seqlens_kv=self.cu_kv, max_seqlen_q=self.max_q,
                                max_seqlen_kv=self.max_kv, scale=self.scale,
                                atomic_dq=not self.deterministic)
        B, Hq, Hkv, Sq, Skv, D = dims(q, k, self.layout)
        mode = "projected" if self.projected else gate_mode_of(gate, q, self.layout)
        return make_problem(dtype=q.dtype, layout=self.layout, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq,
                            Skv=Skv, D=D, q_block=self.q_block, kv_block=self.kv_block,
                            q_valid=self.q_valid, kv_valid=self.kv_valid, scale=self.scale,
                            topk=self.topk, gate_mode=mode, atomic_dq=not self.deterministic,
                            gate_proj=gate if self.projected else None)


def _contig(*ts):
    return tuple(None if t is None else t.contiguous() for t in ts)


def _forward(spec: Spec, q, k, v, gate, block_map, training: bool):
    p = spec.problem(q, k, gate)
    buf = Buffers(p, q, training=training)
    bmap = block_map if spec.topk == 0 else buf.map
    vsa_fwd(p, q, k, v, bmap, None if spec.projected else gate, buf.out, buf.lse,
            buf.saved if training else None, buf.ws_fwd)
    return p, buf, bmap


class _Attention(torch.autograd.Function):
    """Block-sparse attention with autograd through q, k, v and the gate."""

    @staticmethod
    def forward(ctx, q, k, v, gate, block_map, spec: Spec):
        p, buf, bmap = _forward(spec, q, k, v, gate, block_map, training=True)
        ctx.save_for_backward(q, k, v, gate, buf.out, buf.lse)
        ctx.problem, ctx.buffers = p, buf  # saved state and workspace for the backward
        ctx.projected = spec.projected
        ctx.mark_non_differentiable(buf.lse)
        ctx.set_materialize_grads(False)
        return buf.out, buf.lse

    @staticmethod
    def backward(ctx, grad_out, grad_lse):
        del grad_lse  # lse is not differentiable
        q, k, v, gate, out, lse = ctx.saved_tensors
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dgate = torch.empty_like(gate) if gate is not None and ctx.needs_input_grad[3] else None
        # a missing output gradient counts as zeros (the library takes dout = NULL)
        dout = None if grad_out is None else grad_out.contiguous()
        vsa_bwd(ctx.problem, q, k, v, None if ctx.projected else gate, dout, out, lse,
                ctx.buffers.saved, dq, dk, dv, dgate, ctx.buffers.ws_bwd)
        return dq, dk, dv, dgate, None, None


def _theta(gate_proj, Hq: int, D: int) -> torch.Tensor:
    """[w | b] of a projected gate as one fp32 vector (autograd splits the
    gradient back into w and b)."""
    w, b = gate_proj
    if tuple(w.shape) != (Hq, D) or tuple(b.shape) != (Hq,):
        raise ValueError(f"gate projection: w must be [{Hq}, {D}] and b [{Hq}], got "
                         f"{tuple(w.shape)} and {tuple(b.shape)}")
    return torch.cat([w.float().reshape(-1), b.float().reshape(-1)])


def attention(q, k, v, spec: Spec, block_map: Optional[torch.Tensor] = None,
              gate: Optional[torch.Tensor] = None,
              gate_proj: Optional[Tuple[torch.Tensor, torch.Tensor]] = None
              ) -> Tuple[torch.Tensor, torch.Tensor]:
    """(out, lse) of block-sparse attention; autograd when any input needs a
    gradient, else the inference path. gate_proj = (w [H, D], b [H]) selects
    the projected gate (then `gate` must be None)."""
    if gate_proj is not None:
        if gate is not None:
            raise ValueError("give either a gate or a gate projection, not both")
        _, Hq, _, _, _, D = dims(q, k, spec.layout)
        gate = _theta(gate_proj, Hq, D)
        spec = replace(spec, projected=True)
    q, k, v, gate = _contig(q, k, v, gate)
    if block_map is not None:
        block_map = block_map.to(torch.uint8).contiguous()
    need = torch.is_grad_enabled() and any(
        t is not None and t.requires_grad for t in (q, k, v, gate))
    if need:
        return _Attention.apply(q, k, v, gate, block_map, spec)
    _, buf, _ = _forward(spec, q, k, v, gate, block_map, training=False)
    return buf.out, buf.lse


def block_sparse_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_map: torch.Tensor,
                      kv_valid: Counts = None, q_valid: Counts = None, *, layout: str = "bhsd",
                      scale: Optional[float] = None, gate: Optional[torch.Tensor] = None,
                      deterministic: bool = True) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention restricted to a boolean [B, H, Qb, KVb] (or [H, Qb, KVb]) map
    of (Q block, KV block) pairs; block sizes are the sequence lengths over the
    map's extents. kv_valid / q_valid: valid tokens per KV / Q tile (padded
    slots last). Returns (out, lse) with lse [B, H, S], detached."""
    if block_map.dim() == 3:
        block_map = block_map.unsqueeze(0)
    B, Hq, Hkv, Sq, Skv, D = dims(q, k, layout)
    Qb, KVb = int(block_map.shape[2]), int(block_map.shape[3])
    if Sq % Qb or Skv % KVb:
        raise ValueError(f"sequence lengths {Sq}, {Skv} are not multiples of the map's "
                         f"{Qb} x {KVb} blocks")
    if block_map.shape[1] != Hq:
        raise ValueError(f"block_map has {block_map.shape[1]} heads, q has {Hq}")
    if block_map.shape[0] not in (1, B):
        raise ValueError("block_map batch must be 1 or B")
    if block_map.shape[0] != B:
        block_map = block_map.expand(B, -1, -1, -1)
    spec = Spec(layout=layout, q_block=Sq // Qb, kv_block=Skv // KVb, scale=scale,
                q_valid=_counts(q_valid, q.device), kv_valid=_counts(kv_valid, q.device),
                deterministic=deterministic)
    out, lse = attention(q, k, v, spec, block_map=block_map, gate=gate)
    return out, lse.detach()


def block_sparse_attn_tnd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          block_map: torch.Tensor, block_shape: Sequence[int],
                          actual_seq_lengths: Sequence[int],
                          actual_seq_lengths_kv: Sequence[int], *, scale: Optional[float] = None,
                          deterministic: bool = True) -> Tuple[torch.Tensor, torch.Tensor]:
    """Block-sparse attention over packed variable-length sequences (the
    [Ascend] operator's TND layout): q [Tq, Hq, D], k / v [Tkv, Hkv, D] hold
    the sequences back to back, sequence b with actual_seq_lengths[b] query
    and actual_seq_lengths_kv[b] key tokens; block_map [B, Hq, Qb, KVb] over
    the blocks of the longest sequences, block_shape = (q_block, kv_block); Q
    head h reads KV head h // (Hq / Hkv). Returns (out [Tq, Hq, D], lse
    [Hq, Tq]), lse detached."""
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("TND tensors are 3-D [T, H, D]")
    lq = [int(x) for x in actual_seq_lengths]
    lk = [int(x) for x in actual_seq_lengths_kv]
    if len(lq) != len(lk) or not lq:
        raise ValueError("actual_seq_lengths and actual_seq_lengths_kv need one entry per sequence")
    if sum(lq) != q.shape[0] or sum(lk) != k.shape[0]:
        raise ValueError(f"the lengths sum to {sum(lq)} / {sum(lk)} tokens, the tensors hold "
                         f"{q.shape[0]} / {k.shape[0]}")
    qb, kb = (int(x) for x in block_shape)
    mq, mk = max(lq), max(lk)
    want = (len(lq), int(q.shape[1]), -(-mq // qb), -(-mk // kb))
    if block_map.dim() != 4 or tuple(block_map.shape) != want:
        raise ValueError(f"block_map must be {list(want)} (sequences, heads, Q blocks and KV "
                         f"blocks of the longest sequences), got {list(block_map.shape)}")

    def offsets(lens):
        c = [0]
        for x in lens:
            c.append(c[-1] + x)
        return torch.tensor(c, dtype=torch.int32, device=q.device)

    spec = Spec(layout="tnd", q_block=qb, kv_block=kb, scale=scale, deterministic=deterministic,
                cu_q=offsets(lq), cu_kv=offsets(lk), max_q=mq, max_kv=mk)
    out, lse = attention(q, k, v, spec, block_map=block_map)
    return out, lse.detach()


def _video(q, k, v, kv_var, q_var, topk, block_size, gate, scale, layout, deterministic,
           gate_proj=None):
    tile = 1
    for s in block_size:
        tile *= int(s)
    spec = Spec(layout=layout, q_block=tile, kv_block=tile, topk=int(topk), scale=scale,
                q_valid=_counts(q_var, q.device), kv_valid=_counts(kv_var, q.device),
                deterministic=deterministic)
    return attention(q, k, v, spec, gate=gate, gate_proj=gate_proj)[0]


def video_sparse_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_var: Counts,
                      q_var: Counts, topk: int, block_size: Sequence[int] = (4, 8, 8),
                      compress_attn_weight: Optional[torch.Tensor] = None,
                      scale: Optional[float] = None, deterministic: bool = True,
                      gate_proj: Optional[Tuple[torch.Tensor, torch.Tensor]] = None
                      ) -> torch.Tensor:
    """Video sparse attention over [B, H, S, D] tensors laid out in tiles of
    prod(block_size) tokens: each Q tile attends to its `topk` KV tiles of
    highest pooled score (q_var / kv_var valid tokens per tile, [tiles] for the
    whole batch or [B, tiles] per video); with
    compress_attn_weight (or the projected gate gate_proj = (w, b)) the gated
    pooled-tile branch is added. Returns out."""
    return _video(q, k, v, kv_var, q_var, topk, block_size, compress_attn_weight, scale, "bhsd",
                  deterministic, gate_proj)


def video_sparse_attn_bshd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_var: Counts,
                           q_var: Counts, topk: int, block_size: Sequence[int] = (4, 8, 8),
                           compress_attn_weight: Optional[torch.Tensor] = None,
                           scale: Optional[float] = None,
                           deterministic: bool = True,
                           gate_proj: Optional[Tuple[torch.Tensor, torch.Tensor]] = None
                           ) -> torch.Tensor:
    """video_sparse_attn for [B, S, H, D] tensors (the gate likewise in BSHD)."""
    return _video(q, k, v, kv_var, q_var, topk, block_size, compress_attn_weight, scale, "bshd",
                  deterministic, gate_proj)
