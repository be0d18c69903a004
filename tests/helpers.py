"""Test-side helpers: library references and error metrics.

Nothing here is used by the GPU library; nothing here is used by the oracle.
"""

from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def metrics(ref, got):
    """avg_abs = mean |got - ref|; max_rel = max |got - ref| / max |ref|.

    The FastVideo parity test prints these two numbers for every tensor; its
    own definition is off the page, so this tensor-normalised form is the
    reading used throughout (the only one under which the reported ~0.11 on
    N(0,1) data is plausible).
    """
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    if ref.size == 0:
        return 0.0, 0.0
    diff = np.abs(got - ref)
    den = max(np.abs(ref).max(), 1e-30)
    return float(diff.mean()), float(diff.max() / den)


OUT_TOL = (1e-3, 0.2)
GRAD_TOL = (1e-3, 0.25)
# Where a tensor is large enough that rounding the exact result once to the
# 16-bit output type already costs a sizeable part of the avg_abs bar, the bar
# is this many times that rounding error instead (see rounding_floor).
FLOOR_FACTOR = 3.0


def rounding_floor(ref, dtype):
    """mean |round(ref) - ref| for rounding to the 16-bit output type ("bf16"
    or "fp16", nearest even): the avg_abs that an exact computation with a
    16-bit output still shows against a float reference."""
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    r = torch.from_numpy(ref.astype(np.float32)).to(tdt).double().numpy()
    return float(np.abs(r - ref).mean())


def check(tag, ref, got, tol, out_dtype=None):
    """Hold one tensor to an (avg_abs, max_rel) bar against its reference.

    Every value must be finite; the two error figures are logged on one line
    and a single assertion names whichever bound was broken. With out_dtype
    (the 16-bit type the result was stored in), the avg_abs bound is at least
    FLOOR_FACTOR times the rounding floor of the reference in that type: the
    fixed bound presumes gradients of the size the pages' workloads give, and
    a tensor whose entries are ten times larger cannot meet it in bf16 however
    exact its arithmetic. The max_rel bound is unchanged.
    """
    got = np.asarray(got, dtype=np.float64)
    n_bad = int(np.size(got) - np.count_nonzero(np.isfinite(got)))
    if n_bad:
        raise AssertionError(f"{tag}: {n_bad} NaN or infinite entries")
    avg_abs, max_rel = metrics(ref, got)
    if out_dtype is not None:
        tol = (max(tol[0], FLOOR_FACTOR * rounding_floor(ref, out_dtype)), tol[1])
    print(f"  {tag:6s} avg_abs {avg_abs:.2e}  max_rel {max_rel:.2e}  (bar {tol[0]:.3g} / {tol[1]:g})")
    broken = [f"{what} {val:.3e} >= {bound:g}" for what, val, bound in
              (("avg_abs", avg_abs, tol[0]), ("max_rel", max_rel, tol[1])) if not val < bound]
    if broken:
        raise AssertionError(f"{tag}: " + ", ".join(broken))
    return avg_abs, max_rel


def expand_token_mask(bmap_b, q_block, kv_block, q_len, kv_len, kv_var=None):
    """Boolean [H, q_len, kv_len] token mask of one batch entry / sequence:
    each block entry repeated over its tokens and cut to the real lengths, as
    the Ascend test page expands its block mask, and, for video tiles, keys
    past their tile's valid count removed (the FastVideo mask_mod)."""
    m = torch.as_tensor(np.asarray(bmap_b)).bool()
    m = m.repeat_interleave(q_block, 1).repeat_interleave(kv_block, 2)[:, :q_len, :kv_len]
    if kv_var is not None:
        t = torch.arange(kv_len)
        live = (t % kv_block) < torch.as_tensor(np.asarray(kv_var))[t // kv_block]
        m = m & live.view(1, 1, -1)
    return m


def _to_bhsd(x, layout):
    return x.transpose(1, 2) if layout == "bshd" else x


def sdpa_reference(case, bmap, dout=None):
    """float64 dense reference through torch's scaled_dot_product_attention
    with the expanded token mask (GQA through enable_gqa), gradients through
    autograd. Returns out, dq, dk, dv in the case layout (numpy)."""
    q = case.q.double().clone().requires_grad_(True)
    k = case.k.double().clone().requires_grad_(True)
    v = case.v.double().clone().requires_grad_(True)
    do = (case.dout if dout is None else dout).double()
    if case.layout in ("bhsd", "bshd"):
        mask = torch.stack([expand_token_mask(bmap[b], case.q_block, case.kv_block, case.Sq,
                                              case.Skv, case.kv_var) for b in range(case.B)])
        o = F.scaled_dot_product_attention(_to_bhsd(q, case.layout), _to_bhsd(k, case.layout),
                                           _to_bhsd(v, case.layout), attn_mask=mask,
                                           scale=case.scale, enable_gqa=True)
        o = _to_bhsd(o, case.layout)
    else:
        outs = []
        cq = np.concatenate([[0], np.cumsum(case.q_lens)])
        ck = np.concatenate([[0], np.cumsum(case.kv_lens)])
        for b in range(case.B):
            ql, kl = case.q_lens[b], case.kv_lens[b]
            mask = expand_token_mask(bmap[b], case.q_block, case.kv_block, ql, kl)[None]
            qb = q[cq[b]:cq[b + 1]].transpose(0, 1)[None]
            kb = k[ck[b]:ck[b + 1]].transpose(0, 1)[None]
            vb = v[ck[b]:ck[b + 1]].transpose(0, 1)[None]
            ob = F.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask, scale=case.scale,
                                                enable_gqa=True)
            outs.append(ob[0].transpose(0, 1))
        o = torch.cat(outs, 0)
    (o * do).sum().backward()
    return (o.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy())


def _valid_counts(var, block, total):
    """Valid tokens per tile: the tile count when given, never more than exist."""
    n = (total + block - 1) // block
    exist = np.array([min(block, total - i * block) for i in range(n)], np.int64)
    return exist if var is None else np.minimum(np.asarray(var, np.int64), exist)


def _tile_average(var, block, total):
    """[tiles, total] float64 matrix whose row i averages the valid slots of
    tile i (1/count on them, 0 elsewhere; an empty tile gives a zero row)."""
    cnt = _valid_counts(var, block, total)
    w = torch.zeros(len(cnt), total, dtype=torch.float64)
    for i, n in enumerate(cnt):
        if n > 0:
            w[i, i * block:i * block + n] = 1.0 / n
    return w


def torch_vsa_reference(case, bmap, dout=None):
    """float64 torch reference of the whole video-tile path, gradients by autograd.

    Written with tensor operations and independent of the oracle's loops
    (FastVideo test_vsa256_backward.py page: the gated test composes the sparse
    output with the compression output; the partial-Q test: q_var only sets the
    compression divisor):
      * sparse branch: scaled_dot_product_attention with the expanded token
        mask (keys past a tile's valid count removed), GQA by enable_gqa;
      * pooled tiles: a tile-averaging matrix (1/count on the valid slots of
        each tile) applied to q, k and v;
      * coarse scores C = scale Qc Kc^T, KV tiles without a valid token set to
        -inf; O_c = softmax(C) Vc, spread over every slot of its Q tile;
      * out = O_sel + gate * O_c (per-token gates broadcast over D; a
        projected gate is sigmoid(<q_s, w_h> + b_h) with gate = [w | b]).
    Returns numpy out, dq, dk, dv, dgate (None without a gate) in the case
    layout; the backward is torch autograd of sum(out * dout).
    """
    assert case.layout in ("bhsd", "bshd")
    leaf = lambda t: t.double().clone().requires_grad_(True)  # noqa: E731
    q, k, v = leaf(case.q), leaf(case.k), leaf(case.v)
    gate = leaf(case.gate) if case.gate is not None else None
    do = (case.dout if dout is None else dout).double()
    qh, kh, vh = (_to_bhsd(t, case.layout) for t in (q, k, v))  # [B,H,S,D]
    mask = torch.stack([expand_token_mask(bmap[b], case.q_block, case.kv_block, case.Sq,
                                          case.Skv, case.kv_var) for b in range(case.B)])
    out = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=case.scale,
                                         enable_gqa=True)
    if case.gate_mode != "none":
        wq = _tile_average(case.q_var, case.q_block, case.Sq)
        wk = _tile_average(case.kv_var, case.kv_block, case.Skv)
        grp = case.Hq // case.Hkv
        qc = wq @ qh
        kc = (wk @ kh).repeat_interleave(grp, dim=1)
        vc = (wk @ vh).repeat_interleave(grp, dim=1)
        live = torch.as_tensor(_valid_counts(case.kv_var, case.kv_block, case.Skv) > 0)
        scores = (case.scale * qc @ kc.transpose(-1, -2)).masked_fill(~live, float("-inf"))
        oc = torch.softmax(scores, dim=-1) @ vc  # [B,H,Qb,D]
        oc_tok = oc.repeat_interleave(case.q_block, dim=2)[:, :, :case.Sq]
        if case.gate_mode == "per_token":
            g = (gate if case.layout == "bhsd" else gate.transpose(1, 2)).unsqueeze(-1)
        elif case.gate_mode == "projected":  # sigmoid(<q_s, w_h> + b_h), gate = [w | b]
            w = gate[:case.Hq * case.D].view(case.Hq, case.D)
            z = (qh * w[None, :, None, :]).sum(-1) + gate[case.Hq * case.D:][None, :, None]
            g = torch.sigmoid(z).unsqueeze(-1)
        else:
            g = _to_bhsd(gate, case.layout)
        out = out + g * oc_tok
    out = _to_bhsd(out, case.layout)
    (out * do).sum().backward()
    return (out.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy(),
            None if gate is None else gate.grad.numpy())
