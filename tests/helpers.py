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


def check(tag, ref, got, tol):
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{tag}: non-finite values"
    a, r = metrics(ref, got)
    print(f"  {tag}: avg_abs={a:.3e} max_rel={r:.3e}")
    assert a < tol[0], f"{tag}: avg_abs {a:.3e} >= {tol[0]:.3e}"
    assert r < tol[1], f"{tag}: max_rel {r:.3e} >= {tol[1]:.3e}"


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
