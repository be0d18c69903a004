"""Pins of the CPU oracle to things other than itself (no GPU needed).

* special cases that reduce to a library routine: torch's scaled dot-product
  attention (float64, boolean token mask, GQA) with autograd gradients;
* brute force on tiny inputs: central finite differences of L = sum(out*dO)
  in float64, exhaustive enumeration of the block index, sorting for top-k;
* closed forms and invariants: padded slots are inert, unselected tiles get
  no sparse-branch gradient, key-shift and value-shift identities, scale
  invariance, layout transposition, GQA = repeated MHA, one live key,
  block-diagonal maps, single-tile compression, empty rows.

Each check is chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign or index, a transposed operand, a missing mask) fails it.
"""

from __future__ import annotations

import dataclasses
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from tests.helpers import expand_token_mask, sdpa_reference, torch_vsa_reference
from workloads.synth import build_case, make_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


# ---------------------------------------------------------------------------
# Library routine: masked softmax attention through torch SDPA (float64)
# ---------------------------------------------------------------------------

def _sdpa_cases():
    yield build_case("dense_gqa_ragged", dtype="bf16", layout="bhsd", B=2, Hq=4, Hkv=2, D=16,
                     q_block=8, kv_block=8, Sq=37, Skv=45, map_kind="ones", seed=1)
    yield build_case("masked_bhsd", dtype="fp16", layout="bhsd", B=2, Hq=2, Hkv=2, D=16,
                     q_block=8, kv_block=16, Sq=40, Skv=64, map_kind="bernoulli", map_p=0.4,
                     seed=2)
    yield build_case("vsa_tiles_bshd", dtype="bf16", layout="bshd", B=1, Hq=4, Hkv=1, D=16,
                     q_block=16, kv_block=16, q_var=[16, 5, 16], kv_var=[16, 7, 1, 16, 12],
                     map_kind="per_row", map_per_row=2, pad_dout=False, seed=3)
    yield build_case("tnd_gqa", dtype="fp16", layout="tnd", Hq=6, Hkv=2, D=16, q_block=8,
                     kv_block=8, q_lens=[1, 13, 29, 8], kv_lens=[9, 3, 33, 17],
                     map_kind="bernoulli", map_p=0.5, seed=4)


@pytest.mark.parametrize("case", list(_sdpa_cases()), ids=lambda c: c.name)
def test_fwd_bwd_match_sdpa_autograd(case):
    orc = oracle.Oracle(case, np.float64)
    bmap = orc.block_map()
    out, osel, lse = orc.fwd()
    dq, dk, dv, _ = orc.bwd()
    r_out, r_dq, r_dk, r_dv = sdpa_reference(case, bmap)
    assert _rel(out, r_out) < 1e-12
    assert np.array_equal(out, osel)  # no gate: the output is the sparse branch
    assert _rel(dq, r_dq) < 1e-11
    assert _rel(dk, r_dk) < 1e-11
    assert _rel(dv, r_dv) < 1e-11


def test_lse_reconstructs_sdpa_output():
    """exp(z - lse) must be the softmax that SDPA applies: rebuilding P from the
    oracle's lse and multiplying by V reproduces the library output."""
    case = build_case("lse", dtype="bf16", layout="bhsd", B=1, Hq=2, D=16, q_block=8, kv_block=8,
                      Sq=24, Skv=40, map_kind="bernoulli", map_p=0.5, seed=5)
    orc = oracle.Oracle(case, np.float64)
    _, _, lse = orc.fwd()
    r_out = sdpa_reference(case, orc.block_map())[0]
    q, k, v = (t.double() for t in (case.q, case.k, case.v))
    m = expand_token_mask(orc.block_map()[0], 8, 8, 24, 40)
    z = case.scale * q[0] @ k[0].transpose(-1, -2)
    p = torch.exp(z - torch.as_tensor(lse[0])[..., None]) * m
    np.testing.assert_allclose((p @ v[0]).numpy(), r_out[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(p.sum(-1).numpy(), 1.0, atol=1e-12)


# ---------------------------------------------------------------------------
# Brute force: central finite differences (float64, tiny shapes)
# ---------------------------------------------------------------------------

def _loss(case, bmap, tensors):
    orc = oracle.Oracle(case, np.float64, tensors=tensors)
    orc.set_map(bmap)
    out = orc.fwd()[0]
    return float((out * tensors["dout"]).sum())


def _fd_check(case, eps=1e-5, names=("q", "k", "v", "gate")):
    base = oracle.Oracle(case, np.float64)
    bmap = base.block_map()  # held fixed: no gradient flows through the selection
    grads = dict(zip(("q", "k", "v", "gate"), base.bwd()))
    tens = dict(q=base.q, k=base.k, v=base.v, dout=base.dout, gate=base.gate)
    for name in names:
        x = tens[name]
        if x is None:
            continue
        fd = np.zeros_like(x)
        flat = x.reshape(-1)
        for idx in range(flat.size):
            old = flat[idx]
            flat[idx] = old + eps
            lp = _loss(case, bmap, tens)
            flat[idx] = old - eps
            lm = _loss(case, bmap, tens)
            flat[idx] = old
            fd.reshape(-1)[idx] = (lp - lm) / (2 * eps)
        err = _rel(grads[name], fd)
        assert err < 1e-6, f"{case.name} d{name}: rel err {err:.2e}"


FD_CASES = [
    dict(name="fd_plain_bhsd", layout="bhsd", topk=0, map_kind="bernoulli", gate_mode="none"),
    dict(name="fd_topk_bshd", layout="bshd", topk=2, map_kind="none", gate_mode="none"),
    dict(name="fd_gate_token", layout="bhsd", topk=2, map_kind="none", gate_mode="per_token"),
    dict(name="fd_gate_elem", layout="bshd", topk=3, map_kind="none", gate_mode="per_element",
         pad_dout=False),
    dict(name="fd_gate_proj", layout="bshd", topk=2, map_kind="none", gate_mode="projected"),
]


@pytest.mark.parametrize("kw", FD_CASES, ids=lambda k: k["name"])
def test_finite_differences_video_tiles(kw):
    kw = dict(kw)
    name = kw.pop("name")
    case = build_case(name, dtype="bf16", B=1, Hq=2, Hkv=1, D=8, q_block=4, kv_block=4,
                      q_var=[4, 3, 1], kv_var=[4, 2, 0, 3], gate_kind="sigmoid", seed=11, **kw)
    _fd_check(case)


def test_finite_differences_tnd_gqa():
    case = build_case("fd_tnd", dtype="fp16", layout="tnd", Hq=4, Hkv=2, D=8, q_block=4,
                      kv_block=4, q_lens=[5, 2], kv_lens=[7, 4], map_kind="bernoulli",
                      map_p=0.6, seed=12)
    _fd_check(case, names=("q", "k", "v"))


# ---------------------------------------------------------------------------
# Brute force: the block index
# ---------------------------------------------------------------------------

def _brute_index(case, bmap, kv_owned):
    def kv_valid(b, j):
        kv_len = case.kv_lens[b] if case.kv_lens else case.Skv
        exist = max(0, min(case.kv_block, kv_len - j * case.kv_block))
        return min(int(case.kv_var[j]), exist) if case.kv_var is not None else exist

    def blocks(b):
        if case.q_lens:
            return (-(-case.q_lens[b] // case.q_block), -(-case.kv_lens[b] // case.kv_block))
        return case.Qb, case.KVb

    rp, col = [0], []
    for b in range(case.B):
        nq, nk = blocks(b)
        for h in range(case.Hq):
            for r in range(case.KVb if kv_owned else case.Qb):
                for c in range(case.Qb if kv_owned else case.KVb):
                    i, j = (c, r) if kv_owned else (r, c)
                    if i < nq and j < nk and bmap[b, h, i, j] and kv_valid(b, j) > 0:
                        col.append(c)
                rp.append(len(col))
    return np.array(rp, np.int32), np.array(col, np.int32)


@pytest.mark.parametrize("name", ["c1_vsa256_tiny", "c3_tnd_gqa_page", "p3_tnd_uneven",
                                  "p3_bnsd_sparse32"])
def test_block_index_brute_force(name):
    case = make_case(name)
    bmap = case.block_map.numpy()
    for kv_owned in (False, True):
        rp, col = oracle.block_index(case, bmap, kv_owned)
        brp, bcol = _brute_index(case, bmap, kv_owned)
        assert np.array_equal(rp, brp) and np.array_equal(col, bcol)


def test_block_index_golden_lse_case():
    """The FastVideo LSE-shape test selects the first two of 4 KV tiles for every
    Q tile (3 tiles, 2 heads); its index is written out by hand in the fixture."""
    with open(os.path.join(GOLDEN, "index_first_two_tiles.json")) as f:
        g = json.load(f)
    case = build_case("golden_idx", B=1, Hq=2, D=8, q_block=256, kv_block=256,
                      q_var=[256] * 3, kv_var=[256] * 4, map_kind="custom",
                      map_fn=lambda c: torch.tensor(g["block_map"], dtype=torch.uint8))
    bmap = case.block_map.numpy()
    for key, kv_owned in (("q_owned", False), ("kv_owned", True)):
        rp, col = oracle.block_index(case, bmap, kv_owned)
        assert rp.tolist() == g[key]["row_ptr"]
        assert col.tolist() == g[key]["col"]


def test_empty_kv_tiles_are_dropped_from_the_index():
    case = build_case("empty_tiles", B=1, Hq=1, D=8, q_block=4, kv_block=4, q_var=[4, 4],
                      kv_var=[4, 0, 2, 0], map_kind="ones")
    rp, col = oracle.block_index(case, case.block_map.numpy(), False)
    assert rp.tolist() == [0, 2, 4] and col.tolist() == [0, 2, 0, 2]
    rp, col = oracle.block_index(case, case.block_map.numpy(), True)
    assert rp.tolist() == [0, 2, 2, 4, 4] and col.tolist() == [0, 1, 0, 1]


# ---------------------------------------------------------------------------
# Pooling, top-k, compression
# ---------------------------------------------------------------------------

def _vsa_small(topk=3, gate_mode="none", seed=21, Hq=4, Hkv=2):
    return build_case("vsa_small", dtype="bf16", layout="bshd", B=1, Hq=Hq, Hkv=Hkv, D=16,
                      q_block=8, kv_block=8, q_var=[8, 3, 8, 6], kv_var=[8, 1, 0, 8, 5, 8],
                      topk=topk, map_kind="none", gate_mode=gate_mode, seed=seed)


def test_pooling_is_the_mean_of_valid_slots():
    case = _vsa_small()
    qc, kc, vc = oracle.Oracle(case).pooled()
    q = case.q.double().numpy()  # [B,S,H,D]
    k = case.k.double().numpy()
    for i, n in enumerate(case.q_var):
        np.testing.assert_allclose(qc[0, :, i], q[0, i * 8:i * 8 + n].mean(0), atol=1e-14)
    for j, n in enumerate(case.kv_var):
        want = k[0, j * 8:j * 8 + n].mean(0) if n else np.zeros((2, 16))
        np.testing.assert_allclose(kc[0, :, j], want, atol=1e-14)


def test_topk_by_sorting_pooled_scores():
    case = _vsa_small(topk=3)
    orc = oracle.Oracle(case)
    qc, kc, _ = orc.pooled()
    C = orc.coarse_scores()
    group = case.Hq // case.Hkv
    m = orc.topk_map()
    for h in range(case.Hq):
        # scores through a library matmul, GQA head h reads KV head h // group
        s = case.scale * (qc[0, h] @ kc[0, h // group].T)
        valid = np.asarray(case.kv_var) > 0
        np.testing.assert_allclose(C[0, h][:, valid], s[:, valid], atol=1e-13)
        assert np.all(np.isneginf(C[0, h][:, ~valid]))
        for i in range(case.Qb):
            js = [j for j in np.argsort(-s[i], kind="stable") if valid[j]][:3]
            assert sorted(js) == sorted(np.nonzero(m[0, h, i])[0].tolist())


def test_topk_ties_go_to_the_lower_tile_and_clamp():
    # identical K tiles -> identical scores; keys 0 and 1 must win the tie
    case = build_case("ties", B=1, Hq=1, D=8, q_block=4, kv_block=4, q_var=[4], kv_var=[4] * 4,
                      topk=2, map_kind="none")
    case.k = case.k[:, :, :4].repeat(1, 1, 4, 1).contiguous()
    m = oracle.Oracle(case).topk_map()
    assert m[0, 0, 0].tolist() == [1, 1, 0, 0]
    m = oracle.Oracle(case).topk_map(topk=9)
    assert m[0, 0, 0].tolist() == [1, 1, 1, 1]


def test_compression_single_tile_and_softmax():
    case = build_case("one_tile", B=1, Hq=2, D=8, q_block=4, kv_block=4, q_var=[4, 2],
                      kv_var=[3], topk=1, map_kind="none", gate_mode="per_token")
    orc = oracle.Oracle(case)
    oc, lc = orc.coarse()
    _, _, vc = orc.pooled()
    np.testing.assert_allclose(oc[0, 0, 0], vc[0, 0, 0], atol=1e-15)  # P_c = 1
    case = _vsa_small(gate_mode="per_token")
    orc = oracle.Oracle(case)
    oc, lc = orc.coarse()
    qc, kc, vc = orc.pooled()
    C = orc.coarse_scores()
    from scipy.special import logsumexp, softmax
    valid = np.asarray(case.kv_var) > 0
    for h in range(case.Hq):
        P = softmax(C[0, h][:, valid], axis=-1)
        np.testing.assert_allclose(oc[0, h], P @ vc[0, h // 2][valid], atol=1e-14)
        np.testing.assert_allclose(lc[0, h], logsumexp(C[0, h][:, valid], axis=-1), atol=1e-14)


# ---------------------------------------------------------------------------
# The gated compression branch (composition, pooling gradient, coarse domain)
# ---------------------------------------------------------------------------

def _gated_cases():
    # GQA, top-k, per-token gate, a partial Q tile, an empty and a one-slot KV tile
    yield build_case("gated_tok_gqa", dtype="bf16", layout="bshd", B=1, Hq=4, Hkv=2, D=16,
                     q_block=8, kv_block=8, q_var=[8, 3, 8, 6], kv_var=[8, 1, 0, 8, 5, 8],
                     topk=3, map_kind="none", gate_mode="per_token", seed=31)
    # q-shaped signed gate (the FastVideo gated test's form), BHSD, two batch entries
    yield build_case("gated_elem_bhsd", dtype="bf16", layout="bhsd", B=2, Hq=2, Hkv=2, D=16,
                     q_block=8, kv_block=8, q_var=[8, 8, 2], kv_var=[8, 5, 8, 3],
                     topk=2, map_kind="none", gate_mode="per_element", gate_kind="scaled",
                     pad_dout=False, seed=32)
    # a caller-given map with unpadded inputs (no top-k), per-token gate, MQA
    yield build_case("gated_map_mqa", dtype="fp16", layout="bshd", B=1, Hq=3, Hkv=1, D=16,
                     q_block=8, kv_block=8, q_var=[5, 8, 8], kv_var=[8, 7, 8], map_kind="per_row",
                     map_per_row=2, gate_mode="per_token", pad_inputs=False, seed=33)
    # the gate projected from the query rows, GQA, top-k, two batch entries
    yield build_case("gated_proj_gqa", dtype="bf16", layout="bshd", B=2, Hq=4, Hkv=2, D=16,
                     q_block=8, kv_block=8, q_var=[8, 3, 8, 6], kv_var=[8, 1, 0, 8, 5, 8],
                     topk=3, map_kind="none", gate_mode="projected", seed=34)


@pytest.mark.parametrize("case", list(_gated_cases()), ids=lambda c: c.name)
def test_gated_path_matches_torch_autograd_reference(case):
    """out, dq, dk, dv and dgate of the whole gated path against an independent
    float64 torch implementation (SDPA for the sparse branch, a tile-averaging
    matrix for the pooling, softmax over non-empty tiles, additive gate),
    differentiated by autograd."""
    orc = oracle.Oracle(case, np.float64)
    bmap = orc.block_map()
    out, _, _ = orc.fwd()
    dq, dk, dv, dg = orc.bwd()
    r_out, r_dq, r_dk, r_dv, r_dg = torch_vsa_reference(case, bmap)
    for name, got, ref in (("out", out, r_out), ("dq", dq, r_dq), ("dk", dk, r_dk),
                           ("dv", dv, r_dv), ("dgate", dg, r_dg)):
        assert _rel(got, ref) < 1e-11, name


def test_zero_gate_reduces_to_the_ungated_path():
    """gate = 0: out is O_sel exactly and q/k/v get exactly the gradients of
    the path without a gate (the compression branch adds +0 everywhere)."""
    case = next(c for c in _gated_cases() if c.name == "gated_tok_gqa")
    case.gate = torch.zeros_like(case.gate)
    plain = dataclasses.replace(case, gate_mode="none", gate=None)
    orc, ref = oracle.Oracle(case), oracle.Oracle(plain)
    assert np.array_equal(orc.block_map(), ref.block_map())
    out, osel, lse = orc.fwd()
    r_out, _, r_lse = ref.fwd()
    assert np.array_equal(out, osel) and np.array_equal(out, r_out)
    assert np.array_equal(lse, r_lse)
    for got, want in zip(orc.bwd()[:3], ref.bwd()[:3]):
        assert np.array_equal(got, want)


def test_projected_gate_with_zero_weights_is_a_constant_gate():
    """w = 0: the projected gate is sigmoid(b_h) on every token of head h, so
    out, dq, dk and dv are those of a per-token gate holding that constant, and
    the parameter gradients follow from that case's dgate by the chain rule:
    db_h = sum_s dgate_s g(1-g), dw_h = sum_s dgate_s g(1-g) q_s."""
    case = next(c for c in _gated_cases() if c.name == "gated_proj_gqa")
    Hq, D = case.Hq, case.D
    theta = case.gate.clone()
    theta[:Hq * D] = 0
    case.gate = theta
    gh = torch.sigmoid(theta[Hq * D:].double())  # [Hq]
    const = np.ascontiguousarray(np.broadcast_to(gh.numpy(), (case.B, case.Sq, Hq)))
    tok = dataclasses.replace(case, gate_mode="per_token", gate=None)
    orc = oracle.Oracle(case)
    ref = oracle.Oracle(tok, tensors=dict(q=case.q, k=case.k, v=case.v, dout=case.dout,
                                          gate=const))  # float64, not through a float32 cast
    assert np.array_equal(orc.block_map(), ref.block_map())
    np.testing.assert_allclose(orc.fwd()[0], ref.fwd()[0], atol=1e-14)
    dq, dk, dv, dth = orc.bwd()
    r_dq, r_dk, r_dv, r_dg = ref.bwd()
    for got, want in ((dq, r_dq), (dk, r_dk), (dv, r_dv)):
        np.testing.assert_allclose(got, want, atol=1e-13)
    g = gh.numpy()
    dl = r_dg * g * (1 - g)                   # [B, S, H]
    q = case.q.double().numpy()               # [B, S, H, D]
    np.testing.assert_allclose(dth[Hq * D:], dl.sum((0, 1)), atol=1e-12)
    np.testing.assert_allclose(dth[:Hq * D].reshape(Hq, D), np.einsum("bsh,bshd->hd", dl, q),
                               atol=1e-12)


def test_projected_gate_values():
    """The oracle's projected gate values: with w = 0 they are sigmoid(b_h) on
    every token (closed form), and with the case's own parameters out - O_sel
    equals value * O_c of the token's Q tile (the composition of the gated
    output, read back through the oracle's forward)."""
    case = next(c for c in _gated_cases() if c.name == "gated_proj_gqa")
    Hq, D = case.Hq, case.D
    orc = oracle.Oracle(case)
    gv = orc.gate_values()                      # [B, S, H]
    out, osel, _ = orc.fwd()
    oc = orc.coarse()[0]                        # [B, H, Qb, D]
    tile = np.arange(case.Sq) // case.q_block
    oc_tok = oc[:, :, tile, :].transpose(0, 2, 1, 3)  # [B, S, H, D]
    np.testing.assert_allclose(out - osel, gv[..., None] * oc_tok, atol=1e-14)
    assert np.all((gv > 0) & (gv < 1))
    theta = case.gate.clone()
    theta[:Hq * D] = 0
    zero = dataclasses.replace(case, gate=theta)
    gh = 1.0 / (1.0 + np.exp(-theta[Hq * D:].double().numpy()))
    np.testing.assert_allclose(oracle.Oracle(zero).gate_values(),
                               np.broadcast_to(gh, gv.shape), rtol=1e-15)


def test_one_live_kv_tile_compression_closed_form():
    """A single KV tile with valid tokens: P_c = 1, so O_c = Vc (the mean of its
    valid v rows), dgate_s = <dO_s, Vc>, dS_c = 0 (no pooled term in dq, dk)
    and every valid slot t of that tile gets dv += sum_{heads, all slots s}
    gate_s dO_s / valid, padded slots nothing."""
    n = 5
    case = build_case("one_live", dtype="bf16", layout="bshd", B=1, Hq=2, Hkv=1, D=16,
                      q_block=8, kv_block=8, q_var=[8, 6], kv_var=[0, n, 0], map_kind="ones",
                      gate_mode="per_token", pad_inputs=False, seed=41)
    plain = dataclasses.replace(case, gate_mode="none", gate=None)
    orc, ref = oracle.Oracle(case), oracle.Oracle(plain)
    out, osel, _ = orc.fwd()
    dq, dk, dv, dg = orc.bwd()
    p_dq, p_dk, p_dv, _ = ref.bwd()
    v = case.v.double().numpy()[0]        # [S, Hkv, D]
    do = case.dout.double().numpy()[0]    # [S, H, D]
    g = case.gate.double().numpy()[0]     # [S, H]
    vc = v[8:8 + n, 0].mean(0)            # tile 1, its n valid slots
    np.testing.assert_allclose(out[0] - osel[0], g[..., None] * vc, atol=1e-13)
    np.testing.assert_allclose(dg[0], do @ vc, atol=1e-13)
    np.testing.assert_allclose(dq, p_dq, atol=1e-13)
    np.testing.assert_allclose(dk, p_dk, atol=1e-13)
    extra = np.zeros_like(dv)
    extra[0, 8:8 + n, 0] = (g[..., None] * do).sum((0, 1)) / n
    np.testing.assert_allclose(dv - p_dv, extra, atol=1e-12)


@pytest.mark.parametrize("partial", [False, True])
def test_coarse_attention_is_sdpa_over_pooled_tokens(partial):
    """O_c and lse_c equal dense softmax attention (torch SDPA, float64) over
    the mean-pooled tiles as tokens, with the empty KV tiles masked out; the
    pooled tiles are numpy means of each tile's valid rows."""
    q_var = [8, 3, 8, 6] if partial else [8] * 4
    kv_var = [8, 1, 0, 8, 5] if partial else [8] * 5
    case = build_case("pooled_sdpa", dtype="bf16", layout="bhsd", B=1, Hq=4, Hkv=2, D=16,
                      q_block=8, kv_block=8, q_var=q_var, kv_var=kv_var, map_kind="ones",
                      gate_mode="per_token", pad_inputs=False, seed=42)
    oc, lc = oracle.Oracle(case).coarse()
    q, k, v = (t.double().numpy()[0] for t in (case.q, case.k, case.v))  # [H, S, D]

    def means(x, var):
        return np.stack([x[:, i * 8:i * 8 + n].mean(1) if n else np.zeros(x[:, 0].shape)
                         for i, n in enumerate(var)], 1)
    qc, kc, vc = means(q, q_var), means(k, kv_var), means(v, kv_var)
    live = torch.as_tensor(np.asarray(kv_var) > 0)
    t = lambda x: torch.as_tensor(x)[None]  # noqa: E731
    mask = live.expand(len(q_var), -1)
    want = F.scaled_dot_product_attention(t(qc), t(kc), t(vc), attn_mask=mask, scale=case.scale,
                                          enable_gqa=True)[0].numpy()
    np.testing.assert_allclose(oc[0], want, atol=1e-13)
    s = case.scale * torch.as_tensor(qc) @ torch.as_tensor(kc).repeat_interleave(2, 0).transpose(1, 2)
    want_l = torch.logsumexp(s.masked_fill(~live, float("-inf")), -1).numpy()
    np.testing.assert_allclose(lc[0], want_l, atol=1e-13)


# ---------------------------------------------------------------------------
# Invariants and closed forms
# ---------------------------------------------------------------------------

def test_padded_kv_slots_are_inert():
    case = _vsa_small(topk=3, gate_mode="per_token")
    orc = oracle.Oracle(case)
    out, _, lse = orc.fwd()
    dq, dk, dv, _ = orc.bwd()
    # garbage in padded KV slots (BSHD [B,S,H,D])
    pad = np.ones(case.Skv, bool)
    for j, n in enumerate(case.kv_var):
        pad[j * 8:j * 8 + n] = False
    k2, v2 = orc.k.copy(), orc.v.copy()
    k2[:, pad] = 7.0
    v2[:, pad] = -5.0
    orc2 = oracle.Oracle(case, tensors=dict(q=orc.q, k=k2, v=v2, dout=orc.dout, gate=orc.gate))
    out2, _, lse2 = orc2.fwd()
    assert np.array_equal(orc2.block_map(), orc.block_map())
    np.testing.assert_array_equal(out2, out)
    np.testing.assert_array_equal(lse2, lse)
    dq2, dk2, dv2, _ = orc2.bwd()
    np.testing.assert_array_equal(dq2, dq)
    assert np.all(dk[:, pad] == 0) and np.all(dv[:, pad] == 0)
    assert np.all(dk2[:, pad] == 0) and np.all(dv2[:, pad] == 0)


def test_unselected_tile_gets_no_sparse_gradient():
    case = build_case("unsel", dtype="bf16", B=1, Hq=2, Hkv=1, D=8, q_block=4, kv_block=4,
                      q_var=[4, 4], kv_var=[4, 4, 4], map_kind="custom",
                      map_fn=lambda c: torch.tensor([[[[1, 0, 1], [1, 0, 0]],
                                                      [[0, 0, 1], [1, 0, 1]]]]))
    dq, dk, dv, _ = oracle.Oracle(case).bwd()
    assert np.all(dk[0, 0, 4:8] == 0) and np.all(dv[0, 0, 4:8] == 0)
    assert np.abs(dk[0, 0, :4]).max() > 0


@pytest.mark.parametrize("gate_mode", ["none", "per_token"])
def test_key_shift_gives_zero_total_dk(gate_mode):
    case = _vsa_small(topk=3, gate_mode=gate_mode)
    dq, dk, dv, _ = oracle.Oracle(case).bwd()
    tot = dk.sum(axis=1)  # [B,H,D] summed over keys
    assert np.abs(tot).max() < 1e-12 * max(1.0, np.abs(dk).max())


def test_value_shift_gives_total_dv_equal_total_dout():
    case = build_case("vshift", dtype="fp16", layout="bhsd", B=2, Hq=4, Hkv=2, D=16, q_block=8,
                      kv_block=8, Sq=30, Skv=44, map_kind="bernoulli", map_p=0.5, seed=7)
    orc = oracle.Oracle(case)
    _, dk, dv, _ = orc.bwd()
    do = orc.dout.reshape(2, 2, 2, 30, 16).sum(axis=(2, 3))  # over the group and rows
    np.testing.assert_allclose(dv.sum(axis=2), do, atol=1e-12)


def test_scale_invariance():
    case = _vsa_small(topk=0, seed=31)
    case.block_map = torch.ones(1, 4, 4, 6, dtype=torch.uint8)
    out = oracle.Oracle(case).fwd()[0]
    case2 = _vsa_small(topk=0, seed=31)
    case2.block_map = case.block_map
    case2.scale = case.scale / 4.0
    case2.q = case.q * 4  # exact in bf16
    out2 = oracle.Oracle(case2).fwd()[0]
    np.testing.assert_allclose(out2, out, atol=1e-14)


def test_bhsd_equals_bshd_transposed():
    a = build_case("lay", dtype="bf16", layout="bhsd", B=2, Hq=4, Hkv=2, D=16, q_block=8,
                   kv_block=8, q_var=[8, 5, 8], kv_var=[8, 3, 8, 8], topk=2, map_kind="none",
                   gate_mode="per_element", gate_kind="scaled", seed=9)
    b = build_case("lay", dtype="bf16", layout="bhsd", B=2, Hq=4, Hkv=2, D=16, q_block=8,
                   kv_block=8, q_var=[8, 5, 8], kv_var=[8, 3, 8, 8], topk=2, map_kind="none",
                   gate_mode="per_element", gate_kind="scaled", seed=9)
    b.layout = "bshd"
    for name in ("q", "k", "v", "dout", "gate"):
        setattr(b, name, getattr(a, name).transpose(1, 2).contiguous())
    oa, ob = oracle.Oracle(a), oracle.Oracle(b)
    assert np.array_equal(oa.block_map(), ob.block_map())
    fa, fb = oa.fwd(), ob.fwd()
    np.testing.assert_allclose(fb[0].transpose(0, 2, 1, 3), fa[0], atol=1e-14)
    np.testing.assert_allclose(fb[2], fa[2], atol=1e-14)
    for x, y in zip(oa.bwd(), ob.bwd()):
        np.testing.assert_allclose(y.transpose(0, 2, 1, 3), x, atol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    g = build_case("gqa", dtype="bf16", layout="bhsd", B=1, Hq=6, Hkv=2, D=16, q_block=8,
                   kv_block=8, Sq=24, Skv=32, map_kind="bernoulli", map_p=0.5, seed=13)
    m = build_case("gqa", dtype="bf16", layout="bhsd", B=1, Hq=6, Hkv=6, D=16, q_block=8,
                   kv_block=8, Sq=24, Skv=32, map_kind="custom", map_fn=lambda c: g.block_map)
    m.q, m.dout = g.q, g.dout
    m.k = g.k.repeat_interleave(3, dim=1).contiguous()
    m.v = g.v.repeat_interleave(3, dim=1).contiguous()
    og, om = oracle.Oracle(g), oracle.Oracle(m)
    np.testing.assert_allclose(og.fwd()[0], om.fwd()[0], atol=1e-14)
    dqg, dkg, dvg, _ = og.bwd()
    dqm, dkm, dvm, _ = om.bwd()
    np.testing.assert_allclose(dqg, dqm, atol=1e-13)
    np.testing.assert_allclose(dkg, dkm.reshape(1, 2, 3, 32, 16).sum(2), atol=1e-13)
    np.testing.assert_allclose(dvg, dvm.reshape(1, 2, 3, 32, 16).sum(2), atol=1e-13)


def test_tnd_equals_separate_sequences():
    t = make_case("p3_tnd_uneven")
    ot = oracle.Oracle(t)
    out_t, _, lse_t = ot.fwd()
    dq_t, dk_t, dv_t, _ = ot.bwd()
    cq = np.concatenate([[0], np.cumsum(t.q_lens)])
    ck = np.concatenate([[0], np.cumsum(t.kv_lens)])
    for b in range(t.B):
        ql, kl = t.q_lens[b], t.kv_lens[b]
        s = build_case("one", dtype="fp16", layout="bhsd", B=1, Hq=t.Hq, Hkv=t.Hkv, D=t.D,
                       q_block=t.q_block, kv_block=t.kv_block, Sq=ql, Skv=kl, map_kind="custom",
                       map_fn=lambda c: t.block_map[b:b + 1, :, :c.Qb, :c.KVb])
        s.q = t.q[cq[b]:cq[b + 1]].transpose(0, 1)[None].contiguous()
        s.k = t.k[ck[b]:ck[b + 1]].transpose(0, 1)[None].contiguous()
        s.v = t.v[ck[b]:ck[b + 1]].transpose(0, 1)[None].contiguous()
        s.dout = t.dout[cq[b]:cq[b + 1]].transpose(0, 1)[None].contiguous()
        os_ = oracle.Oracle(s)
        out_s, _, lse_s = os_.fwd()
        dq_s, dk_s, dv_s, _ = os_.bwd()
        np.testing.assert_allclose(out_t[cq[b]:cq[b + 1]], out_s[0].transpose(1, 0, 2), atol=1e-14)
        np.testing.assert_allclose(lse_t[:, cq[b]:cq[b + 1]], lse_s[0], atol=1e-14)
        np.testing.assert_allclose(dq_t[cq[b]:cq[b + 1]], dq_s[0].transpose(1, 0, 2), atol=1e-13)
        np.testing.assert_allclose(dk_t[ck[b]:ck[b + 1]], dk_s[0].transpose(1, 0, 2), atol=1e-13)
        np.testing.assert_allclose(dv_t[ck[b]:ck[b + 1]], dv_s[0].transpose(1, 0, 2), atol=1e-13)


def test_one_live_key_and_block_diagonal():
    # one live key per row: out = v of that key exactly, dq = dk = 0
    case = build_case("one_key", dtype="bf16", B=1, Hq=2, D=8, q_block=4, kv_block=4,
                      q_var=[4, 4], kv_var=[1, 4], map_kind="custom",
                      map_fn=lambda c: torch.tensor([[[[1, 0], [1, 0]], [[1, 0], [1, 0]]]]))
    orc = oracle.Oracle(case)
    out, _, lse = orc.fwd()
    v = orc.v
    assert np.array_equal(out[0, :, :], np.broadcast_to(v[0, :, :1], out[0].shape))
    dq, dk, dv, _ = orc.bwd()
    assert np.abs(dq).max() < 1e-15 and np.abs(dk).max() < 1e-15
    np.testing.assert_allclose(dv[0, :, 0], orc.dout[0].sum(1), atol=1e-14)
    # block-diagonal map = dense attention inside each block pair
    case = build_case("diag", dtype="bf16", B=1, Hq=1, D=8, q_block=4, kv_block=4, Sq=12,
                      Skv=12, map_kind="custom",
                      map_fn=lambda c: torch.eye(3, dtype=torch.uint8)[None, None])
    out = oracle.Oracle(case).fwd()[0]
    for i in range(3):
        sub = build_case("blk", dtype="bf16", B=1, Hq=1, D=8, q_block=4, kv_block=4, Sq=4, Skv=4,
                         map_kind="ones")
        sub.q = case.q[:, :, 4 * i:4 * i + 4].contiguous()
        sub.k = case.k[:, :, 4 * i:4 * i + 4].contiguous()
        sub.v = case.v[:, :, 4 * i:4 * i + 4].contiguous()
        np.testing.assert_allclose(out[:, :, 4 * i:4 * i + 4], oracle.Oracle(sub).fwd()[0],
                                   atol=1e-15)


def test_page_sparse_pattern_equals_one_block_dense():
    """The Ascend page's sparse case selects KV block i mod 2 for Q block i; every
    Q block then attends densely to one 128-key block."""
    case = make_case("p3_bnsd_sparse32")
    out = oracle.Oracle(case).fwd(heads=[(1, 3)])[0]
    q, k, v = (t.double() for t in (case.q, case.k, case.v))
    for i in range(case.Qb):
        j = i % case.KVb
        s = q[1, 3, 32 * i:32 * i + 32] @ k[1, 3, 128 * j:128 * j + 128].T * case.scale
        want = torch.softmax(s, -1) @ v[1, 3, 128 * j:128 * j + 128]
        np.testing.assert_allclose(out[1, 3, 32 * i:32 * i + 32], want.numpy(), atol=1e-13)


def test_empty_row_gives_zero_output_and_no_gradient():
    case = build_case("empty", dtype="bf16", B=1, Hq=1, D=8, q_block=4, kv_block=4, Sq=8, Skv=8,
                      map_kind="custom",
                      map_fn=lambda c: torch.tensor([[[[1, 1], [0, 0]]]], dtype=torch.uint8))
    orc = oracle.Oracle(case)
    out, _, lse = orc.fwd()
    assert np.all(out[0, 0, 4:] == 0) and np.all(np.isneginf(lse[0, 0, 4:]))
    assert np.all(np.isfinite(lse[0, 0, :4]))
    dq, dk, dv, _ = orc.bwd()
    assert np.all(dq[0, 0, 4:] == 0)
    # the rows of Q block 0 alone account for dv
    np.testing.assert_allclose(dv[0, 0].sum(0), orc.dout[0, 0, :4].sum(0), atol=1e-14)


def test_float32_and_float64_oracles_agree():
    case = make_case("c1_vsa256_tiny")
    o32 = oracle.Oracle(case, np.float32)
    o64 = oracle.Oracle(case, np.float64)
    for a, b in zip(o32.fwd(), o64.fwd()):
        assert _rel(a, b) < 1e-5
    for a, b in zip(o32.bwd()[:3], o64.bwd()[:3]):
        assert _rel(a, b) < 1e-4


def test_sampled_rows_match_full_evaluation():
    case = _vsa_small(topk=3, gate_mode="per_token")
    orc = oracle.Oracle(case)
    out, _, lse = orc.fwd()
    dq = orc.bwd()[0]
    rows = np.array([[0, 0, 0], [0, 3, 9], [0, 1, 31], [0, 2, 17]], np.int32)
    o_r, l_r = orc.fwd_rows(rows)
    d_r = orc.dq_rows(rows)
    for n, (b, h, s) in enumerate(rows):
        np.testing.assert_allclose(o_r[n], out[b, s, h], atol=1e-15)  # BSHD
        np.testing.assert_allclose(l_r[n], lse[b, h, s], atol=1e-15)
        np.testing.assert_allclose(d_r[n], dq[b, s, h], atol=1e-14)


def test_sampled_tiles_match_full_backward():
    for gm in ("none", "per_token"):
        case = _vsa_small(topk=3, gate_mode=gm)
        orc = oracle.Oracle(case)
        _, dk, dv, _ = orc.bwd()
        tiles = np.array([[0, 0, 0], [0, 1, 4], [0, 1, 1], [0, 0, 2]], np.int32)
        tk, tv = orc.dkdv_tiles(tiles)
        for n, (b, hk, j) in enumerate(tiles):
            np.testing.assert_allclose(tk[n], dk[b, j * 8:(j + 1) * 8, hk], atol=1e-14)  # BSHD
            np.testing.assert_allclose(tv[n], dv[b, j * 8:(j + 1) * 8, hk], atol=1e-14)


def test_per_entry_valid_counts_equal_separate_runs():
    """Valid counts given per batch entry ([B, tiles]): each entry's out, lse,
    selection and gradients are those of that entry run alone (B = 1) with its
    own counts -- batch entries share nothing but the launch."""
    q_var = [[8, 3, 8], [5, 8, 2]]
    kv_var = [[8, 1, 0, 8, 5], [6, 8, 8, 3, 0]]
    case = build_case("per_entry", dtype="bf16", layout="bshd", B=2, Hq=4, Hkv=2, D=16,
                      q_block=8, kv_block=8, q_var=q_var, kv_var=kv_var, topk=2,
                      map_kind="none", gate_mode="per_token", seed=61)
    orc = oracle.Oracle(case)
    full = orc.fwd()
    grads = orc.bwd()
    m = orc.block_map()
    for b in range(2):
        one = dataclasses.replace(
            case, B=1, q_var=np.asarray(q_var[b], np.int32), kv_var=np.asarray(kv_var[b], np.int32),
            q=case.q[b:b + 1], k=case.k[b:b + 1], v=case.v[b:b + 1], dout=case.dout[b:b + 1],
            gate=case.gate[b:b + 1])
        ref = oracle.Oracle(one)
        assert np.array_equal(m[b:b + 1], ref.block_map()), b
        for got, want in zip(full, ref.fwd()):
            np.testing.assert_allclose(got[b:b + 1], want, rtol=0, atol=1e-15)
        for got, want in zip(grads, ref.bwd()):
            np.testing.assert_allclose(got[b:b + 1], want, rtol=0, atol=1e-15)
    # and the two entries really differ in their counts' effect
    assert not np.array_equal(m[0], m[1])
