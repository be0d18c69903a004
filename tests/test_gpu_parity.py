"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Bars (the spec acceptance): index bit-exact; out and lse avg_abs < 1e-3
and max_rel < 0.2; dq/dk/dv (and dgate) avg_abs < 1e-3 and max_rel < 0.25,
with avg_abs = mean|got-ref| and max_rel = max|got-ref| / max|ref|. Where
several selections are correct (top-k near-ties) the GPU selection is checked
for validity against the oracle's scores and only agreeing rows are compared.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import GRAD_TOL, OUT_TOL, check, metrics
from workloads.synth import build_case, make_case

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # the CPU container collects but skips these
    pytest.skip("needs a GPU", allow_module_level=True)

from tests.gpu_run import device_inputs, problem_for, run_case  # noqa: E402
import bwd_block_map_amd as vsa  # noqa: E402


def _say(*a):
    print(*a, flush=True)


def _topk_agreement(orc, gpu_map):
    """GPU top-k rows must be valid selections under the oracle's scores: every
    selected tile scores at least as high as every unselected one, up to a
    near-tie margin. Returns a [B,H,Qb] mask of rows identical to the oracle's."""
    omap = orc.block_map()
    same = (omap == gpu_map).all(-1)
    if same.all():
        return same
    C = orc.coarse_scores()
    for b, h, i in zip(*np.nonzero(~same)):
        row = C[b, h, i]
        valid = np.isfinite(row)
        sel = gpu_map[b, h, i].astype(bool)
        assert sel.sum() == omap[b, h, i].sum(), "selection size differs"
        eps = 1e-5 * np.abs(row[valid]).max()
        lo = row[sel & valid].min()
        hi = row[~sel & valid].max() if (~sel & valid).any() else -np.inf
        assert lo >= hi - eps, f"invalid top-k row {(b, h, i)}: {lo} < {hi}"
    return same


def _compare_case(case, res, orc, *, rows_ok=None, tol_out=OUT_TOL, tol_grad=GRAD_TOL):
    out, osel, lse = orc.fwd()
    dt = case.dtype  # out and the gradients are stored in it; lse is float
    check("out", out, res["out"], tol_out, dt)
    lse_g = res["lse"]
    fin = np.isfinite(lse)
    assert np.array_equal(fin, np.isfinite(lse_g)), "empty rows differ"
    check("lse", lse[fin], lse_g[fin], tol_out)
    if "dq" in res:
        dq, dk, dv, dg = orc.bwd()
        check("dq", dq, res["dq"], tol_grad, dt)
        check("dk", dk, res["dk"], tol_grad, dt)
        check("dv", dv, res["dv"], tol_grad, dt)
        if dg is not None and res.get("dgate") is not None:
            # the projected gate's parameter gradient is stored in float
            check("dgate", dg, res["dgate"], tol_grad,
                  None if case.gate_mode == "projected" else dt)


SMALL = [
    ("c1_vsa256_tiny", dict(layout="bhsd")),
    ("c1_vsa256_tiny", dict(layout="bshd")),
    ("p1_fwd_bwd", dict(layout="bhsd")),
    ("p1_fwd_bwd", dict(layout="bshd")),
    ("p1_gated", dict(layout="bhsd")),
    ("p1_gated", dict(layout="bshd")),
    ("p1_partial_q", dict(layout="bhsd")),
    ("p1_partial_q", dict(layout="bshd")),
    ("p1_cross", dict(layout="bhsd")),
    ("p1_cross", dict(layout="bshd")),
    ("p3_bnsd_fp16", {}),
    ("p3_bnsd_bf16", {}),
    ("p3_bnsd_sparse32", {}),
    ("p3_bnsd_q8", {}),
    ("p3_bnsd_q16", {}),
    ("p3_tnd_full", {}),
    ("p3_tnd_sparse", {}),
    ("p3_tnd_single", {}),
    ("p3_tnd_uneven", {}),
    ("p3_tnd_group4", {}),
    ("p3_tnd_mqa", {}),
    ("p3_tnd_tail64", {}),
    ("p3_tnd_q8", {}),
    ("p3_bnsd_kv64", {}),
    ("p3_tnd_kv192", {}),
    ("p3_tnd_kv320", {}),
    ("p3_bnsd_kv512", {}),
    ("c3_tnd_gqa", {}),
    ("c3_tnd_gqa_page", {}),
]


@pytest.mark.parametrize("name,kw", SMALL, ids=[f"{n}-{k.get('layout', '')}" for n, k in SMALL])
def test_fwd_bwd_parity_small(name, kw):
    case = make_case(name, **kw)
    _say(f"[{name} {kw}] B={case.B} Hq={case.Hq} Hkv={case.Hkv} Sq={case.Sq} Skv={case.Skv}")
    res = run_case(case)
    orc = oracle.Oracle(case, np.float32)
    if case.topk > 0:
        same = _topk_agreement(orc, res["map"])
        assert same.all(), "top-k near-tie in a small case"
    _compare_case(case, res, orc)


@pytest.mark.parametrize("name,kw", SMALL, ids=[f"{n}-{k.get('layout', '')}" for n, k in SMALL])
def test_atomic_dq_parity_small(name, kw):
    """The backward variant that adds dQ = dS K inside the KV-owned dK/dV walk
    with float atomics (VSA_FLAG_ATOMIC_DQ), on every small case."""
    case = make_case(name, **kw)
    _say(f"[atomic dq {name} {kw}] B={case.B} Hq={case.Hq} Hkv={case.Hkv} Sq={case.Sq}")
    res = run_case(case, atomic_dq=True)
    orc = oracle.Oracle(case, np.float32)
    if case.topk > 0:
        assert _topk_agreement(orc, res["map"]).all(), "top-k near-tie in a small case"
    _compare_case(case, res, orc)


def test_atomic_dq_edge_cases():
    """Atomic dQ on the cases that stress its masking: zero-q/zero-dO rows past
    each block's live extent (61 and 199 valid rows, a tile without valid rows),
    KV spans of 256, 100 and 64 live keys (the last two in the 128-key shape),
    an empty KV tile, empty rows and block lists longer than one LDS page; the
    gradient of a row with no live key must be zero."""
    cases = [
        build_case("aq_zero_rows", dtype="bf16", layout="bshd", B=1, Hq=2, Hkv=1, D=128,
                   q_var=[61, 256, 199, 0], kv_var=[256, 100, 64, 256], map_kind="ones",
                   seed=23),
        build_case("aq_empty_kv", dtype="fp16", layout="bhsd", B=1, Hq=4, Hkv=2, D=128,
                   q_var=[256, 130, 256], kv_var=[256, 0, 100, 0, 64], topk=4, map_kind="none",
                   gate_mode="per_token", seed=37),
        build_case("aq_empty_rows", dtype="bf16", B=1, Hq=2, Hkv=1, D=128, q_block=128,
                   kv_block=128, Sq=384, Skv=512, map_kind="custom",
                   map_fn=lambda c: torch.tensor([[[[1, 0, 1, 0], [0, 0, 0, 0], [0, 1, 0, 0]],
                                                   [[0, 0, 0, 0], [1, 1, 0, 0], [1, 0, 0, 0]]]])),
        build_case("aq_long_kv_list", dtype="bf16", layout="bhsd", B=1, Hq=2, Hkv=1, D=128,
                   q_block=256, kv_block=64, Sq=256, Skv=64 * 1040, map_kind="ones", seed=23),
    ]
    for case in cases:
        _say(f"[{case.name}]")
        res = run_case(case, atomic_dq=True)
        _compare_case(case, res, oracle.Oracle(case, np.float32))
        if case.name == "aq_empty_rows":  # head 0, Q block 1 selects nothing
            assert np.all(res["dq"][0, 0, 128:256] == 0)


def test_persistent_dkdv_grid_is_bit_identical():
    """The persistent, longest-first dK/dV grid (VSA_FLAG_PERSISTENT) gives
    exactly the outputs and gradients of one work-group per span: every span
    is computed by the same code whichever work-group takes it. Spans of all
    three shapes, GQA, TND, empty tiles, skipped rows, the atomic-dQ
    combination and the two video workloads at full size."""
    cases = [make_case(n, **kw) for n, kw in (("p1_gated", dict(layout="bshd")),
                                              ("p3_tnd_kv320", {}), ("c3_tnd_gqa", {}),
                                              ("c2_bnsd_mha", {}))]
    cases.append(build_case("pers_mixed", dtype="bf16", layout="bshd", B=1, Hq=4, Hkv=2, D=128,
                            q_var=[61, 256, 199, 0], kv_var=[256, 100, 0, 64, 256],
                            topk=3, map_kind="none", gate_mode="per_token", seed=29))
    for case in cases:
        d = device_inputs(case)
        for atomic in (False, True):  # each against the same variant with one group per span
            ref = run_case(case, d=d, keep_device=True, atomic_dq=atomic, persistent=False)
            got = run_case(case, d=d, keep_device=True, persistent=True, atomic_dq=atomic)
            names = ("out", "lse", "dk", "dv") if atomic else ("out", "lse", "dq", "dk", "dv", "dgate")
            for n in names:
                if ref[n] is not None:
                    assert torch.equal(ref[n], got[n]), (case.name, atomic, n)
            if atomic:  # dq differs only by the order of the float additions
                a = metrics(ref["dq"].float().cpu().numpy(), got["dq"].float().cpu().numpy())
                assert a[0] < 1e-4 and a[1] < 1e-2, (case.name, a)
        _say(f"[{case.name}] persistent dK/dV grid identical")
    for name in ("c4_vsa256_video", "c5_vsa256_720p_gate"):
        case = make_case(name, device="cuda")
        d = device_inputs(case)
        ref = run_case(case, d=d, keep_device=True, persistent=False)
        got = run_case(case, d=d, keep_device=True, persistent=True)
        for n in ("out", "lse", "dq", "dk", "dv", "dgate"):
            if ref[n] is not None:
                assert torch.equal(ref[n], got[n]), (name, n)
        _say(f"[{name}] persistent dK/dV grid identical")
        del d, ref, got, case
        torch.cuda.empty_cache()


def _index_cases():
    for n in ("c1_vsa256_tiny", "c2_bnsd_mha", "c3_tnd_gqa", "c3_tnd_gqa_page", "p3_tnd_uneven",
              "p3_bnsd_sparse32", "p3_tnd_tail64", "p3_bnsd_q8", "p3_tnd_q8"):
        yield make_case(n)
    # empty KV tiles, an all-zero row and a 3-D (batch-shared) map
    yield build_case("idx_empty", B=2, Hq=2, D=128, q_block=64, kv_block=64,
                     q_var=[64, 64, 10], kv_var=[64, 0, 7, 0, 64], map_kind="bernoulli",
                     map_p=0.6, seed=3)
    # over 8192 rows and a million map entries in both directions: the
    # multi-launch build (the cases above take the one-launch one)
    yield build_case("idx_big", B=1, Hq=8, D=128, q_block=8, kv_block=64, Sq=8800, Skv=8800,
                     map_kind="bernoulli", map_p=0.1, seed=5)


@pytest.mark.parametrize("case", list(_index_cases()), ids=lambda c: c.name)
def test_block_index_bit_exact(case):
    d = device_inputs(case)
    p = problem_for(case, d)
    cap = vsa.vsa_sizes(p)["nnz_capacity"]
    bmap = case.block_map.numpy()
    for kv_owned in (False, True):
        rows = case.B * case.Hq * (case.KVb if kv_owned else case.Qb)
        rp = torch.full((rows + 1,), -7, dtype=torch.int32, device="cuda")
        col = torch.full((max(cap, 1),), -7, dtype=torch.int32, device="cuda")
        vsa.block_map_to_index(p, d["map"], kv_owned, rp, col, cap)
        torch.cuda.synchronize()
        want_rp, want_col = oracle.block_index(case, bmap, kv_owned)
        got_rp = rp.cpu().numpy()
        assert np.array_equal(got_rp, want_rp)
        assert np.array_equal(col.cpu().numpy()[:got_rp[-1]], want_col)


def test_block_index_shared_map_over_batch():
    case = build_case("idx_shared", B=3, Hq=2, D=128, q_block=128, kv_block=128, Sq=300,
                      Skv=700, map_kind="bernoulli", map_p=0.5, seed=9)
    shared = case.block_map[:1].contiguous()
    d = device_inputs(case)
    p = problem_for(case, d, map_batch_stride=0)
    cap = vsa.vsa_sizes(p)["nnz_capacity"]
    rp = torch.zeros(case.B * case.Hq * case.Qb + 1, dtype=torch.int32, device="cuda")
    col = torch.zeros(cap, dtype=torch.int32, device="cuda")
    vsa.block_map_to_index(p, shared.cuda(), False, rp, col, cap)
    want_rp, want_col = oracle.block_index(case, shared.expand(3, -1, -1, -1).numpy().copy(), False)
    assert np.array_equal(rp.cpu().numpy(), want_rp)
    assert np.array_equal(col.cpu().numpy()[:want_rp[-1]], want_col)


def test_inference_forward_equals_training_forward():
    case = make_case("p1_infer", layout="bshd")
    d = device_inputs(case)
    a = run_case(case, training=False, backward=False, d=d, keep_device=True)
    b = run_case(case, training=True, backward=False, d=d, keep_device=True)
    assert torch.equal(a["out"], b["out"]) and torch.equal(a["lse"], b["lse"])
    g = make_case("p1_gated", layout="bshd")
    dg = device_inputs(g)
    a = run_case(g, training=False, backward=False, d=dg, keep_device=True)
    b = run_case(g, training=True, backward=False, d=dg, keep_device=True)
    assert torch.equal(a["out"], b["out"]) and torch.equal(a["lse"], b["lse"])


def _as_bshd(case):
    """The same case with every q/kv-shaped tensor transposed to [B,S,H,D]."""
    import copy
    b = copy.copy(case)
    b.layout = "bshd"
    for n in ("q", "k", "v", "dout", "gate"):
        t = getattr(case, n)
        if t is not None:
            setattr(b, n, (t.transpose(1, 2) if t.dim() == 4 else t.transpose(1, 2)).contiguous())
    return b


def test_zero_query_rows_of_a_block_share_one_output():
    """Padded slots of partial video tiles hold zero queries. Such rows go
    through identical arithmetic, so every one of them in a block has the same
    output and LSE, whether its wave computed it or copied it from the block's
    leading all-zero wave (the 61-valid tile: rows 61-63 are computed in a
    wave with live rows, rows 64-255 by one wave and copied to five). The
    oracle comparison of the same case is in test_fwd_bwd_parity_small."""
    for layout in ("bhsd", "bshd"):
        case = make_case("p1_partial_q", layout=layout)
        res = run_case(case, backward=False)
        out = res["out"] if layout == "bhsd" else res["out"].transpose(0, 2, 1, 3)
        lse = res["lse"]
        for i, qv in enumerate(case.q_var.tolist()):
            if qv == 256:
                continue
            rows = slice(i * 256 + qv, (i + 1) * 256)
            o, l = out[:, :, rows], lse[:, :, rows]
            assert np.array_equal(o, np.broadcast_to(o[:, :, :1], o.shape)), (layout, i)
            assert np.array_equal(l, np.broadcast_to(l[:, :, :1], l.shape)), (layout, i)
            assert np.isfinite(l).all()


def test_rows_with_zero_query_and_zero_gradient_are_skipped_exactly():
    """Partial query tiles whose padded slots hold zero q and zero dO (a
    training caller passes no gradient for padded outputs): those rows have
    dS = 0, so the backward stops each block's walk at its last live row and
    skips dQ waves past it. The tiles' valid counts (61, 199) end in the middle
    of a 32-, 64- and 128-row chunk of the three dK/dV span shapes (256, 100
    and 64 live keys), and a tile without valid rows is passed over; results
    must still match the oracle, with dq exactly zero on the padded rows."""
    for dtype, layout in (("bf16", "bshd"), ("fp16", "bhsd")):
        case = build_case(f"zero_rows_{dtype}_{layout}", dtype=dtype, layout=layout, B=1, Hq=2,
                          Hkv=1, D=128, q_var=[61, 256, 199, 0], kv_var=[256, 100, 64, 256],
                          map_kind="ones", seed=23)
        _say(f"[{case.name}]")
        res = run_case(case)
        _compare_case(case, res, oracle.Oracle(case, np.float32))
        dq = res["dq"] if layout == "bhsd" else res["dq"].transpose(0, 2, 1, 3)
        for i, qv in enumerate(case.q_var.tolist()):
            assert np.all(dq[:, :, i * 256 + qv:(i + 1) * 256] == 0), (case.name, i)


def test_rows_with_zero_gradient_and_nonzero_query_are_skipped_exactly():
    """The backward's live extent follows dO alone: padded slots with a
    non-zero query but a zero gradient (dP = 0 and Dr = 0, so dS = 0) are
    skipped like all-zero ones, and dq stays exactly zero there."""
    case = build_case("zero_grad_rows", dtype="bf16", layout="bshd", B=1, Hq=2, Hkv=1, D=128,
                      q_var=[61, 256, 199], kv_var=[256, 100, 64], map_kind="ones", seed=29)
    # queries in the padded slots (the gradient there stays zero)
    pad = np.concatenate([np.arange(i * 256 + n, (i + 1) * 256) for i, n in enumerate(case.q_var.tolist())])
    noise = torch.randn(case.q.shape, generator=torch.Generator().manual_seed(31)).to(case.q.dtype)
    q = case.q.clone()
    q[:, pad] = noise[:, pad]
    case = dataclasses.replace(case, q=q)
    _say(f"[{case.name}]")
    assert float(case.dout[:, pad].abs().max()) == 0 and float(case.q[:, pad].abs().max()) > 0
    res = run_case(case)
    _compare_case(case, res, oracle.Oracle(case, np.float32))
    dq = res["dq"].transpose(0, 2, 1, 3)
    for i, qv in enumerate(case.q_var.tolist()):
        assert np.all(dq[:, :, i * 256 + qv:(i + 1) * 256] == 0), i


@pytest.mark.parametrize("q_lens,kv_lens", [([20, 50], [0, 40]), ([0, 50, 7], [30, 0, 9])],
                         ids=["no_keys", "no_queries_and_no_keys"])
def test_tnd_sequences_of_length_zero(q_lens, kv_lens):
    """Packed sequences without queries or without keys: a sequence with no
    keys gives rows without a live key (out = 0, lse = -inf, dq = 0), one with
    no queries contributes nothing, and the other sequences are unaffected."""
    case = build_case("tnd_empty", dtype="bf16", layout="tnd", Hq=2, Hkv=1, D=128, q_block=32,
                      kv_block=64, q_lens=q_lens, kv_lens=kv_lens, map_kind="ones", seed=3)
    _say(f"[tnd_empty] q_lens={q_lens} kv_lens={kv_lens}")
    res = run_case(case)
    _compare_case(case, res, oracle.Oracle(case, np.float32))


@pytest.mark.parametrize("gate_mode", ["per_token", "projected"])
def test_batch_entry_without_any_key(gate_mode):
    """Per-entry valid counts where one batch entry has no valid key at all:
    its coarse softmax has an empty domain (lse_c = -inf, O_c = 0), top-k
    selects nothing, its rows come out as zero with lse = -inf and zero
    gradients, and the other entry is unaffected."""
    case = build_case("no_keys_entry", dtype="bf16", layout="bshd", B=2, Hq=2, Hkv=1, D=128,
                      q_var=[[256, 61], [256, 256]], kv_var=[[256, 0, 100], [0, 0, 0]], topk=2,
                      map_kind="none", gate_mode=gate_mode, seed=41)
    _say(f"[no_keys_entry {gate_mode}]")
    res = run_case(case)
    orc = oracle.Oracle(case, np.float32)
    assert _topk_agreement(orc, res["map"]).all()
    _compare_case(case, res, orc)
    assert not res["map"][1].any()


def test_bhsd_and_bshd_are_bit_identical():
    a = make_case("p1_gated", layout="bhsd")
    b = _as_bshd(a)
    ra, rb = run_case(a), run_case(b)
    assert np.array_equal(ra["out"], rb["out"].transpose(0, 2, 1, 3))
    assert np.array_equal(ra["lse"], rb["lse"])
    for n in ("dq", "dk", "dv", "dgate"):
        assert np.array_equal(ra[n], rb[n].transpose(0, 2, 1, 3)), n


def test_runs_are_deterministic():
    case = make_case("c3_tnd_gqa")
    d = device_inputs(case)
    r1 = run_case(case, d=d, keep_device=True)
    r2 = run_case(case, d=d, keep_device=True)
    for n in ("out", "lse", "dq", "dk", "dv"):
        assert torch.equal(r1[n], r2[n]), n


def test_missing_dout_gives_zero_gradients():
    case = make_case("p1_gated", layout="bshd")
    res = run_case(case, dout_none=True)
    for n in ("dq", "dk", "dv", "dgate"):
        assert np.all(res[n] == 0), n


def test_empty_rows_and_unselected_tiles():
    case = build_case("empty_rows", dtype="bf16", B=1, Hq=2, Hkv=1, D=128, q_block=128,
                      kv_block=128, Sq=384, Skv=512, map_kind="custom",
                      map_fn=lambda c: torch.tensor([[[[1, 0, 1, 0], [0, 0, 0, 0], [0, 1, 0, 0]],
                                                      [[0, 0, 0, 0], [1, 1, 0, 0], [1, 0, 0, 0]]]]))
    res = run_case(case)
    assert np.all(res["out"][0, 0, 128:256] == 0) and np.all(np.isneginf(res["lse"][0, 0, 128:256]))
    assert np.all(res["dq"][0, 0, 128:256] == 0)
    assert np.all(res["dk"][0, 0, 384:] == 0) and np.all(res["dv"][0, 0, 384:] == 0)
    _compare_case(case, res, oracle.Oracle(case, np.float32))


def test_ragged_tails_and_q_block_64():
    case = build_case("ragged", dtype="fp16", layout="bshd", B=2, Hq=4, Hkv=2, D=128,
                      q_block=64, kv_block=128, Sq=300, Skv=333, map_kind="bernoulli",
                      map_p=0.5, seed=17)
    _compare_case(case, run_case(case), oracle.Oracle(case, np.float32))


def test_ragged_tails_and_q_blocks_8_and_16():
    for qb in (8, 16):
        case = build_case(f"ragged_q{qb}", dtype="bf16", layout="bshd", B=2, Hq=4, Hkv=2, D=128,
                          q_block=qb, kv_block=128, Sq=100, Skv=333, map_kind="bernoulli",
                          map_p=0.4, seed=19 + qb)
        _say(f"[ragged q_block={qb}]")
        _compare_case(case, run_case(case), oracle.Oracle(case, np.float32))


def test_video_tiles_with_shared_kv_heads():
    """Pooled-score top-k and the gated compression branch with 4 query heads
    on 2 KV heads: coarse scores per query head against the shared pooled K,
    dK_c / dV_c and the sparse dK / dV summed over each KV head's group; also
    two batch entries in fp16 (a map per batch entry)."""
    for dtype, layout, B, gate in (("bf16", "bshd", 1, "per_token"), ("bf16", "bshd", 1, "per_element"),
                                   ("fp16", "bhsd", 2, "per_token")):
        case = build_case(f"video_gqa_{dtype}_{layout}_b{B}_{gate}", dtype=dtype, layout=layout, B=B,
                          Hq=4, Hkv=2, D=128, q_var=[256, 256, 97, 256],
                          kv_var=[256, 64, 256, 173, 16], topk=3, map_kind="none", gate_mode=gate,
                          gate_kind="sigmoid", seed=31)
        _say(f"[{case.name}]")
        res = run_case(case)
        orc = oracle.Oracle(case, np.float32)
        assert _topk_agreement(orc, res["map"]).all(), "top-k near-tie in a small case"
        _compare_case(case, res, orc)


def test_host_pointers_are_rejected_before_any_launch():
    """The C ABI itself (not only the Python wrapper) refuses a plain host
    pointer for a tensor or for a valid-count array, with INVALID_ARG."""
    import ctypes as C
    case = make_case("c1_vsa256_tiny")
    d = device_inputs(case)
    p = problem_for(case, d)
    buf = vsa.Buffers(p, d["q"], training=True)
    bmap = d["map"] if case.topk == 0 else buf.map
    assert case.gate_mode == "none"
    host_q = d["q"].cpu()
    L = vsa.lib()

    def fwd(prob, q):
        return L.vsa_fwd(prob.ref, C.c_void_p(q.data_ptr()), C.c_void_p(d["k"].data_ptr()),
                         C.c_void_p(d["v"].data_ptr()), C.c_void_p(bmap.data_ptr()), None,
                         C.c_void_p(buf.out.data_ptr()), C.c_void_p(buf.lse.data_ptr()),
                         C.c_void_p(buf.saved.data_ptr()), C.c_size_t(buf.saved.numel()),
                         C.c_void_p(buf.ws_fwd.data_ptr()), C.c_size_t(buf.ws_fwd.numel()),
                         C.c_void_p(torch.cuda.current_stream().cuda_stream))

    assert fwd(p, host_q) == vsa.ERR_INVALID_ARG
    assert vsa.vsa_last_error() == "q must be a device tensor"
    host_kv = d["kv_valid"].cpu()
    p2 = problem_for(case, dict(d, kv_valid=host_kv))
    assert fwd(p2, d["q"]) == vsa.ERR_INVALID_ARG
    assert vsa.vsa_last_error() == "kv_valid must be a device tensor"
    assert fwd(p, d["q"]) == vsa.OK  # the same call with device memory runs
    torch.cuda.synchronize()


def test_block_lists_longer_than_one_page():
    """More than 1024 selected blocks per row: the Q-owned walk (forward, dQ)
    and the KV-owned walk (dK/dV) page their block lists through LDS; GQA makes
    dK/dV walk a second head after the first one's pages."""
    cases = [
        build_case("long_kv_list", dtype="bf16", layout="bhsd", B=1, Hq=2, Hkv=1, D=128,
                   q_block=256, kv_block=64, Sq=256, Skv=64 * 1040, map_kind="ones", seed=23),
        build_case("long_q_list", dtype="fp16", layout="bshd", B=1, Hq=2, Hkv=1, D=128,
                   q_block=32, kv_block=64, Sq=32 * 1040, Skv=128, map_kind="ones", seed=29),
    ]
    for case in cases:
        _say(f"[{case.name}] Qb={case.Qb} KVb={case.KVb}")
        _compare_case(case, run_case(case), oracle.Oracle(case, np.float32))


def test_c2_full_size_sampled_heads():
    """BNSD S=4096 at its full size; the oracle evaluates two whole heads."""
    case = make_case("c2_bnsd_mha")
    res = run_case(case)
    orc = oracle.Oracle(case, np.float32)
    heads = [(0, 1), (1, 6)]
    out, _, lse = orc.fwd(heads=heads)
    dq, dk, dv, _ = orc.bwd(groups=heads)
    for b, h in heads:
        _say(f"[c2 head {b},{h}]")
        check("out", out[b, h], res["out"][b, h], OUT_TOL)
        check("lse", lse[b, h], res["lse"][b, h], OUT_TOL)
        check("dq", dq[b, h], res["dq"][b, h], GRAD_TOL)
        check("dk", dk[b, h], res["dk"][b, h], GRAD_TOL)
        check("dv", dv[b, h], res["dv"][b, h], GRAD_TOL)


def test_empty_kv_tiles_and_topk_above_the_live_tiles():
    """KV tiles without a valid token (kv_var = 0) are never selected, never
    attended and get zero gradients; topk above the number of non-empty tiles
    selects every non-empty tile. GQA with the per-token gate, so the coarse
    softmax also runs over the non-empty tiles only."""
    for layout in ("bshd", "bhsd"):
        case = build_case(f"empty_kv_topk_{layout}", dtype="bf16", layout=layout, B=1, Hq=4,
                          Hkv=2, D=128, q_var=[256, 130, 256], kv_var=[256, 0, 100, 0, 64],
                          topk=4, map_kind="none", gate_mode="per_token", seed=37)
        _say(f"[{case.name}]")
        res = run_case(case)
        m = res["map"]
        assert np.all(m[..., [1, 3]] == 0) and np.all(m[..., [0, 2, 4]] == 1)
        orc = oracle.Oracle(case, np.float32)
        assert np.array_equal(orc.block_map(), m)
        _compare_case(case, res, orc)
        dk = res["dk"] if layout == "bhsd" else res["dk"].transpose(0, 2, 1, 3)
        dv = res["dv"] if layout == "bhsd" else res["dv"].transpose(0, 2, 1, 3)
        for j in (1, 3):
            assert np.all(dk[:, :, j * 256:(j + 1) * 256] == 0) and \
                np.all(dv[:, :, j * 256:(j + 1) * 256] == 0), (layout, j)


def _projected_cases():
    # GQA, top-k, two batch entries, a partial Q tile, an empty and a short KV tile
    yield build_case("proj_gqa_bshd", dtype="bf16", layout="bshd", B=2, Hq=4, Hkv=2, D=128,
                     q_var=[256, 61, 256], kv_var=[256, 0, 200, 256, 17], topk=3,
                     map_kind="none", gate_mode="projected", seed=51)
    # BHSD fp16 with unpadded inputs: padded q rows are live and get their own gate
    yield build_case("proj_bhsd_fp16", dtype="fp16", layout="bhsd", B=1, Hq=2, Hkv=2, D=128,
                     q_var=[256, 100], kv_var=[256, 256, 31], topk=2, map_kind="none",
                     gate_mode="projected", pad_inputs=False, seed=52)
    # a caller-given map, MQA, a ragged Q tail (q_var not given: whole tiles)
    yield build_case("proj_map_mqa", dtype="bf16", layout="bshd", B=1, Hq=3, Hkv=1, D=128,
                     q_block=128, kv_block=128, Sq=300, Skv=520, map_kind="per_row",
                     map_per_row=2, gate_mode="projected", seed=53)


@pytest.mark.parametrize("atomic_dq", [False, True], ids=["two_pass", "atomic_dq"])
@pytest.mark.parametrize("case", list(_projected_cases()), ids=lambda c: c.name)
def test_projected_gate_parity(case, atomic_dq):
    """The gate projected from the query rows, sigmoid(<q, w_h> + b_h): the
    gate values the forward writes, out, lse and every gradient, the
    parameter gradient [dw | db] included, against the oracle in fp32."""
    _say(f"[{case.name} atomic_dq={atomic_dq}] B={case.B} Hq={case.Hq} Sq={case.Sq}")
    res = run_case(case, atomic_dq=atomic_dq)
    orc = oracle.Oracle(case, np.float32)
    if case.topk > 0:
        assert _topk_agreement(orc, res["map"]).all(), "top-k near-tie in a small case"
    gv = orc.gate_values()
    # the gate values are rounded to the element type once
    check("gate", gv, res["gate_vals"], (2e-3, 1e-2))
    _compare_case(case, res, orc)
    # [dw | db] is an fp32 sum of fp32 terms on both sides: a much tighter bar
    dth = orc.bwd()[3]
    avg_abs, max_rel = metrics(dth, res["dgate"])
    _say(f"  dtheta avg_abs={avg_abs:.3e} max_rel={max_rel:.3e}")
    assert max_rel < 1e-4, (avg_abs, max_rel)


def test_projected_gate_without_dout_and_gate_output():
    """dout = NULL gives zero gradients, [dw | db] included; the forward may
    leave the gate values unwritten (gate = NULL) and then gives the same out."""
    case = next(_projected_cases())
    res = run_case(case, dout_none=True)
    for n in ("dq", "dk", "dv", "dgate"):
        assert np.all(res[n] == 0), n
    d = device_inputs(case)
    p = problem_for(case, d)
    buf = vsa.Buffers(p, d["q"], training=False)
    vsa.vsa_fwd(p, d["q"], d["k"], d["v"], None, None, buf.out, buf.lse, None, buf.ws_fwd)
    torch.cuda.synchronize()
    assert np.array_equal(buf.out.float().cpu().numpy(), res["out"])


def test_per_entry_valid_counts():
    """Valid counts per batch entry ([B, tiles], the stride fields of the
    problem): pooled top-k with the gate in BSHD, and a caller map in BHSD
    fp16 with an entry whose Q tile and KV tile are empty."""
    cases = [
        build_case("per_entry_gated", dtype="bf16", layout="bshd", B=2, Hq=4, Hkv=2, D=128,
                   q_var=[[256, 61, 256], [100, 256, 17]],
                   kv_var=[[256, 0, 200, 256, 17], [64, 256, 256, 0, 130]], topk=3,
                   map_kind="none", gate_mode="per_token", seed=71),
        build_case("per_entry_map", dtype="fp16", layout="bhsd", B=3, Hq=2, Hkv=1, D=128,
                   q_var=[[256, 256], [0, 200], [31, 256]],
                   kv_var=[[256, 99, 256], [256, 256, 0], [1, 256, 64]], map_kind="per_row",
                   map_per_row=2, seed=72),
    ]
    for case in cases:
        _say(f"[{case.name}] B={case.B} q_var={case.q_var.tolist()} kv_var={case.kv_var.tolist()}")
        res = run_case(case)
        orc = oracle.Oracle(case, np.float32)
        if case.topk > 0:
            assert _topk_agreement(orc, res["map"]).all(), "top-k near-tie in a small case"
        _compare_case(case, res, orc)


def _small_head_cases():
    # D = 64: VSA tiles with top-k and the per-token gate, GQA, BSHD
    yield build_case("d64_gated", dtype="bf16", layout="bshd", B=1, Hq=4, Hkv=2, D=64,
                     q_var=[256, 61, 256], kv_var=[256, 0, 200, 256, 17], topk=3,
                     map_kind="none", gate_mode="per_token", seed=81)
    # D = 96: caller map, ragged tails, fp16 BHSD, a q-shaped gate
    yield build_case("d96_elem", dtype="fp16", layout="bhsd", B=2, Hq=2, Hkv=1, D=96,
                     q_block=64, kv_block=128, Sq=300, Skv=333, map_kind="bernoulli", map_p=0.5,
                     gate_mode="per_element", gate_kind="scaled", seed=82)
    # D = 40: the projected gate
    yield build_case("d40_proj", dtype="bf16", layout="bshd", B=1, Hq=2, Hkv=2, D=40,
                     q_var=[256, 100], kv_var=[256, 256, 31], topk=2, map_kind="none",
                     gate_mode="projected", seed=83)
    # D = 8: TND varlen GQA
    yield build_case("d8_tnd", dtype="bf16", layout="tnd", Hq=4, Hkv=2, D=8, q_block=128,
                     kv_block=128, q_lens=[65, 300, 7], kv_lens=[129, 400, 90],
                     map_kind="bernoulli", map_p=0.6, seed=84)


@pytest.mark.parametrize("case", list(_small_head_cases()), ids=lambda c: c.name)
def test_head_dimensions_below_128(case):
    """D < 128 runs the 128-column kernels on zero-widened copies: every output
    and gradient (the projection's [dw | db] included) against the oracle at
    the case's own D."""
    _say(f"[{case.name}] D={case.D} layout={case.layout}")
    res = run_case(case)
    orc = oracle.Oracle(case, np.float32)
    if case.topk > 0:
        assert _topk_agreement(orc, res["map"]).all(), "top-k near-tie in a small case"
    _compare_case(case, res, orc)
    if case.gate_mode == "projected":
        check("gate", orc.gate_values(), res["gate_vals"], (2e-3, 1e-2))


def test_many_kv_tiles_at_the_coarse_kernels_limits():
    """Pooled top-k over very many KV tiles, where the coarse forward holds only
    a few score rows per work-group: the gated path with 1001 (a tile count
    that is not a multiple of 4 or 16), 2640, 8000, 12000 and 36000 KV tiles
    (16, 8, 4, 2 and 1 rows per work-group; the compression backward's LDS
    does not grow with the tile count) and top-k alone at 20000 tiles (1.28 M
    keys, one row), against the oracle (selection exact, outputs and gradients
    within the bars)."""
    cases = [
        build_case(f"many_kv_gated_{n}", dtype="bf16", layout="bshd", B=1, Hq=2, Hkv=1, D=128,
                   q_block=256, kv_block=64, Sq=512, Skv=64 * n, topk=6, map_kind="none",
                   gate_mode="per_token", seed=95 + n)
        for n in (1001, 2640, 8000, 12000, 36000)
    ] + [
        build_case("many_kv_topk", dtype="bf16", layout="bhsd", B=1, Hq=1, Hkv=1, D=128,
                   q_block=256, kv_block=64, Sq=256, Skv=64 * 20000, topk=8, map_kind="none",
                   seed=96),
    ]
    for case in cases:
        _say(f"[{case.name}] KVb={case.KVb} topk={case.topk} gate={case.gate_mode}")
        res = run_case(case)
        orc = oracle.Oracle(case, np.float32, threads=16)
        assert _topk_agreement(orc, res["map"]).all(), "top-k near-tie"
        _compare_case(case, res, orc)
        del res, orc, case
        torch.cuda.empty_cache()
