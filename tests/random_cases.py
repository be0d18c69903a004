"""Seeded random problems for parity beyond the fixed cases.

Each index draws, from its own numpy generator, one problem of one of three
kinds (index % 3): video tiles with per-tile valid counts (optionally per batch
entry), pooled-score top-k (at times above the live tile count) and a
compression gate of a random form; plain BHSD/BSHD sequences with a ragged last
block and either a Bernoulli block map or top-k; packed TND sequences of random
lengths. Block shapes, head groupings, head dimensions, dtypes, whether the
padded slots of dO are zero, and the backward variant (two passes or atomic dQ;
span grid or persistent) are drawn too. Sizes stay small enough for the oracle
to finish each problem in seconds.
"""

from __future__ import annotations

import numpy as np

from workloads.synth import build_case

N_CASES = 120  # problems 36 .. 119 are larger (more tiles, blocks and heads)


def _counts(rng, tiles, tile, batch):
    """Valid tokens per tile: mostly full tiles, some partial, at times empty."""
    shape = (batch, tiles) if batch else (tiles,)
    full = rng.random(shape) < 0.6
    part = rng.integers(0, tile, shape)
    return np.where(full, tile, part).astype(np.int32)


def random_case(i: int):
    """Problem i: (case, run options) with run options {atomic_dq, persistent}."""
    rng = np.random.default_rng(7100 + i)
    kind = ("video", "plain", "tnd")[i % 3]
    big = i >= 36
    dtype = ("bf16", "fp16")[int(rng.integers(2))]
    D = int(rng.choice([128, 128, 128, 96, 64, 40]))
    Hkv = int(rng.integers(1, 5 if big else 3))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    seed = 500 + i
    if kind == "video":
        tile = int(rng.choice([64, 128, 256]))
        B = int(rng.integers(1, 3))
        per_entry = B > 1 and rng.random() < 0.5
        nq, nk = int(rng.integers(1, 21 if big else 7)), int(rng.integers(1, 41 if big else 9))
        q_var = _counts(rng, nq, tile, B if per_entry else 0)
        kv_var = _counts(rng, nk, tile, B if per_entry else 0)
        gate = str(rng.choice(["none", "per_token", "per_element", "projected"]))
        case = build_case(f"rand{i}_video", dtype=dtype, layout=str(rng.choice(["bhsd", "bshd"])),
                          B=B, Hq=Hq, Hkv=Hkv, D=D, q_block=tile, kv_block=tile,
                          q_var=q_var.tolist(), kv_var=kv_var.tolist(),
                          topk=int(rng.integers(1, min(nk, 12) + 2)), map_kind="none", gate_mode=gate,
                          pad_dout=bool(rng.integers(2)), seed=seed)
    elif kind == "plain":
        qb = int(rng.choice([8, 16, 32, 64, 96, 128, 256]))
        kb = int(rng.choice([64, 128, 192, 256, 320]))
        Sq, Skv = int(rng.integers(1, 3000 if big else 700)), int(rng.integers(1, 4000 if big else 1000))
        topk = int(rng.integers(1, 4)) if rng.random() < 0.3 else 0
        gate = str(rng.choice(["none", "per_token"])) if topk else "none"
        case = build_case(f"rand{i}_plain", dtype=dtype, layout=str(rng.choice(["bhsd", "bshd"])),
                          B=int(rng.integers(1, 3)), Hq=Hq, Hkv=Hkv, D=D, q_block=qb, kv_block=kb,
                          Sq=Sq, Skv=Skv, topk=topk, map_kind="none" if topk else "bernoulli",
                          map_p=float(rng.uniform(0.1, 0.9)), gate_mode=gate, seed=seed)
    else:
        n = int(rng.integers(1, 5))
        q_lens = rng.integers(1, 1200 if big else 300, n).tolist()
        kv_lens = rng.integers(1, 1600 if big else 400, n).tolist()
        case = build_case(f"rand{i}_tnd", dtype=dtype, layout="tnd", Hq=Hq, Hkv=Hkv, D=D,
                          q_block=int(rng.choice([16, 32, 64, 128])),
                          kv_block=int(rng.choice([64, 128])), q_lens=q_lens, kv_lens=kv_lens,
                          map_kind="bernoulli", map_p=float(rng.uniform(0.2, 0.9)), seed=seed)
    opts = dict(atomic_dq=bool(rng.random() < 0.3),
                persistent=[None, True, False][int(rng.integers(3))])
    return case, opts


def describe(case, opts) -> str:
    return (f"{case.name}: {case.dtype} {case.layout} B={case.B} Hq={case.Hq} Hkv={case.Hkv} "
            f"D={case.D} blocks=({case.q_block},{case.kv_block}) Qb={case.Qb} KVb={case.KVb} "
            f"topk={case.topk} gate={case.gate_mode} {opts}")
