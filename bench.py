#!/usr/bin/env python3
"""Benchmark of the block-sparse attention hot path on one MI355X.

One step = the whole path over one batch of synthetic input: vsa_fwd (pooling,
pooled-score top-k, block index in both directions, coarse attention, sparse
forward with the gated composition) followed by vsa_bwd (row term, coarse
backward, KV-owned dK/dV, Q-owned dQ). Inputs are resident in HBM before the
timed region starts.

Throughput is effective TFLOP/s over the selected blocks only, counting valid
query x valid key pairs: 4*D flops per pair for the forward (QK^T and PV) and
10*D for the backward (recomputed S, dP, dV, dQ, dK). `value` is the fwd+bwd
rate; fwd and bwd are also reported separately, with their fraction of the
MI355X dense bf16 MFMA peak.

Prints one JSON line. `--gpus N` with N > 1 is refused: the library runs on
one GPU.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "block-sparse attn fwd/bwd effective TFLOP/s (bf16) and % of MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def device_inputs(case):
    d = {n: getattr(case, n) for n in ("q", "k", "v", "dout", "gate")}
    dev = case.q.device
    d["q_valid"] = torch.as_tensor(case.q_var, dtype=torch.int32, device=dev) \
        if case.q_var is not None else None
    d["kv_valid"] = torch.as_tensor(case.kv_var, dtype=torch.int32, device=dev) \
        if case.kv_var is not None else None
    if case.layout == "tnd":
        d["cu_q"] = torch.as_tensor(np.concatenate([[0], np.cumsum(case.q_lens)]),
                                    dtype=torch.int32, device=dev)
        d["cu_kv"] = torch.as_tensor(np.concatenate([[0], np.cumsum(case.kv_lens)]),
                                     dtype=torch.int32, device=dev)
    else:
        d["cu_q"] = d["cu_kv"] = None
    d["map"] = case.block_map.to(dev).contiguous() if case.block_map is not None else None
    return d


def valid_pairs(case, bmap: torch.Tensor):
    """(valid q x valid k pairs, padded pairs) over the selected blocks."""
    dev = bmap.device
    if case.layout == "tnd":
        qv = torch.zeros(case.B, case.Qb, device=dev)
        kv = torch.zeros(case.B, case.KVb, device=dev)
        for b in range(case.B):
            for i in range(case.Qb):
                qv[b, i] = max(0, min(case.q_block, case.q_lens[b] - i * case.q_block))
            for j in range(case.KVb):
                kv[b, j] = max(0, min(case.kv_block, case.kv_lens[b] - j * case.kv_block))
    else:
        qi = torch.arange(case.Qb, device=dev)
        kj = torch.arange(case.KVb, device=dev)
        qv = (case.Sq - qi * case.q_block).clamp(0, case.q_block).float()
        kv = (case.Skv - kj * case.kv_block).clamp(0, case.kv_block).float()
        if case.q_var is not None:
            qv = torch.minimum(qv, torch.as_tensor(case.q_var, device=dev).float())
            kv = torch.minimum(kv, torch.as_tensor(case.kv_var, device=dev).float())
        qv = qv.expand(case.B, -1)
        kv = kv.expand(case.B, -1)
    m = bmap.float()
    w = qv[:, None, :, None] * kv[:, None, None, :]
    live = (kv > 0).float()[:, None, None, :]
    valid = float((m * w).sum().item())
    padded = float((m * live).sum().item()) * case.q_block * case.kv_block
    return valid, padded


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _host_threads():
    """Threads for the oracle: every core of the affinity set, but no more than
    the job's CPU share when the environment states one (OMP_NUM_THREADS)."""
    aff = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS")
    return (min(aff, int(share)) if share and share.isdigit() and int(share) > 0 else aff), aff


def _head0(case):
    """Head 0 (and the KV head it reads) of every batch entry of a workload, with
    its own geometry, block map and gate; tensors on the host."""
    import dataclasses
    if case.layout == "bshd":
        sl = (slice(None), slice(None), slice(0, 1))
    else:  # bhsd [B, H, S, D] and tnd [T, H, D]: heads on dim 1
        sl = (slice(None), slice(0, 1))
    pick = {n: getattr(case, n)[sl].contiguous().cpu() for n in ("q", "k", "v", "dout")}
    gate = case.gate
    if gate is not None:
        if case.gate_mode == "projected":  # [w (Hq x D) | b (Hq)]: head 0's row and bias
            gate = torch.cat([gate[:case.D], gate[case.Hq * case.D:case.Hq * case.D + 1]])
        else:
            gate = gate[sl]
        gate = gate.contiguous().cpu()
    bmap = case.block_map[:, 0:1].contiguous().cpu() if case.block_map is not None else None
    return dataclasses.replace(case, name=case.name + "_head0", Hq=1, Hkv=1, gate=gate,
                               block_map=bmap, **pick)


def cpu_baseline(case, gpu_valid_pairs, target_s=12.0):
    """The CPU oracle, as it stands, on a bounded sample of the same workload,
    fwd and bwd timed separately and each extrapolated linearly to the whole
    workload by its valid (q, k) pair count (labelled as such).

    Sample: head 0 of every batch entry, with the workload's own selection (its
    pooled-score top-k, or its block map). fwd: every row of a random set of
    (batch entry, Q tile) pairs (oracle fwd_rows). bwd: the full oracle backward
    (row pass with dq, key pass with dk/dv, compression backward) of the same
    head with the selection restricted to a random set of them. Rates are in
    the bench's unit: 4*D (fwd) and 10*D (bwd) flop per valid pair of the
    sample."""
    import oracle

    threads, aff = _host_threads()
    sub = _head0(case)
    orc = oracle.Oracle(sub, np.float32, threads=threads)
    t0 = time.perf_counter()
    bmap = orc.block_map()  # the head's selection (pooling + top-k when the workload has it)
    t_sel = time.perf_counter() - t0
    Bm = bmap.shape[0]
    rng = np.random.default_rng(1234)
    tiles = rng.permutation(sub.B * sub.Qb)  # (batch entry, Q tile) as b * Qb + t

    def rows_end(b):  # rows of entry b that exist
        return sub.q_lens[b] if sub.layout == "tnd" else sub.Sq

    def masked(ts):  # the selection restricted to the listed tiles
        m = np.zeros((sub.B, 1, sub.Qb, sub.KVb), np.uint8)
        for x in ts:
            b, t = divmod(int(x), sub.Qb)
            m[b, 0, t] = bmap[b if Bm > 1 else 0, 0, t]
        return m

    def pairs(ts):  # valid (q, k) pairs of the listed tiles
        return valid_pairs(sub, torch.from_numpy(masked(ts)))[0]

    def rows_of(ts):
        rows = []
        for x in ts:
            b, t = divmod(int(x), sub.Qb)
            rows += [[b, 0, s] for s in range(t * sub.q_block, min((t + 1) * sub.q_block, rows_end(b)))]
        return np.array(rows, np.int32).reshape(-1, 3)

    def bwd_of(ts):
        o = oracle.Oracle(sub, np.float32, threads=threads)
        o.set_map(masked(ts))
        t = time.perf_counter()
        o.bwd()
        return time.perf_counter() - t

    n = len(tiles)
    def timed(fn, reps):
        t = time.perf_counter()
        for _ in range(reps):
            fn()
        return (time.perf_counter() - t) / reps

    def reps_for(one, budget):
        return int(min(1000, max(1, budget / max(one, 1e-5))))

    # forward: a warm-up tile (thread start-up) and a calibration on up to four
    # tiles give the cost of one tile; the sample is the whole head (repeated)
    # when it fits 40 % of the time target, else a random set of tiles that does
    orc.fwd_rows(rows_of(tiles[:1]))
    cal = tiles[:min(n, 4)]
    one = timed(lambda: orc.fwd_rows(rows_of(cal)), 1) / len(cal)
    if n * one <= 0.4 * target_s:
        fs = tiles
        rows = rows_of(fs)
        reps_f = reps_for(n * one, 0.4 * target_s)
    else:
        fs = tiles[:int(max(1, min(n, 0.4 * target_s / one)))]
        rows = rows_of(fs)
        reps_f = 1
    t_f = timed(lambda: orc.fwd_rows(rows), reps_f)
    # backward: a call has a fixed cost (the head's pooling, coarse branch and
    # key scan) besides its per-tile one; two calibration calls separate them,
    # and the sample (whole head or a tile set) gets 60 % of the time target
    lo, hi = tiles[-min(n, 2):], tiles[-min(n, 8):]
    c_lo, c_hi = bwd_of(lo), bwd_of(hi)
    per = max((c_hi - c_lo) / max(len(hi) - len(lo), 1), 1e-5)
    fixed = max(c_lo - len(lo) * per, 0.0)
    if fixed + n * per <= 0.6 * target_s:
        bs = tiles
        reps_b = reps_for(fixed + n * per, 0.6 * target_s)
    else:
        bs = tiles[-int(max(1, min(n, (0.6 * target_s - fixed) / per))):]
        reps_b = 1
    t_b = sum(bwd_of(bs) for _ in range(reps_b)) / reps_b
    pf, pb = pairs(fs), pairs(bs)
    if pf <= 0 or pb <= 0:
        return {"value": None, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": "the sampled tiles hold no valid pair", "cpu_model": _cpu_model(),
                "affinity_cores": aff}
    fwd_rate = 4.0 * sub.D * pf / t_f / 1e12
    bwd_rate = 10.0 * sub.D * pb / t_b / 1e12
    t_f_all = t_f * gpu_valid_pairs / pf
    t_b_all = t_b * gpu_valid_pairs / pb
    sel = "its own top-k selection" if case.topk > 0 else "the workload's block map"
    return {
        "value": (4.0 + 10.0) * sub.D * gpu_valid_pairs / (t_f_all + t_b_all) / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"fp32 oracle on head 0 of {case.Hq} with {sel}: fwd of the rows of "
                   f"{len(fs)} random (batch entry, Q tile) pairs ({t_f:.2f} s), full backward "
                   + ("of the head" if len(bs) == n else f"with the selection cut to {len(bs)} of them")
                   + f" ({t_b:.2f} s)"
                   + (f", the mean of {reps_f} and {reps_b} runs" if reps_f * reps_b > 1 else "")
                   + "; rates over the sampled valid pairs; whole-workload seconds "
                   "extrapolated linearly by valid pairs"),
        "fwd_tflops": round(fwd_rate, 4), "bwd_tflops": round(bwd_rate, 4),
        "fwd_seconds_sample": round(t_f, 2), "bwd_seconds_sample": round(t_b, 2),
        "fwd_seconds_extrapolated": round(t_f_all, 1),
        "bwd_seconds_extrapolated": round(t_b_all, 1),
        "selection_seconds": round(t_sel, 2),
        "cpu_model": _cpu_model(), "affinity_cores": aff,
    }


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_{workload}.json")
CSRC = os.path.join(ROOT, "bwd_block_map_amd", "csrc")
# rocprofv3 kernel names of each stage
STAGE_KERNELS = {"sparse_fwd": "sparse_fwd_kernel", "sparse_dkdv": "sparse_dkdv_kernel",
                 "sparse_dq": "sparse_dq_kernel"}


def _code_only(text):
    """C++ source without its comments and blank lines (a comment edit does not
    change what the kernels do)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash(csrc=None):
    """sha256 over the device sources (.hip kernels and their headers, comments
    left out; the host-side C ABI is left out too): a traffic figure is only
    reported for the kernels it was measured on."""
    import hashlib
    csrc = CSRC if csrc is None else csrc
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, name)) as f:
                h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()


def _counter_rows(path, counter):
    """(kernel name, dispatch id) -> counter value (KiB) from a rocprofv3 counter CSV."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                key = (r["Kernel_Name"], r["Dispatch_Id"])
                out[key] = out.get(key, 0.0) + float(r["Counter_Value"])
    return out


COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_{workload}.txt")
PMC_COUNTERS = ("SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_SALU SQ_VALU_MFMA_BUSY_CYCLES "
                "SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VMEM GRBM_GUI_ACTIVE")


def _short_kernel(name):
    """A kernel's name without argument lists and namespaces, as the summaries print it."""
    import re
    n = name.replace("vsa::(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*$", "", n)


def summarize_counters(counter_csv, agent_csv, workload, command):
    """Per-kernel MFMA use from one rocprofv3 --pmc pass (PMC_COUNTERS) over a
    bench step: executed MFMA work (the attention kernels issue 32x32x16 bf16 or
    fp16 MFMAs, 32768 flop each, against the 2.5 PF dense peak; the coarse
    kernels 16x16x4 fp32 ones, 2048 flop, against 157.3 TF), the share of
    cycles the MFMA pipes were busy, the sustained clock,
    instruction mix per MFMA and, for the sparse stages, HBM GB/s from the
    traffic file. Durations are the counter run's own dispatch timestamps."""
    import csv
    import re
    agent = next(a for a in csv.DictReader(open(agent_csv)) if a.get("Name", "").startswith("gfx"))
    n_xcc, n_simd = int(agent["Num_Xcc"]), int(agent["Simd_Count"])
    per = {}
    with open(counter_csv) as f:
        for r in csv.DictReader(f):
            if "vsa" not in r["Kernel_Name"]:
                continue
            d = per.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"], "c": {}})
            d["c"][r["Counter_Name"]] = d["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            d["s"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    agg = {}
    for d in per.values():
        n = _short_kernel(d["name"])
        a = agg.setdefault(n, {"n": 0, "s": 0.0, "c": {}})
        a["n"] += 1
        a["s"] += d["s"]
        for c, v in d["c"].items():
            a["c"][c] = a["c"].get(c, 0.0) + v
    traffic = {}
    tpath = TRAFFIC_FILE.format(workload=workload)
    if os.path.exists(tpath):
        tr = json.load(open(tpath))
        if tr.get("source_hash") == kernel_source_hash():
            traffic = tr.get("kernels", {})
    lines = [f"# rocprofv3 counter summary, {workload} ({agent['Name']}: {agent['Cu_Count']} CUs, "
             f"{n_simd} SIMDs, {n_xcc} XCDs)",
             f"# command: {command}",
             f"# counters: {PMC_COUNTERS}",
             "# MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x SIMDs): the share of",
             "# cycles the MFMA pipes worked; clock = GRBM_GUI_ACTIVE / XCDs / duration (the",
             "# sustained engine clock during the kernel); executed TFLOP/s counts every issued",
             "# MFMA (padding included); % peak against the dense peak of the kernel's MFMA",
             "# type at 2.4 GHz: 2.5 PF for the bf16/fp16 attention kernels, 157.3 TF for the",
             "# fp32 coarse kernels.",
             "# HBM GB/s: FETCH_SIZE + WRITE_SIZE bytes per launch (traffic file, copy-calibrated)",
             "# / duration.",
             "",
             f"{'kernel':44s} {'calls':>5s} {'ms':>8s} {'GHz':>5s} {'exec TF/s':>9s} {'%peak':>6s} "
             f"{'MFMA busy':>9s} {'VALU/MFMA':>9s} {'LDS/MFMA':>8s} {'SALU/MFMA':>9s} {'HBM GB/s':>8s}"]
    for n, a in sorted(agg.items(), key=lambda kv: -kv[1]["s"]):
        c, k = a["c"], a["n"]
        sec = a["s"] / k
        mf = c.get("SQ_INSTS_MFMA", 0.0) / k
        grbm = c.get("GRBM_GUI_ACTIVE", 0.0) / k
        ghz = grbm / n_xcc / sec * 1e-9 if sec > 0 else 0.0
        fp32 = n.startswith("coarse")  # v_mfma_f32_16x16x4_f32
        peak = 157.3 if fp32 else 2500.0
        tf = mf * (2048 if fp32 else 32768) / sec * 1e-12 if sec > 0 else 0.0
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / k / (grbm / n_xcc * n_simd) if grbm else 0.0
        ratio = (lambda x: f"{c.get(x, 0.0) / k / mf:9.2f}" if mf else f"{'-':>9s}")
        gbs = f"{traffic[n]['bytes'] / sec * 1e-9:8.0f}" if n in traffic and sec > 0 else "-"
        lines.append(f"{n[:44]:44s} {k:5d} {sec * 1e3:8.2f} {ghz:5.2f} {tf:9.1f} {100 * tf / peak:6.1f} "
                     f"{100 * busy:8.1f}% {ratio('SQ_INSTS_VALU')} {ratio('SQ_INSTS_LDS')[1:]} "
                     f"{ratio('SQ_INSTS_SALU')} {gbs:>8s}")
    path = COUNTERS_FILE.format(workload=workload)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    print(f"wrote {path}")


KERNELS_FILE = os.path.join(ROOT, "profiles", "kernels_{workload}.txt")


def summarize_trace(db_path, workload, command):
    """Per-kernel calls, mean and total duration from a rocprofv3 --kernel-trace
    results database, as a short text table."""
    import sqlite3
    db = sqlite3.connect(db_path)
    rows = list(db.execute("select name, count(*), sum(duration), avg(duration) from kernels "
                           "group by name order by sum(duration) desc"))
    total = sum(r[2] for r in rows) or 1
    lines = [f"# rocprofv3 kernel-trace summary, {workload}", f"# command: {command}", "",
             f"{'kernel':62s} {'calls':>5s} {'avg_ms':>10s} {'total_ms':>10s} {'pct':>6s}"]
    for name, calls, tot, avg in rows:
        n = _short_kernel(name)
        n = "torch: " + n[len("at::"):] if n.startswith("at::") else n
        lines.append(f"{n[:62]:62s} {calls:5d} {avg / 1e6:10.3f} {tot / 1e6:10.3f} {100 * tot / total:6.2f}")
    path = KERNELS_FILE.format(workload=workload)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    print(f"wrote {path}")


def summarize_traffic(fetch_csv, write_csv, copy_bytes, workload, command):
    """Turn a FETCH_SIZE pass and a WRITE_SIZE pass (one bench run each, with a
    copy probe of copy_bytes) into HBM bytes per stage launch. Each counter is
    scaled by what it reads for the copy kernel, which moves copy_bytes in and
    copy_bytes out."""
    fetch = _counter_rows(fetch_csv, "FETCH_SIZE")
    write = _counter_rows(write_csv, "WRITE_SIZE")

    def copy_kib(rows):
        vals = [v for (n, _), v in rows.items() if "copyBuffer" in n or "copy_kernel" in n]
        return max(vals) if vals else None

    kib = copy_bytes / 1024.0
    cf, cw = copy_kib(fetch), copy_kib(write)
    if not cf or not cw:
        raise SystemExit("no copy kernel found in the counter files (run bench.py with --copy-probe)")
    ff, fw = kib / cf, kib / cw

    def per_launch(rows, pattern):
        vals = [v for (n, _), v in rows.items() if pattern in n]
        n_disp = len(vals)
        return (sum(vals) / n_disp if n_disp else 0.0), n_disp

    stages = {}
    for stage, pat in STAGE_KERNELS.items():
        # per-kernel means, summed over the distinct kernels of the stage
        names = sorted({n for (n, _) in fetch if pat in n})
        b_f = b_w = 0.0
        for n in names:
            vf = [v for (m, _), v in fetch.items() if m == n]
            vw = [v for (m, _), v in write.items() if m == n]
            b_f += (sum(vf) / len(vf)) * ff * 1024.0 if vf else 0.0
            b_w += (sum(vw) / len(vw)) * fw * 1024.0 if vw else 0.0
        stages[stage] = {"fetch_bytes": b_f, "write_bytes": b_w, "bytes": b_f + b_w,
                         "kernels": len(names)}
    # every kernel of the library, per launch (pooling, index, coarse, ... too)
    kernels = {}
    for n in sorted({n for (n, _) in fetch if "vsa" in n}):
        vf = [v for (m, _), v in fetch.items() if m == n]
        vw = [v for (m, _), v in write.items() if m == n]
        b_f = (sum(vf) / len(vf)) * ff * 1024.0
        b_w = (sum(vw) / len(vw)) * fw * 1024.0 if vw else 0.0
        kernels[_short_kernel(n)] = {"fetch_bytes": b_f, "write_bytes": b_w, "bytes": b_f + b_w,
                                     "launches": len(vf)}
    out = {"workload": workload, "command": command, "source_hash": kernel_source_hash(),
           "copy_probe_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_scale": ff, "write_scale": fw, "stages": stages, "kernels": kernels,
           "note": "HBM bytes per stage launch; "
                   "FETCH_SIZE and WRITE_SIZE are scaled by what they read for a plain "
                   "copy of copy_probe_bytes"}
    path = TRAFFIC_FILE.format(workload=workload)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out["stages"], indent=1))
    print(f"wrote {path}")


def stage_traffic(workload, stage):
    """Measured HBM bytes per launch of a stage, or None when no measurement
    exists or the kernels changed since it was taken."""
    path = TRAFFIC_FILE.format(workload=workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t["stages"].get(stage, {}).get("bytes")


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="c5_vsa256_720p_gate")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--atomic-dq", action="store_true",
                    help="time the backward that adds dQ inside the dK/dV pass with atomics")
    ap.add_argument("--grid", choices=("auto", "persistent", "per-item"), default="auto",
                    help="grid of the dK/dV pass: the library's choice, the persistent "
                         "longest-first grid, or one work-group per span")
    ap.add_argument("--gate", choices=("workload", "none", "per_token", "per_element", "projected"),
                    default="workload",
                    help="another gate form than the workload's (the 720p workload only)")
    ap.add_argument("--dout-unpadded", action="store_true",
                    help="draw dO without zeroing the padded slots of partial tiles")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="after timing, copy BYTES on the device once (counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc "
                         "passes (FETCH_SIZE, WRITE_SIZE) of a --copy-probe run, and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("COUNTER_CSV", "AGENT_CSV"),
                    help="write profiles/counters_<workload>.txt from one rocprofv3 --pmc pass "
                         "over the counters in PMC_COUNTERS, and exit")
    ap.add_argument("--summarize-trace", metavar="RESULTS_DB",
                    help="write profiles/kernels_<workload>.txt from a rocprofv3 --kernel-trace "
                         "results database, and exit")
    ap.add_argument("--trace-command", default="",
                    help="the profiling command, recorded with --summarize-trace")
    ap.add_argument("--counters-command", default="",
                    help="the profiling command, recorded with --summarize-counters")
    ap.add_argument("--traffic-command", default="",
                    help="the profiling command, recorded with --summarize-traffic")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.workload, args.trace_command)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.workload,
                           args.counters_command)
        return
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1],
                          args.copy_probe, args.workload, args.traffic_command)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the path would shard by head groups, each GPU running its heads independently)", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    import bwd_block_map_amd as vsa
    from workloads.synth import make_case

    torch.cuda.set_device(0)
    log(f"[bench] generating {args.workload} on cuda:0")
    kw = {"pad_dout": False} if args.dout_unpadded else {}
    if args.gate != "workload":
        kw["gate_mode"] = args.gate
    case = make_case(args.workload, device="cuda", **kw)
    d = device_inputs(case)
    proj = case.gate_mode == "projected"
    p = vsa.make_problem(
        dtype=case.torch_dtype, layout=case.layout, B=case.B, Hq=case.Hq, Hkv=case.Hkv,
        Sq=case.Sq, Skv=case.Skv, D=case.D, q_block=case.q_block, kv_block=case.kv_block,
        q_valid=d["q_valid"], kv_valid=d["kv_valid"], cu_seqlens_q=d["cu_q"],
        cu_seqlens_kv=d["cu_kv"], max_seqlen_q=max(case.q_lens) if case.q_lens else 0,
        max_seqlen_kv=max(case.kv_lens) if case.kv_lens else 0, scale=case.scale,
        topk=case.topk, gate_mode=case.gate_mode, atomic_dq=args.atomic_dq,
        persistent={"auto": None, "persistent": True, "per-item": False}[args.grid],
        gate_proj=d["gate"] if proj else None)
    buf = vsa.Buffers(p, d["q"], training=True)
    bmap = d["map"] if case.topk == 0 else buf.map
    dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
    # the projected gate: its parameters are in the problem, the forward
    # computes the gate values and the backward returns [dw | db]
    gate = None if proj else d["gate"]
    dg = torch.empty_like(d["gate"]) if d["gate"] is not None else None

    def fwd():
        vsa.vsa_fwd(p, d["q"], d["k"], d["v"], bmap, gate, buf.out, buf.lse, buf.saved,
                    buf.ws_fwd)

    def bwd():
        vsa.vsa_bwd(p, d["q"], d["k"], d["v"], gate, d["dout"], buf.out, buf.lse, buf.saved,
                    dq, dk, dv, dg, buf.ws_bwd)

    for w in range(args.warmup):
        fwd()
        bwd()
        torch.cuda.synchronize()
        log(f"[bench] warmup step {w + 1}/{args.warmup} done")
    valid, padded = valid_pairs(case, bmap)
    fwd_flops, bwd_flops = 4.0 * case.D * valid, 10.0 * case.D * valid

    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    vsa.vsa_profile_begin()
    t_start = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(st)
        fwd()
        ev[s][1].record(st)
        bwd()
        ev[s][2].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    prof = vsa.vsa_profile_end()
    fwd_all = [a.elapsed_time(b) for a, b, _ in ev]
    bwd_all = [b.elapsed_time(c) for _, b, c in ev]
    fwd_ms, bwd_ms = float(np.median(fwd_all)), float(np.median(bwd_all))
    step_ms = wall * 1e3 / args.steps
    log(f"[bench] timed {args.steps} steps: fwd {fwd_ms:.2f} ms, bwd {bwd_ms:.2f} ms")
    # the same steps once more, without the per-kernel and per-call events (an
    # untimed extra: on the small workloads the events add visible latency)
    t0 = time.perf_counter()
    for s in range(args.steps):
        fwd()
        bwd()
    torch.cuda.synchronize()
    plain_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # --graph: one step captured in a HIP graph (the library allocates nothing
    # and records no memset node) and replayed; an untimed extra showing what a
    # caller that captures its step sees where launch latency dominates
    graph_ms = None
    if args.graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # a warm-up step on the capture stream
            fwd()
            bwd()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fwd()
            bwd()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        log(f"[bench] graph replay: {graph_ms:.3f} ms per step")

    per_kernel = {k: {"ms_per_launch": (ms / n if n else 0.0), "launches_per_step": n / args.steps}
                  for k, (ms, n) in prof.items()}
    # algorithmic work of each stage (the metric's 4*D + 10*D per valid pair:
    # dK/dV does S, dP, dV, dK; dQ adds only its own GEMM, its recomputed S and
    # dP being overhead) and the work each stage executes
    # (with --atomic-dq the dK/dV pass also does the dQ GEMM: 10*D per pair)
    kflops = {"sparse_fwd": 4.0 * case.D * valid,
              "sparse_dkdv": (10.0 if args.atomic_dq else 8.0) * case.D * valid,
              "sparse_dq": 2.0 * case.D * valid}
    kflops_exec = dict(kflops, sparse_dq=6.0 * case.D * valid)
    dom = max(kflops, key=lambda k: prof[k][0])
    dom_ms = prof[dom][0] / max(prof[dom][1], 1)
    achieved = kflops[dom] / (dom_ms * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": stage_traffic(case.name, dom),
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                "copy-calibrated; null if not measured on these kernels)",
                "ms_per_launch": round(dom_ms, 3)}

    fwd_t = fwd_flops / (fwd_ms * 1e-3) / 1e12
    bwd_t = bwd_flops / (bwd_ms * 1e-3) / 1e12
    value = (fwd_flops + bwd_flops) / (step_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": case.dtype, "data": "synthetic (seeded N(0,1) inputs, sigmoid(N(0,1)) gate)",
        "config": {"workload": case.name, "layout": case.layout, "B": case.B, "H": case.Hq,
                   "D": case.D, "tiles": case.Qb, "tile": case.q_block, "topk": case.topk,
                   "gate": case.gate_mode, "tokens_valid": int(np.sum(case.q_var))
                   if case.q_var is not None else case.Sq,
                   "dout": "unpadded" if args.dout_unpadded else "zero in padded slots",
                   "dq": "atomic in the dK/dV pass" if args.atomic_dq else "separate Q-owned pass",
                   "dkdv_grid": {"auto": "library's choice (persistent at >= 8 spans per CU)",
                                 "persistent": "persistent, longest first",
                                 "per-item": "one work-group per span"}[args.grid]},
        "ms_per_step_without_events": round(plain_ms, 3),
        "ms_per_step_graph": None if graph_ms is None else round(graph_ms, 4),
        "fwd_ms": round(fwd_ms, 3), "bwd_ms": round(bwd_ms, 3),
        "fwd_ms_min": round(float(min(fwd_all)), 3), "bwd_ms_min": round(float(min(bwd_all)), 3),
        "fwd_tflops": round(fwd_t, 2), "bwd_tflops": round(bwd_t, 2),
        "fwd_frac_of_peak": round(fwd_t / PEAK_BF16_TFLOPS, 4),
        "bwd_frac_of_peak": round(bwd_t / PEAK_BF16_TFLOPS, 4),
        "valid_pairs": valid, "padded_pairs": padded,
        "fwd_tflops_padded": round(4.0 * case.D * padded / (fwd_ms * 1e-3) / 1e12, 2),
        "per_kernel_ms": {k: round(v["ms_per_launch"] * v["launches_per_step"], 3)
                          for k, v in per_kernel.items()},
        "stage_tflops": {k: {"algorithmic": round(kflops[k] / (prof[k][0] / max(prof[k][1], 1) * 1e-3) / 1e12, 1),
                             "executed": round(kflops_exec[k] / (prof[k][0] / max(prof[k][1], 1) * 1e-3) / 1e12, 1)}
                         for k in kflops if prof.get(k, (0, 0))[1]},
        "roofline": roofline,
    }
    if args.copy_probe > 0:  # a plain copy of known size, for counter calibration
        src = torch.empty(args.copy_probe, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(case, valid, target_s=args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
