"""The oracle's pins catch plausible mistakes (CPU only).

Each case below plants one typical slip in a copy of oracle/oracle.cpp (a
dropped scale, a flipped sign, an off-by-one mask, the wrong GQA head map, a
wrong pooling divisor, the other tie order, a missing unpool term, log base 2,
a lost sequence offset, a transposed operand, the convex gate blend, ...),
builds that copy, and runs tests/test_oracle_pins.py against it in a fresh
process (ORACLE_LIB points the loader at the copy). The pins must fail for
every mutant, and not only the finite-difference ones (those compare the
oracle with its own definition), and pass for an unmodified copy built the
same way.

The slips are planted only in the oracle, on the CPU; nothing here touches the
GPU library.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.cpp")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in oracle.cpp, replacement): every occurrence is replaced
MUTANTS = [
    ("dq_drops_scale",
     "o[e] += sc * ds * k[kl.off[t] + e];", "o[e] += ds * k[kl.off[t] + e];"),
    ("ds_sign_flipped",
     "(dot(dout + qo, v + kl.off[t], D) - r)", "(r - dot(dout + qo, v + kl.off[t], D))"),
    ("last_valid_key_dropped",
     "for (int u = 0; u < n; ++u) kl.off.push_back", "for (int u = 0; u + 1 < n; ++u) kl.off.push_back"),
    ("gqa_head_by_modulo",
     "int kv_head(int h) const { return h / group(); }", "int kv_head(int h) const { return h % p.Hkv; }"),
    ("q_pool_divides_by_block",
     "if (n > 0)\n          for (int d = 0; d < D; ++d) o[d] /= (T)n;",
     "if (n > 0)\n          for (int d = 0; d < D; ++d) o[d] /= (T)p.q_block;"),
    ("kv_pool_divides_by_block",
     "ok[d] /= (T)n;\n            ov[d] /= (T)n;", "ok[d] /= (T)p.kv_block;\n            ov[d] /= (T)p.kv_block;"),
    ("topk_ties_to_higher_tile",
     "for (int j = 0; j < p.KVb; ++j)\n          if (g.kv_valid(b, j) > 0) idx.push_back(j);",
     "for (int j = p.KVb - 1; j >= 0; --j)\n          if (g.kv_valid(b, j) > 0) idx.push_back(j);"),
    ("coarse_scores_unscaled",
     "C[j] = (T)p.scale * dot(qc + g.pq(b, h, i), kc + g.pk(b, hk, j), p.D);",
     "C[j] = dot(qc + g.pq(b, h, i), kc + g.pk(b, hk, j), p.D);"),
    ("dk_unpool_term_missing",
     "dko[e] += a[e] / (T)n;", "dko[e] += 0 * a[e];"),
    ("dq_unpool_on_padded_slots",
     "if (s % p.q_block < n) {", "if (n > 0) {"),
    ("lse_log2",
     "lse = m + std::log(l);", "lse = m + std::log2(l);"),
    ("tnd_lse_row_without_sequence_offset",
     "if (p.layout == 2) return (int64_t)h * p.Sq + cq[b] + s;",
     "if (p.layout == 2) return (int64_t)h * p.Sq + s;"),
    ("dv_uses_q_not_dout",
     "dvo[e] += P * dout[qo + e];", "dvo[e] += P * q[qo + e];"),
    ("gate_blend_convex",
     "o[d] += gate_at(g, q, gate, b, h, s, d) * ocr[d];",
     "o[d] = (1 - gate_at(g, q, gate, b, h, s, d)) * o[d] + gate_at(g, q, gate, b, h, s, d) * ocr[d];"),
    ("projected_gate_sigmoid_sign",
     "return T(1) / (T(1) + std::exp(-z));", "return T(1) / (T(1) + std::exp(z));"),
    ("projected_gate_dq_term_missing",
     "for (int e = 0; e < D; ++e) o[e] += dl * gate[(int64_t)h * D + e];",
     "for (int e = 0; e < D; ++e) o[e] += 0 * dl;"),
    ("projected_gate_dlogit_without_sigmoid_derivative",
     "* gv * (T(1) - gv);", "* gv;"),
    ("coarse_grad_ignores_gate",
     "d[e] += gv * dout[qo + e];", "d[e] += dout[qo + e];"),
    ("coarse_dv_missing_softmax_weight",
     "dv[e] += pc * dO[e];", "dv[e] += dO[e];"),
    ("per_entry_counts_ignore_the_batch_entry",
     "p.kv_var[b * p.kv_var_bstride + j]", "p.kv_var[j]"),
    ("tnd_blocks_not_clipped_to_sequence",
     "if (i >= nqb(b) || j >= nkb(b)) return false;", "if (i >= p.Qb || j >= p.KVb) return false;"),
]


def _run_pins(lib_path: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, ORACLE_LIB=lib_path, OMP_NUM_THREADS="1")
    return subprocess.run([sys.executable, "-m", "pytest", PINS, "-q", "-rf", "-p", "no:cacheprovider"],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def _build_and_run(tmp, name, old, new):
    src = open(SRC).read()
    assert old in src, f"{name}: the mutated text is no longer in oracle.cpp"
    path = os.path.join(tmp, f"{name}.cpp")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.build(src=path, out=os.path.join(tmp, f"lib_{name}.so"))
    return _run_pins(lib)


def test_every_planted_mistake_fails_a_pin(tmp_path):
    tmp = str(tmp_path)
    jobs = [("unmodified", "", "")] + MUTANTS
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        res = list(ex.map(lambda m: _build_and_run(tmp, *m), jobs))
    clean = res[0]
    assert clean.returncode == 0, "pins fail on an unmodified copy:\n" + clean.stdout[-2000:]
    survivors, self_only = [], []
    for (name, _, _), r in zip(MUTANTS, res[1:]):
        failed = [ln.split()[1].split("::")[1] for ln in r.stdout.splitlines()
                  if ln.startswith("FAILED")]
        print(f"  {name}: {len(failed)} pins fail, e.g. {failed[:3]}")
        if r.returncode == 0:
            survivors.append(name)
        # finite differences only check the oracle against its own definition:
        # each slip must also break a pin that stands outside it
        elif all(f.startswith("test_finite_differences") for f in failed):
            self_only.append(name)
    assert not survivors, f"planted mistakes no pin catches: {survivors}"
    assert not self_only, f"caught only by finite differences of the oracle itself: {self_only}"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutated_text_is_present(name, old, new):
    assert old in open(SRC).read() and old != new
