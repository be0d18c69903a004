// Oracle: a plain, slow CPU reference for softmax attention restricted to a
// Q-block x KV-block map, with its explicit backward, the video-tile pooling,
// pooled-score top-k selection and the gated compression branch.
//
// TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's CPU
// baseline call it; the GPU library never does, and the two share no code.
//
// Every output is evaluated from its own defining formula with plain loops
// (OpenMP only splits independent outputs across threads). The accumulation
// type T is float or double; inputs are the exact (bf16/fp16-representable)
// values the GPU receives, widened to T.
//
// Sources (the pages this follows):
//  * FastVideo block_sparse_attn_cute_fwd.py: `_build_vbs_mask_mod` (a key is
//    live iff its block's valid count is positive and its offset inside the
//    block is below that count), `_build_sparse_tensors` (empty KV tiles are
//    dropped; the backward index is the map transposed), `_map_to_index`.
//  * Ascend op-plugin test_npu_block_sparse_attention_backward.py:
//    `cpu_block_sparse_attention_bnsd_with_lse` / `..._tnd_gqa_with_lse`
//    (masked row softmax, natural-log LSE), `_softmax_backward_np` and the
//    explicit backward goldens (dS = P*(dP - rowsum(dP*P)) * scale, dQ = dS K,
//    dK = dS^T Q and dV = P^T dO summed over the Q heads sharing a KV head,
//    Q head n reading KV head n / (Hq/Hkv)), `_expand_block_sparse_mask`
//    (block grid aligned to each sequence start, ceil-sized).
//  * FastVideo test_vsa256_backward.py: 256-token tiles with per-tile valid
//    counts, zero-padded tails, `topk` tiles per Q tile, the gated compression
//    branch composed with the sparse output, q_var entering only the
//    compression divisor.
//
// Readings where the pages are silent (each also listed in the design notes):
//  * a row with no live key gets O = 0 and lse = -inf and contributes nothing;
//  * pooled tile means divide by the valid count (0 -> pooled vector 0);
//  * coarse scores C = scale * <Qc_i, Kc_j>; top-k keeps the topk largest over
//    non-empty KV tiles, ties to the lower tile index;
//  * compression: softmax of C over all non-empty KV tiles, Oc = P_c Vc;
//    out = O_sel + gate (.) Oc[tile of the row] on every slot of the tile;
//  * the gradient flows through the pooled q/k/v (valid slots get grad/count)
//    but not through the top-k choice;
//  * a projected gate (mode 3) is sigmoid(<q_s, w_h> + b_h) per token and
//    head, a learnable projection of the row's own query; its gradient reaches
//    w, b and q.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <numeric>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

extern "C" {
typedef struct oracle_problem {
  int32_t layout;  // 0: [B,H,S,D]  1: [B,S,H,D]  2: packed [T,H,D] + per-sequence lengths
  int32_t B, Hq, Hkv, Sq, Skv, D;  // packed layout: Sq, Skv = total tokens
  int32_t q_block, kv_block, Qb, KVb;
  const int32_t* q_var;   // [Qb] valid tokens per Q tile, or NULL
  const int32_t* kv_var;  // [KVb] valid tokens per KV tile, or NULL
  const int32_t* q_lens;  // [B] packed layout only
  const int32_t* kv_lens;
  double scale;
  // 0 none, 1 one gate per (token, head), 2 one gate per element, 3 one gate
  // per (token, head) projected from the query row: sigmoid(<q, w_h> + b_h),
  // with the gate argument holding the parameters [w (Hq x D) | b (Hq)]
  int32_t gate_mode;
  int32_t threads;    // OpenMP threads, 0 = runtime default
  // entries between the batch entries of q_var / kv_var: 0 = one set of
  // counts for every batch entry, else entry b's counts start at b * stride
  int64_t q_var_bstride, kv_var_bstride;
} oracle_problem;
}

namespace {

struct Geo {
  const oracle_problem& p;
  std::vector<int64_t> cq, ckv;  // packed layout: start token of each sequence
  explicit Geo(const oracle_problem& pr) : p(pr) {
    if (p.layout == 2) {
      cq.assign(p.B + 1, 0);
      ckv.assign(p.B + 1, 0);
      for (int b = 0; b < p.B; ++b) {
        cq[b + 1] = cq[b] + p.q_lens[b];
        ckv[b + 1] = ckv[b] + p.kv_lens[b];
      }
    }
  }
  int group() const { return p.Hq / p.Hkv; }
  int kv_head(int h) const { return h / group(); }
  int q_len(int b) const { return p.layout == 2 ? p.q_lens[b] : p.Sq; }
  int kv_len(int b) const { return p.layout == 2 ? p.kv_lens[b] : p.Skv; }
  int nqb(int b) const { return (q_len(b) + p.q_block - 1) / p.q_block; }
  int nkb(int b) const { return (kv_len(b) + p.kv_block - 1) / p.kv_block; }
  // rows of Q block i that exist in memory
  int q_exist(int b, int i) const {
    return std::max(0, std::min(p.q_block, q_len(b) - i * p.q_block));
  }
  int kv_exist(int b, int j) const {
    return std::max(0, std::min(p.kv_block, kv_len(b) - j * p.kv_block));
  }
  // valid tokens: the tile count when given, never beyond what exists
  int q_valid(int b, int i) const {
    int e = q_exist(b, i);
    return p.q_var ? std::min(p.q_var[b * p.q_var_bstride + i], e) : e;
  }
  int kv_valid(int b, int j) const {
    int e = kv_exist(b, j);
    return p.kv_var ? std::min(p.kv_var[b * p.kv_var_bstride + j], e) : e;
  }
  // offset of element (b, h, s, 0) of a q-shaped / kv-shaped tensor
  int64_t q_off(int b, int h, int s) const {
    if (p.layout == 0) return (((int64_t)b * p.Hq + h) * p.Sq + s) * p.D;
    if (p.layout == 1) return (((int64_t)b * p.Sq + s) * p.Hq + h) * p.D;
    return ((cq[b] + s) * p.Hq + h) * p.D;
  }
  int64_t kv_off(int b, int hk, int t) const {
    if (p.layout == 0) return (((int64_t)b * p.Hkv + hk) * p.Skv + t) * p.D;
    if (p.layout == 1) return (((int64_t)b * p.Skv + t) * p.Hkv + hk) * p.D;
    return ((ckv[b] + t) * p.Hkv + hk) * p.D;
  }
  // lse: [B,Hq,Sq] for the padded layouts, [Hq, T] for the packed one
  int64_t row_id(int b, int h, int s) const {
    if (p.layout == 2) return (int64_t)h * p.Sq + cq[b] + s;
    return ((int64_t)b * p.Hq + h) * p.Sq + s;
  }
  int64_t rows_total() const { return (int64_t)p.B * p.Hq * p.Sq; }
  // one gate per (token, head): [B,H,S] next to [B,H,S,D], [B,S,H] next to [B,S,H,D]
  int64_t gate_tok(int b, int h, int s) const {
    if (p.layout == 0) return ((int64_t)b * p.Hq + h) * p.Sq + s;
    return ((int64_t)b * p.Sq + s) * p.Hq + h;
  }
  int64_t map_at(int b, int h, int i, int j) const {
    return (((int64_t)b * p.Hq + h) * p.Qb + i) * p.KVb + j;
  }
  // the block (i, j) takes part in the attention of (b, h)
  bool live_block(const uint8_t* map, int b, int h, int i, int j) const {
    if (i >= nqb(b) || j >= nkb(b)) return false;
    return map[map_at(b, h, i, j)] != 0 && kv_valid(b, j) > 0;
  }
  int64_t pq(int b, int h, int i) const { return (((int64_t)b * p.Hq + h) * p.Qb + i) * p.D; }
  int64_t pk(int b, int hk, int j) const { return (((int64_t)b * p.Hkv + hk) * p.KVb + j) * p.D; }
};

void set_threads(const oracle_problem* p) {
#ifdef _OPENMP
  if (p->threads > 0) omp_set_num_threads(p->threads);
#endif
}

template <class T>
T dot(const T* a, const T* b, int n) {
  T s = 0;
  for (int d = 0; d < n; ++d) s += a[d] * b[d];
  return s;
}

// ---------------------------------------------------------------------------
// The gate of row (b, h, s), element d: given per token (1) or per element
// (2), or projected from the row's query (3): z = <q_s, w_h> + b_h,
// gate = 1 / (1 + exp(-z)).
// ---------------------------------------------------------------------------
template <class T>
T proj_gate(const Geo& g, const T* q, const T* theta, int b, int h, int s) {
  const int D = g.p.D;
  const T z = dot(q + g.q_off(b, h, s), theta + (int64_t)h * D, D) + theta[(int64_t)g.p.Hq * D + h];
  return T(1) / (T(1) + std::exp(-z));
}

template <class T>
T gate_at(const Geo& g, const T* q, const T* gate, int b, int h, int s, int d) {
  if (g.p.gate_mode == 1) return gate[g.gate_tok(b, h, s)];
  if (g.p.gate_mode == 2) return gate[g.q_off(b, h, s) + d];
  return proj_gate(g, q, gate, b, h, s);
}

// dL/dz of a projected gate: (sum_e dO_e Oc_e) * gate * (1 - gate), with Oc
// the coarse output of the row's Q tile.
template <class T>
T proj_dlogit(const Geo& g, const T* q, const T* theta, const T* dout, const T* oc, int b, int h,
              int s) {
  const T gv = proj_gate(g, q, theta, b, h, s);
  return dot(dout + g.q_off(b, h, s), oc + g.pq(b, h, s / g.p.q_block), g.p.D) * gv * (T(1) - gv);
}

// ---------------------------------------------------------------------------
// Live keys of one query row: every valid key of every live block of its
// Q block, as offsets into k / v (block mask x per-tile valid counts).
// ---------------------------------------------------------------------------
struct KeyList {
  std::vector<int64_t> off;  // kv offsets
};

void row_keys(const Geo& g, const uint8_t* map, int b, int h, int s, KeyList& kl) {
  kl.off.clear();
  const int i = s / g.p.q_block, hk = g.kv_head(h);
  for (int j = 0; j < g.p.KVb; ++j) {
    if (!g.live_block(map, b, h, i, j)) continue;
    const int n = g.kv_valid(b, j);
    for (int u = 0; u < n; ++u) kl.off.push_back(g.kv_off(b, hk, j * g.p.kv_block + u));
  }
}

// Masked row softmax of z_t = scale <q_s, k_t> over the live keys:
// m = max z, l = sum exp(z - m), P = exp(z - m) / l, lse = m + ln l.
template <class T>
void row_softmax(const Geo& g, const T* q, const T* k, int64_t qo, const KeyList& kl,
                 std::vector<T>& P, T& lse) {
  const int D = g.p.D;
  const T sc = (T)g.p.scale;
  const size_t n = kl.off.size();
  P.resize(n);
  if (n == 0) {
    lse = -std::numeric_limits<T>::infinity();
    return;
  }
  T m = -std::numeric_limits<T>::infinity();
  for (size_t t = 0; t < n; ++t) {
    P[t] = sc * dot(q + qo, k + kl.off[t], D);
    m = std::max(m, P[t]);
  }
  T l = 0;
  for (size_t t = 0; t < n; ++t) {
    P[t] = std::exp(P[t] - m);
    l += P[t];
  }
  for (size_t t = 0; t < n; ++t) P[t] /= l;
  lse = m + std::log(l);
}

// ---------------------------------------------------------------------------
// Pooling, coarse scores, top-k and the compression branch (video tiles).
// ---------------------------------------------------------------------------
template <class T>
void pool(const Geo& g, const T* q, const T* k, const T* v, T* qc, T* kc, T* vc) {
  const auto& p = g.p;
  const int D = p.D;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < p.B; ++b)
    for (int h = 0; h < p.Hq; ++h)
      for (int i = 0; i < p.Qb; ++i) {
        T* o = qc + g.pq(b, h, i);
        const int n = g.q_valid(b, i);
        for (int d = 0; d < D; ++d) o[d] = 0;
        for (int r = 0; r < n; ++r) {
          const T* x = q + g.q_off(b, h, i * p.q_block + r);
          for (int d = 0; d < D; ++d) o[d] += x[d];
        }
        if (n > 0)
          for (int d = 0; d < D; ++d) o[d] /= (T)n;
      }
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < p.B; ++b)
    for (int hk = 0; hk < p.Hkv; ++hk)
      for (int j = 0; j < p.KVb; ++j) {
        T* ok = kc + g.pk(b, hk, j);
        T* ov = vc + g.pk(b, hk, j);
        const int n = g.kv_valid(b, j);
        for (int d = 0; d < D; ++d) ok[d] = ov[d] = 0;
        for (int r = 0; r < n; ++r) {
          const int64_t o = g.kv_off(b, hk, j * p.kv_block + r);
          for (int d = 0; d < D; ++d) {
            ok[d] += k[o + d];
            ov[d] += v[o + d];
          }
        }
        if (n > 0)
          for (int d = 0; d < D; ++d) {
            ok[d] /= (T)n;
            ov[d] /= (T)n;
          }
      }
}

// C[i, j] = scale <Qc_i, Kc_j> over non-empty KV tiles (others -inf).
template <class T>
void coarse_row(const Geo& g, const T* qc, const T* kc, int b, int h, int i, std::vector<T>& C) {
  const auto& p = g.p;
  C.assign(p.KVb, -std::numeric_limits<T>::infinity());
  const int hk = g.kv_head(h);
  for (int j = 0; j < p.KVb; ++j)
    if (g.kv_valid(b, j) > 0) C[j] = (T)p.scale * dot(qc + g.pq(b, h, i), kc + g.pk(b, hk, j), p.D);
}

template <class T>
void topk_map(const Geo& g, const T* qc, const T* kc, int topk, uint8_t* map) {
  const auto& p = g.p;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < p.B; ++b)
    for (int h = 0; h < p.Hq; ++h) {
      std::vector<T> C;
      std::vector<int> idx;
      for (int i = 0; i < p.Qb; ++i) {
        coarse_row(g, qc, kc, b, h, i, C);
        idx.clear();
        for (int j = 0; j < p.KVb; ++j)
          if (g.kv_valid(b, j) > 0) idx.push_back(j);
        // largest score first; equal scores: lower tile index first
        std::stable_sort(idx.begin(), idx.end(), [&](int a, int c) { return C[a] > C[c]; });
        const size_t keep = std::min<size_t>((size_t)std::max(topk, 0), idx.size());
        uint8_t* row = map + g.map_at(b, h, i, 0);
        for (int j = 0; j < p.KVb; ++j) row[j] = 0;
        for (size_t u = 0; u < keep; ++u) row[idx[u]] = 1;
      }
    }
}

template <class T>
void coarse_fwd(const Geo& g, const T* qc, const T* kc, const T* vc, T* oc, T* lse_c) {
  const auto& p = g.p;
  const int D = p.D;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < p.B; ++b)
    for (int h = 0; h < p.Hq; ++h) {
      std::vector<T> C;
      const int hk = g.kv_head(h);
      for (int i = 0; i < p.Qb; ++i) {
        coarse_row(g, qc, kc, b, h, i, C);
        T m = -std::numeric_limits<T>::infinity();
        for (int j = 0; j < p.KVb; ++j) m = std::max(m, C[j]);
        T* o = oc + g.pq(b, h, i);
        for (int d = 0; d < D; ++d) o[d] = 0;
        const int64_t li = ((int64_t)b * p.Hq + h) * p.Qb + i;
        if (m == -std::numeric_limits<T>::infinity()) {
          lse_c[li] = m;
          continue;
        }
        T l = 0;
        for (int j = 0; j < p.KVb; ++j)
          if (g.kv_valid(b, j) > 0) l += std::exp(C[j] - m);
        for (int j = 0; j < p.KVb; ++j) {
          if (g.kv_valid(b, j) == 0) continue;
          const T pc = std::exp(C[j] - m) / l;
          const T* vv = vc + g.pk(b, hk, j);
          for (int d = 0; d < D; ++d) o[d] += pc * vv[d];
        }
        lse_c[li] = m + std::log(l);
      }
    }
}

// ---------------------------------------------------------------------------
// Forward of the sparse branch for one row, plus the gate composition.
// ---------------------------------------------------------------------------
template <class T>
void fwd_row(const Geo& g, const T* q, const T* k, const T* v, const T* gate, const uint8_t* map,
             const T* oc, int b, int h, int s, T* out_row, T* osel_row, T* lse_out, KeyList& kl,
             std::vector<T>& P) {
  const int D = g.p.D;
  row_keys(g, map, b, h, s, kl);
  T lse;
  row_softmax(g, q, k, g.q_off(b, h, s), kl, P, lse);
  std::vector<T> o(D, (T)0);
  for (size_t t = 0; t < kl.off.size(); ++t)
    for (int d = 0; d < D; ++d) o[d] += P[t] * v[kl.off[t] + d];
  if (osel_row)
    for (int d = 0; d < D; ++d) osel_row[d] = o[d];
  if (g.p.gate_mode != 0) {
    const T* ocr = oc + g.pq(b, h, s / g.p.q_block);
    for (int d = 0; d < D; ++d) o[d] += gate_at(g, q, gate, b, h, s, d) * ocr[d];
  }
  if (out_row)
    for (int d = 0; d < D; ++d) out_row[d] = o[d];
  *lse_out = lse;
}

template <class T>
void fwd_heads(const Geo& g, const T* q, const T* k, const T* v, const T* gate, const uint8_t* map,
               const T* oc, const uint8_t* head_mask, T* out, T* osel, T* lse) {
  const auto& p = g.p;
  std::vector<int64_t> jobs;  // (b*Hq+h)*Sq_max + s, only rows that exist
  for (int b = 0; b < p.B; ++b)
    for (int h = 0; h < p.Hq; ++h) {
      if (head_mask && !head_mask[b * p.Hq + h]) continue;
      for (int s = 0; s < g.q_len(b); ++s) jobs.push_back(((int64_t)(b * p.Hq + h) << 32) | s);
    }
#pragma omp parallel
  {
    KeyList kl;
    std::vector<T> P;
#pragma omp for schedule(dynamic, 16)
    for (int64_t u = 0; u < (int64_t)jobs.size(); ++u) {
      const int bh = (int)(jobs[u] >> 32), s = (int)(jobs[u] & 0xffffffff);
      const int b = bh / p.Hq, h = bh % p.Hq;
      const int64_t qo = g.q_off(b, h, s);
      fwd_row(g, q, k, v, gate, map, oc, b, h, s, out ? out + qo : nullptr,
              osel ? osel + qo : nullptr, lse + g.row_id(b, h, s), kl, P);
    }
  }
}

// Forward of sampled rows (b, h, s) triples; out_rows is [nrows, D].
template <class T>
void fwd_rows(const Geo& g, const T* q, const T* k, const T* v, const T* gate, const uint8_t* map,
              const T* oc, int64_t nrows, const int32_t* rows, T* out_rows, T* lse_rows) {
#pragma omp parallel
  {
    KeyList kl;
    std::vector<T> P;
#pragma omp for schedule(dynamic, 4)
    for (int64_t u = 0; u < nrows; ++u)
      fwd_row(g, q, k, v, gate, map, oc, rows[3 * u], rows[3 * u + 1], rows[3 * u + 2],
              out_rows + u * g.p.D, (T*)nullptr, lse_rows + u, kl, P);
  }
}

// ---------------------------------------------------------------------------
// Backward. L = sum(out * dO). The sparse branch sees dO unchanged.
// Row pass: lse_s, Dr_s = sum_t P dP, dq_s = scale sum_t dS k_t.
// Key pass: dk_t = scale sum_{h in group} sum_s dS k-side q_s,
//           dv_t = sum_{h in group} sum_s P_{s,t} dO_s,
// with P_{s,t} = exp(z_{s,t} - lse_s), dS = P (dP - Dr_s), dP = <dO_s, v_t>.
// ---------------------------------------------------------------------------
template <class T>
struct Coarse {
  std::vector<T> qc, kc, vc, oc, lse_c, doc, dqc, dkc, dvc;
};

template <class T>
void coarse_bwd(const Geo& g, const T* q, const T* gate, const T* dout, Coarse<T>& c, T* dgate,
                const uint8_t* group_mask) {
  const auto& p = g.p;
  const int D = p.D;
  const int64_t nq = (int64_t)p.B * p.Hq * p.Qb * D, nk = (int64_t)p.B * p.Hkv * p.KVb * D;
  c.doc.assign(nq, 0);
  c.dqc.assign(nq, 0);
  c.dkc.assign(nk, 0);
  c.dvc.assign(nk, 0);
  // dOc[i] = sum over every slot s of tile i of gate_s (.) dO_s ; dgate_s = dO_s (.) Oc[i]
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < p.B; ++b)
    for (int h = 0; h < p.Hq; ++h) {
      if (group_mask && !group_mask[b * p.Hkv + g.kv_head(h)]) continue;
      for (int s = 0; s < g.q_len(b); ++s) {
        const int i = s / p.q_block;
        const int64_t qo = g.q_off(b, h, s);
        T* d = c.doc.data() + g.pq(b, h, i);
        const T* o = c.oc.data() + g.pq(b, h, i);
        T tok = 0;
        for (int e = 0; e < D; ++e) {
          const T gv = gate_at(g, q, gate, b, h, s, e);
          d[e] += gv * dout[qo + e];
          if (p.gate_mode == 2 && dgate) dgate[qo + e] = dout[qo + e] * o[e];
          tok += dout[qo + e] * o[e];
        }
        if (p.gate_mode == 1 && dgate) dgate[g.gate_tok(b, h, s)] = tok;
      }
    }
  // coarse softmax backward, row form for dQc
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < p.B; ++b)
    for (int h = 0; h < p.Hq; ++h) {
      if (group_mask && !group_mask[b * p.Hkv + g.kv_head(h)]) continue;
      std::vector<T> C;
      const int hk = g.kv_head(h);
      for (int i = 0; i < p.Qb; ++i) {
        const T lc = c.lse_c[((int64_t)b * p.Hq + h) * p.Qb + i];
        if (lc == -std::numeric_limits<T>::infinity()) continue;
        coarse_row(g, c.qc.data(), c.kc.data(), b, h, i, C);
        const T* dO = c.doc.data() + g.pq(b, h, i);
        T dr = 0;
        for (int j = 0; j < p.KVb; ++j)
          if (g.kv_valid(b, j) > 0)
            dr += std::exp(C[j] - lc) * dot(dO, c.vc.data() + g.pk(b, hk, j), D);
        T* dq = c.dqc.data() + g.pq(b, h, i);
        for (int j = 0; j < p.KVb; ++j) {
          if (g.kv_valid(b, j) == 0) continue;
          const T pc = std::exp(C[j] - lc);
          const T ds = pc * (dot(dO, c.vc.data() + g.pk(b, hk, j), D) - dr);
          const T* kk = c.kc.data() + g.pk(b, hk, j);
          for (int e = 0; e < D; ++e) dq[e] += (T)p.scale * ds * kk[e];
        }
      }
    }
  // column form for dKc, dVc (summed over the Q heads of the group)
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < p.B; ++b)
    for (int hk = 0; hk < p.Hkv; ++hk) {
      if (group_mask && !group_mask[b * p.Hkv + hk]) continue;
      std::vector<T> C;
      for (int h = hk * g.group(); h < (hk + 1) * g.group(); ++h)
        for (int i = 0; i < p.Qb; ++i) {
          const T lc = c.lse_c[((int64_t)b * p.Hq + h) * p.Qb + i];
          if (lc == -std::numeric_limits<T>::infinity()) continue;
          coarse_row(g, c.qc.data(), c.kc.data(), b, h, i, C);
          const T* dO = c.doc.data() + g.pq(b, h, i);
          T dr = 0;
          for (int j = 0; j < p.KVb; ++j)
            if (g.kv_valid(b, j) > 0)
              dr += std::exp(C[j] - lc) * dot(dO, c.vc.data() + g.pk(b, hk, j), D);
          const T* qq = c.qc.data() + g.pq(b, h, i);
          for (int j = 0; j < p.KVb; ++j) {
            if (g.kv_valid(b, j) == 0) continue;
            const T pc = std::exp(C[j] - lc);
            const T ds = pc * (dot(dO, c.vc.data() + g.pk(b, hk, j), D) - dr);
            T* dk = c.dkc.data() + g.pk(b, hk, j);
            T* dv = c.dvc.data() + g.pk(b, hk, j);
            for (int e = 0; e < D; ++e) {
              dk[e] += (T)p.scale * ds * qq[e];
              dv[e] += pc * dO[e];
            }
          }
        }
    }
}

// Gradient of the projection parameters of a projected gate (mode 3):
// dw_h = sum over rows of dL/dz q_s, db_h = sum of dL/dz; dtheta = [dw | db].
template <class T>
void proj_bwd(const Geo& g, const T* q, const T* theta, const T* dout, const T* oc, T* dtheta,
              const uint8_t* group_mask) {
  const auto& p = g.p;
  const int D = p.D;
  std::fill(dtheta, dtheta + (int64_t)p.Hq * D + p.Hq, T(0));
#pragma omp parallel for schedule(dynamic)
  for (int h = 0; h < p.Hq; ++h) {
    T* dw = dtheta + (int64_t)h * D;
    T& db = dtheta[(int64_t)p.Hq * D + h];
    for (int b = 0; b < p.B; ++b) {
      if (group_mask && !group_mask[b * p.Hkv + g.kv_head(h)]) continue;
      for (int s = 0; s < g.q_len(b); ++s) {
        const T dl = proj_dlogit(g, q, theta, dout, oc, b, h, s);
        const T* qs = q + g.q_off(b, h, s);
        for (int e = 0; e < D; ++e) dw[e] += dl * qs[e];
        db += dl;
      }
    }
  }
}

template <class T>
void bwd(const Geo& g, const T* q, const T* k, const T* v, const T* gate, const T* dout,
         const uint8_t* map, const uint8_t* group_mask, T* dq, T* dk, T* dv, T* dgate) {
  const auto& p = g.p;
  const int D = p.D;
  const T sc = (T)p.scale;
  Coarse<T> c;
  if (p.gate_mode != 0) {
    const int64_t nq = (int64_t)p.B * p.Hq * p.Qb * D, nk = (int64_t)p.B * p.Hkv * p.KVb * D;
    c.qc.assign(nq, 0);
    c.kc.assign(nk, 0);
    c.vc.assign(nk, 0);
    c.oc.assign(nq, 0);
    c.lse_c.assign((int64_t)p.B * p.Hq * p.Qb, 0);
    pool(g, q, k, v, c.qc.data(), c.kc.data(), c.vc.data());
    coarse_fwd(g, c.qc.data(), c.kc.data(), c.vc.data(), c.oc.data(), c.lse_c.data());
    coarse_bwd(g, q, gate, dout, c, p.gate_mode == 3 ? (T*)nullptr : dgate, group_mask);
    if (p.gate_mode == 3 && dgate) proj_bwd(g, q, gate, dout, c.oc.data(), dgate, group_mask);
  }
  // row pass
  std::vector<T> lse(g.rows_total(), 0), dr(g.rows_total(), 0);
  std::vector<int64_t> jobs;
  for (int b = 0; b < p.B; ++b)
    for (int h = 0; h < p.Hq; ++h) {
      if (group_mask && !group_mask[b * p.Hkv + g.kv_head(h)]) continue;
      for (int s = 0; s < g.q_len(b); ++s) jobs.push_back(((int64_t)(b * p.Hq + h) << 32) | s);
    }
#pragma omp parallel
  {
    KeyList kl;
    std::vector<T> P;
#pragma omp for schedule(dynamic, 16)
    for (int64_t u = 0; u < (int64_t)jobs.size(); ++u) {
      const int bh = (int)(jobs[u] >> 32), s = (int)(jobs[u] & 0xffffffff);
      const int b = bh / p.Hq, h = bh % p.Hq;
      const int64_t qo = g.q_off(b, h, s), rid = g.row_id(b, h, s);
      row_keys(g, map, b, h, s, kl);
      row_softmax(g, q, k, qo, kl, P, lse[rid]);
      T r = 0;
      for (size_t t = 0; t < kl.off.size(); ++t) r += P[t] * dot(dout + qo, v + kl.off[t], D);
      dr[rid] = r;
      T* o = dq + qo;
      for (int e = 0; e < D; ++e) o[e] = 0;
      for (size_t t = 0; t < kl.off.size(); ++t) {
        const T ds = P[t] * (dot(dout + qo, v + kl.off[t], D) - r);
        for (int e = 0; e < D; ++e) o[e] += sc * ds * k[kl.off[t] + e];
      }
      if (p.gate_mode != 0) {
        const int i = s / p.q_block, n = g.q_valid(b, i);
        if (s % p.q_block < n) {
          const T* a = c.dqc.data() + g.pq(b, h, i);
          for (int e = 0; e < D; ++e) o[e] += a[e] / (T)n;
        }
      }
      if (p.gate_mode == 3) {  // the projected gate's own path: dq += dL/dz w_h
        const T dl = proj_dlogit(g, q, gate, dout, c.oc.data(), b, h, s);
        for (int e = 0; e < D; ++e) o[e] += dl * gate[(int64_t)h * D + e];
      }
    }
  }
  // key pass
  std::vector<int64_t> kjobs;
  for (int b = 0; b < p.B; ++b)
    for (int hk = 0; hk < p.Hkv; ++hk) {
      if (group_mask && !group_mask[b * p.Hkv + hk]) continue;
      for (int t = 0; t < g.kv_len(b); ++t) kjobs.push_back(((int64_t)(b * p.Hkv + hk) << 32) | t);
    }
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t u = 0; u < (int64_t)kjobs.size(); ++u) {
    const int bh = (int)(kjobs[u] >> 32), t = (int)(kjobs[u] & 0xffffffff);
    const int b = bh / p.Hkv, hk = bh % p.Hkv;
    const int j = t / p.kv_block, n = g.kv_valid(b, j);
    const int64_t ko = g.kv_off(b, hk, t);
    T* dko = dk + ko;
    T* dvo = dv + ko;
    for (int e = 0; e < D; ++e) dko[e] = dvo[e] = 0;
    if (t % p.kv_block >= n) continue;  // padded slot: masked out everywhere
    for (int h = hk * g.group(); h < (hk + 1) * g.group(); ++h)
      for (int i = 0; i < g.nqb(b); ++i) {
        if (!g.live_block(map, b, h, i, j)) continue;
        for (int r = 0; r < g.q_exist(b, i); ++r) {
          const int s = i * p.q_block + r;
          const int64_t qo = g.q_off(b, h, s), rid = g.row_id(b, h, s);
          const T P = std::exp(sc * dot(q + qo, k + ko, D) - lse[rid]);
          const T ds = P * (dot(dout + qo, v + ko, D) - dr[rid]);
          for (int e = 0; e < D; ++e) {
            dko[e] += sc * ds * q[qo + e];
            dvo[e] += P * dout[qo + e];
          }
        }
      }
    if (p.gate_mode != 0) {
      const T* a = c.dkc.data() + g.pk(b, hk, j);
      const T* bb = c.dvc.data() + g.pk(b, hk, j);
      for (int e = 0; e < D; ++e) {
        dko[e] += a[e] / (T)n;
        dvo[e] += bb[e] / (T)n;
      }
    }
  }
}

// dq of sampled rows only (sparse branch plus the unpooled compression term).
template <class T>
void dq_rows(const Geo& g, const T* q, const T* k, const T* v, const T* gate, const T* dout,
             const uint8_t* map, int64_t nrows, const int32_t* rows, T* dq_out) {
  const auto& p = g.p;
  const int D = p.D;
  const T sc = (T)p.scale;
  Coarse<T> c;
  if (p.gate_mode != 0) {
    // the unpooled term needs dQc of the row's tile, which needs the coarse
    // state of that head: computed for the sampled heads only
    const int64_t nq = (int64_t)p.B * p.Hq * p.Qb * D, nk = (int64_t)p.B * p.Hkv * p.KVb * D;
    c.qc.assign(nq, 0);
    c.kc.assign(nk, 0);
    c.vc.assign(nk, 0);
    c.oc.assign(nq, 0);
    c.lse_c.assign((int64_t)p.B * p.Hq * p.Qb, 0);
    pool(g, q, k, v, c.qc.data(), c.kc.data(), c.vc.data());
    coarse_fwd(g, c.qc.data(), c.kc.data(), c.vc.data(), c.oc.data(), c.lse_c.data());
    std::vector<uint8_t> gm((size_t)p.B * p.Hkv, 0);
    for (int64_t u = 0; u < nrows; ++u) gm[rows[3 * u] * p.Hkv + g.kv_head(rows[3 * u + 1])] = 1;
    coarse_bwd(g, q, gate, dout, c, (T*)nullptr, gm.data());
  }
#pragma omp parallel
  {
    KeyList kl;
    std::vector<T> P;
#pragma omp for schedule(dynamic, 4)
    for (int64_t u = 0; u < nrows; ++u) {
      const int b = rows[3 * u], h = rows[3 * u + 1], s = rows[3 * u + 2];
      const int64_t qo = g.q_off(b, h, s);
      T lse;
      row_keys(g, map, b, h, s, kl);
      row_softmax(g, q, k, qo, kl, P, lse);
      T r = 0;
      for (size_t t = 0; t < kl.off.size(); ++t) r += P[t] * dot(dout + qo, v + kl.off[t], D);
      T* o = dq_out + u * D;
      for (int e = 0; e < D; ++e) o[e] = 0;
      for (size_t t = 0; t < kl.off.size(); ++t) {
        const T ds = P[t] * (dot(dout + qo, v + kl.off[t], D) - r);
        for (int e = 0; e < D; ++e) o[e] += sc * ds * k[kl.off[t] + e];
      }
      if (p.gate_mode != 0) {
        const int i = s / p.q_block, n = g.q_valid(b, i);
        if (s % p.q_block < n) {
          const T* a = c.dqc.data() + g.pq(b, h, i);
          for (int e = 0; e < D; ++e) o[e] += a[e] / (T)n;
        }
      }
      if (p.gate_mode == 3) {
        const T dl = proj_dlogit(g, q, gate, dout, c.oc.data(), b, h, s);
        for (int e = 0; e < D; ++e) o[e] += dl * gate[(int64_t)h * D + e];
      }
    }
  }
}

// dK / dV of sampled KV tiles (b, hk, j): the key-pass formulas above for the
// keys of those tiles only, with the row statistics (lse_s, Dr_s) of every row
// that attends them evaluated from their own rows. Outputs [n, kv_block, D].
template <class T>
void dkdv_tiles(const Geo& g, const T* q, const T* k, const T* v, const T* gate, const T* dout,
                const uint8_t* map, int64_t ntiles, const int32_t* tiles, T* dk_out, T* dv_out) {
  const auto& p = g.p;
  const int D = p.D;
  const T sc = (T)p.scale;
  Coarse<T> c;
  if (p.gate_mode != 0) {
    const int64_t nq = (int64_t)p.B * p.Hq * p.Qb * D, nk = (int64_t)p.B * p.Hkv * p.KVb * D;
    c.qc.assign(nq, 0);
    c.kc.assign(nk, 0);
    c.vc.assign(nk, 0);
    c.oc.assign(nq, 0);
    c.lse_c.assign((int64_t)p.B * p.Hq * p.Qb, 0);
    pool(g, q, k, v, c.qc.data(), c.kc.data(), c.vc.data());
    coarse_fwd(g, c.qc.data(), c.kc.data(), c.vc.data(), c.oc.data(), c.lse_c.data());
    std::vector<uint8_t> gm((size_t)p.B * p.Hkv, 0);
    for (int64_t u = 0; u < ntiles; ++u) gm[tiles[3 * u] * p.Hkv + tiles[3 * u + 1]] = 1;
    coarse_bwd(g, q, gate, dout, c, (T*)nullptr, gm.data());
  }
  // rows attending any requested tile
  std::vector<uint8_t> need(g.rows_total(), 0);
  for (int64_t u = 0; u < ntiles; ++u) {
    const int b = tiles[3 * u], hk = tiles[3 * u + 1], j = tiles[3 * u + 2];
    for (int h = hk * g.group(); h < (hk + 1) * g.group(); ++h)
      for (int i = 0; i < g.nqb(b); ++i)
        if (g.live_block(map, b, h, i, j))
          for (int r = 0; r < g.q_exist(b, i); ++r) need[g.row_id(b, h, i * p.q_block + r)] = 1;
  }
  std::vector<int64_t> jobs;
  for (int b = 0; b < p.B; ++b)
    for (int h = 0; h < p.Hq; ++h)
      for (int s = 0; s < g.q_len(b); ++s)
        if (need[g.row_id(b, h, s)]) jobs.push_back(((int64_t)(b * p.Hq + h) << 32) | s);
  std::vector<T> lse(g.rows_total(), 0), dr(g.rows_total(), 0);
#pragma omp parallel
  {
    KeyList kl;
    std::vector<T> P;
#pragma omp for schedule(dynamic, 16)
    for (int64_t u = 0; u < (int64_t)jobs.size(); ++u) {
      const int bh = (int)(jobs[u] >> 32), s = (int)(jobs[u] & 0xffffffff);
      const int b = bh / p.Hq, h = bh % p.Hq;
      const int64_t qo = g.q_off(b, h, s), rid = g.row_id(b, h, s);
      row_keys(g, map, b, h, s, kl);
      row_softmax(g, q, k, qo, kl, P, lse[rid]);
      T r = 0;
      for (size_t t = 0; t < kl.off.size(); ++t) r += P[t] * dot(dout + qo, v + kl.off[t], D);
      dr[rid] = r;
    }
  }
#pragma omp parallel for collapse(2) schedule(dynamic, 8)
  for (int64_t u = 0; u < ntiles; ++u)
    for (int tk = 0; tk < p.kv_block; ++tk) {
      const int b = tiles[3 * u], hk = tiles[3 * u + 1], j = tiles[3 * u + 2];
      T* dko = dk_out + (u * p.kv_block + tk) * D;
      T* dvo = dv_out + (u * p.kv_block + tk) * D;
      for (int e = 0; e < D; ++e) dko[e] = dvo[e] = 0;
      const int n = g.kv_valid(b, j);
      if (tk >= n) continue;
      const int64_t ko = g.kv_off(b, hk, j * p.kv_block + tk);
      for (int h = hk * g.group(); h < (hk + 1) * g.group(); ++h)
        for (int i = 0; i < g.nqb(b); ++i) {
          if (!g.live_block(map, b, h, i, j)) continue;
          for (int r = 0; r < g.q_exist(b, i); ++r) {
            const int s = i * p.q_block + r;
            const int64_t qo = g.q_off(b, h, s), rid = g.row_id(b, h, s);
            const T P = std::exp(sc * dot(q + qo, k + ko, D) - lse[rid]);
            const T ds = P * (dot(dout + qo, v + ko, D) - dr[rid]);
            for (int e = 0; e < D; ++e) {
              dko[e] += sc * ds * q[qo + e];
              dvo[e] += P * dout[qo + e];
            }
          }
        }
      if (p.gate_mode != 0) {
        const T* a = c.dkc.data() + g.pk(b, hk, j);
        const T* bb = c.dvc.data() + g.pk(b, hk, j);
        for (int e = 0; e < D; ++e) {
          dko[e] += a[e] / (T)n;
          dvo[e] += bb[e] / (T)n;
        }
      }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// C entry points (_f32: float accumulation and I/O, _f64: double)
// ---------------------------------------------------------------------------
extern "C" {

// CSR of the live blocks. kv_owned = 0: rows (b*Hq+h)*Qb+i, columns j ascending;
// kv_owned = 1: rows (b*Hq+h)*KVb+j, columns i ascending (the map transposed).
// Returns nnz, or -1 when col_capacity is too small (row_ptr still written).
int64_t oracle_block_index(const oracle_problem* p, const uint8_t* map, int32_t kv_owned,
                           int32_t* row_ptr, int32_t* col, int64_t col_capacity) {
  Geo g(*p);
  const int64_t BH = (int64_t)p->B * p->Hq;
  const int nr = kv_owned ? p->KVb : p->Qb, nc = kv_owned ? p->Qb : p->KVb;
  int64_t nnz = 0;
  row_ptr[0] = 0;
  for (int64_t bh = 0; bh < BH; ++bh) {
    const int b = (int)(bh / p->Hq), h = (int)(bh % p->Hq);
    for (int r = 0; r < nr; ++r) {
      for (int c2 = 0; c2 < nc; ++c2) {
        const int i = kv_owned ? c2 : r, j = kv_owned ? r : c2;
        if (!g.live_block(map, b, h, i, j)) continue;
        if (nnz < col_capacity) col[nnz] = c2;
        ++nnz;
      }
      row_ptr[bh * nr + r + 1] = (int32_t)nnz;
    }
  }
  return nnz <= col_capacity ? nnz : -1;
}

#define ORACLE_ENTRY_POINTS(SUF, T)                                                             \
  void oracle_pool_##SUF(const oracle_problem* p, const T* q, const T* k, const T* v, T* qc,    \
                         T* kc, T* vc) {                                                        \
    set_threads(p);                                                                             \
    Geo g(*p);                                                                                  \
    pool(g, q, k, v, qc, kc, vc);                                                               \
  }                                                                                             \
  void oracle_topk_##SUF(const oracle_problem* p, const T* qc, const T* kc, int32_t topk,       \
                         uint8_t* map) {                                                        \
    set_threads(p);                                                                             \
    Geo g(*p);                                                                                  \
    topk_map(g, qc, kc, topk, map);                                                             \
  }                                                                                             \
  void oracle_coarse_scores_##SUF(const oracle_problem* p, const T* qc, const T* kc, T* C) {    \
    Geo g(*p);                                                                                  \
    std::vector<T> row;                                                                         \
    for (int b = 0; b < p->B; ++b)                                                              \
      for (int h = 0; h < p->Hq; ++h)                                                           \
        for (int i = 0; i < p->Qb; ++i) {                                                       \
          coarse_row(g, qc, kc, b, h, i, row);                                                  \
          std::copy(row.begin(), row.end(), C + g.map_at(b, h, i, 0));                          \
        }                                                                                       \
  }                                                                                             \
  void oracle_coarse_fwd_##SUF(const oracle_problem* p, const T* qc, const T* kc, const T* vc,  \
                               T* oc, T* lse_c) {                                               \
    set_threads(p);                                                                             \
    Geo g(*p);                                                                                  \
    coarse_fwd(g, qc, kc, vc, oc, lse_c);                                                       \
  }                                                                                             \
  void oracle_fwd_##SUF(const oracle_problem* p, const T* q, const T* k, const T* v,            \
                        const T* gate, const uint8_t* map, const T* oc,                         \
                        const uint8_t* head_mask, T* out, T* osel, T* lse) {                    \
    set_threads(p);                                                                             \
    Geo g(*p);                                                                                  \
    fwd_heads(g, q, k, v, gate, map, oc, head_mask, out, osel, lse);                            \
  }                                                                                             \
  void oracle_fwd_rows_##SUF(const oracle_problem* p, const T* q, const T* k, const T* v,       \
                             const T* gate, const uint8_t* map, const T* oc, int64_t nrows,     \
                             const int32_t* rows, T* out_rows, T* lse_rows) {                   \
    set_threads(p);                                                                             \
    Geo g(*p);                                                                                  \
    fwd_rows(g, q, k, v, gate, map, oc, nrows, rows, out_rows, lse_rows);                       \
  }                                                                                             \
  void oracle_bwd_##SUF(const oracle_problem* p, const T* q, const T* k, const T* v,            \
                        const T* gate, const T* dout, const uint8_t* map,                       \
                        const uint8_t* group_mask, T* dq, T* dk, T* dv, T* dgate) {             \
    set_threads(p);                                                                             \
    Geo g(*p);                                                                                  \
    bwd(g, q, k, v, gate, dout, map, group_mask, dq, dk, dv, dgate);                            \
  }                                                                                             \
  void oracle_dq_rows_##SUF(const oracle_problem* p, const T* q, const T* k, const T* v,        \
                            const T* gate, const T* dout, const uint8_t* map, int64_t nrows,    \
                            const int32_t* rows, T* dq_rows_out) {                              \
    set_threads(p);                                                                             \
    Geo g(*p);                                                                                  \
    dq_rows(g, q, k, v, gate, dout, map, nrows, rows, dq_rows_out);                             \
  }

// The projected gate's values (mode 3) in the per-token layout of a gate.
#define ORACLE_GATE_ENTRY(SUF, T)                                                              \
  void oracle_gate_values_##SUF(const oracle_problem* p, const T* q, const T* theta, T* out) { \
    Geo g(*p);                                                                                 \
    for (int b = 0; b < p->B; ++b)                                                             \
      for (int h = 0; h < p->Hq; ++h)                                                          \
        for (int s = 0; s < g.q_len(b); ++s)                                                   \
          out[g.gate_tok(b, h, s)] = proj_gate(g, q, theta, b, h, s);                          \
  }
ORACLE_GATE_ENTRY(f32, float)
ORACLE_GATE_ENTRY(f64, double)

#define ORACLE_TILE_ENTRY(SUF, T)                                                                \
  void oracle_dkdv_tiles_##SUF(const oracle_problem* p, const T* q, const T* k, const T* v,      \
                               const T* gate, const T* dout, const uint8_t* map, int64_t ntiles, \
                               const int32_t* tiles, T* dk_out, T* dv_out) {                     \
    set_threads(p);                                                                              \
    Geo g(*p);                                                                                   \
    dkdv_tiles(g, q, k, v, gate, dout, map, ntiles, tiles, dk_out, dv_out);                      \
  }
ORACLE_TILE_ENTRY(f32, float)
ORACLE_TILE_ENTRY(f64, double)

ORACLE_ENTRY_POINTS(f32, float)
ORACLE_ENTRY_POINTS(f64, double)

}  // extern "C"
