// Launch interface of the gfx950 kernels (called by the C ABI in vsa_api.cpp).
#pragma once

#include "common.hpp"

namespace vsa {

// Sparse-branch forward (plus the gate composition in its epilogue).
struct FwdArgs {
  Geom g;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* gate;  // PER_TOKEN / PER_ELEMENT gate
  const float* oc;       // pooled coarse output [B,Hq,Qb,HD] (gate only)
  int gate_mode;
  const float* gproj;    // PROJECTED: [w (Hq x HD) | b (Hq)]
  uint16_t* gate_out;    // PROJECTED: per-token gate values, or null
  uint16_t* out;
  uint16_t* osel;  // un-gated sparse output (gate + training), else null
  float* lse;
  const int32_t* row_ptr;  // Q-owned CSR
  const int32_t* col;
};

// Backward of the sparse branch.
struct BwdArgs {
  Geom g;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse2;       // lse * log2(e), +inf for rows without a live key
  const float* dr;         // rowsum(dO * O_sel), laid out like lse
  // per Q block [B,Hq,Qb]: 1 + its last row whose dO is not zero (the rows
  // after it add nothing to dK / dV and have dS = 0)
  const int32_t* qlive;
  const int32_t* row_ptr;  // Q-owned (dQ) or KV-owned (dK/dV) CSR
  const int32_t* col;
  const float* dqc;  // gate: pooled-tile gradients added to valid slots, else null
  const float* dkc;
  const float* dvc;
  // projected gate: [w | b] and dL/dz per row (laid out like lse), else null;
  // every row's dq gets dL/dz w_h
  const float* gproj;
  const float* dlogit;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  // atomic-dQ backward: float accumulator laid out like q (zeroed before the
  // dK/dV launch, which adds dS K into it); null for the two-kernel backward
  float* dqacc;
  // persistent dK/dV: the spans in longest-first order, the item counter
  // (zeroed before the launch), the number of spans and the grid; lpt_order
  // null for one work-group per span
  const int32_t* lpt_order;
  int32_t* lpt_counter;
  int n_items;
  int persist_grid;
  // keys per dK/dV work item: DKDV_SPAN, or DKDV_SPAN_MIN when the items of
  // that size still fit on the compute units at once
  int span;
};

// Row term and gate-side reductions of the backward.
struct PreArgs {
  Geom g;
  const uint16_t* q;
  const uint16_t* dout;
  const uint16_t* osel;  // sparse-branch output
  const uint16_t* gate;
  const float* oc;
  int gate_mode;
  const float* lse;
  float* dr;
  float* lse2;
  float* doc;       // gate: [B,Hq,Qb,HD] sum over the tile of gate * dO
  uint16_t* dgate;  // PER_TOKEN / PER_ELEMENT gate: optional
  int32_t* qlive;  // [B,Hq,Qb] live extents (see BwdArgs)
  // projected gate: [w | b]; out: dL/dz per row (laid out like lse) and, per
  // Q block, the partial sums of dL/dz q ([B,Hq,Qb,HD]) and of dL/dz ([B,Hq,Qb])
  const float* gproj;
  float* dlogit;
  float* dwp;
  float* dbp;
};

// Pooled tiles, coarse scores, top-k and coarse attention.
struct CoarseArgs {
  Geom g;
  const float* qc;  // [B,Hq,Qb,HD]
  const float* kc;  // [B,Hkv,KVb,HD]
  const float* vc;
  int topk;
  uint8_t* map;   // topk > 0: [B,Hq,Qb,KVb]
  float* oc;      // gate: [B,Hq,Qb,HD]
  float* lse_c;   // gate: [B,Hq,Qb]
  // backward
  const float* doc;
  float* ps;      // workspace [B,Hq,Qb,KVb]: P_c
  float* dss;     // workspace [B,Hq,Qb,KVb]: W = P_c dP_c (dS_c = W - csum P_c)
  float* csum;    // workspace [B,Hq,Qb]: row sums of W
  float* dqc;
  float* dkc;
  float* dvc;
};

hipError_t launch_index(const Geom& g, const uint8_t* map, int kv_owned, int32_t* row_ptr,
                        int32_t* col, long long cap, hipStream_t st);
// both directions (Q-owned, then KV-owned); one launch for small maps
hipError_t launch_index_both(const Geom& g, const uint8_t* map, int32_t* q_rp, int32_t* q_col,
                             int32_t* kv_rp, int32_t* kv_col, long long cap, hipStream_t st);
hipError_t launch_pool(const Geom& g, int dtype, const void* q, const void* k, const void* v,
                       float* qc, float* kc, float* vc, hipStream_t st);
hipError_t launch_coarse_fwd(const CoarseArgs& a, bool want_topk, bool want_gate, hipStream_t st);
hipError_t launch_coarse_bwd(const CoarseArgs& a, hipStream_t st);
hipError_t launch_sparse_fwd(const FwdArgs& a, int dtype, hipStream_t st);
hipError_t launch_bwd_pre(const PreArgs& a, int dtype, hipStream_t st);
hipError_t launch_sparse_dkdv(const BwdArgs& a, int dtype, hipStream_t st);
hipError_t launch_sparse_dq(const BwdArgs& a, int dtype, hipStream_t st);
hipError_t launch_dq_cast(const BwdArgs& a, int dtype, hipStream_t st);
constexpr int DKDV_SPAN = 256;     // keys per dK/dV work item
constexpr int DKDV_SPAN_MIN = 64;  // ... on problems whose 64-key items fit on the CUs at once
long long dkdv_items(const Geom& g, int span);  // dK/dV spans of a problem
long long lpt_hist_entries(const Geom& g);  // int32 entries of the order's histogram
// longest-first order of the dK/dV spans into `order` (a.n_items entries);
// `hist` (lpt_hist_entries) must be zero unless lpt_order_small(g), whose one
// launch also clears a.lpt_counter
bool lpt_order_small(const Geom& g, int span);
hipError_t launch_lpt_order(const BwdArgs& a, int32_t* hist, int32_t* order, hipStream_t st);
hipError_t launch_exclusive_scan(int32_t* a, long long n, hipStream_t st);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);
// rows of D elements (2 or 4 bytes) <-> rows of HD elements, the extra ones zero
hipError_t launch_widen_rows(const void* src, void* dst, long long rows, int D, int elem_bytes,
                             hipStream_t st);
hipError_t launch_narrow_rows(const void* src, void* dst, long long rows, int D, int elem_bytes,
                              hipStream_t st);
hipError_t launch_copy_words(const void* src, void* dst, long long words, hipStream_t st);
// gradient of the projected gate's parameters [dw | db] from bwd_pre's partials
hipError_t launch_gate_proj_grad(const Geom& g, const float* dwp, const float* dbp, float* dtheta,
                                 hipStream_t st);

}  // namespace vsa
