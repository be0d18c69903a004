// Backward of the sparse branch and the gate-side row reductions.
//
// Semantics: Ascend op-plugin test page, explicit backward goldens
// (`_softmax_backward_np` and the TND/GQA golden): P recomputed from the
// forward's LSE, dP = dO V^T, dS = P (dP - rowsum(dP P)) with
// rowsum(dP P) = rowsum(dO O), dQ = scale dS K, dK = scale dS^T Q,
// dV = P^T dO, dK / dV summed over the Q heads that share a KV head.
// FastVideo block_sparse_attn_cute_fwd.py: the backward is KV-owned (for every
// KV tile, the Q tiles that selected it), so dK / dV need no atomics.
//
// gfx950 design.
//  * bwd_pre: one work-group per (b, h, Q block); coalesced 16-byte loads of
//    dO and O_sel, 16-lane shuffles for the row dot products; with a gate it
//    also sums gate * dO over the tile (LDS) and forms dgate (a projected gate
//    is recomputed from the query row: dL/dz per row and per-block partial
//    sums of dw, db, summed per head by gate_proj_grad_kernel); it also writes
//    lse * log2(e) for the exp2-based recomputation of P.
//  * dK/dV: one 8-wave work-group per span of up to 256 keys of a KV block, in
//    one of three shapes picked by the span's live keys (below); on large
//    problems a persistent grid takes the spans longest first from a device
//    list. The K tile stays in LDS, V^T columns and the dK^T / dV^T
//    accumulators in registers; the heads of the group and the Q blocks of the
//    KV-owned list are walked in row chunks that arrive in LDS through a ring
//    of direct loads. No atomics: one plain store per element at the end
//    (the opt-in atomic-dQ variant adds dS K of every chunk to a float dQ
//    accumulator instead of running the dQ pass).
//  * dQ: like the forward (Q-owned list, 64-key chunks through the shared
//    K/V ring walker, S^T and dP^T with lane = query row); dQ^T += K^T dS^T
//    with K^T read transposed from the K tile; the epilogue adds the pooled
//    compression term and, for a projected gate, dL/dz * w_h.
#include "kernels.hpp"
#include "kv_walk.hpp"

namespace vsa {

namespace {

// ---------------------------------------------------------------------------
// Row term Dr = rowsum(dO * O_sel); gate: dO_c and dgate. PROJ: the gate is
// projected from q (its dL/dz per row and the partial sums of dw, db).
// ---------------------------------------------------------------------------
template <class ET, bool PROJ>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const PreArgs a) {
  using E = Elem<ET>;
  __shared__ float red[16][HD];
  const Geom& g = a.g;
  int id = blockIdx.x;
  const int i = id % g.Qb;
  id /= g.Qb;
  const int h = id % g.Hq, b = id / g.Hq;
  const int qlen = g.q_len(b), blk0 = i * g.q_block;
  if (blk0 >= qlen) return;
  const int qexist = min(g.q_block, qlen - blk0);
  const int tid = threadIdx.x, slot = tid >> 4, dg = tid & 15;
  const long long qrs = g.q_rs(), qb = g.q_base(b, h);
  const bool gated = a.gate_mode != VSA_GATE_NONE;
  // live extent: 1 + the last row whose dO has a non-zero element (a row with
  // dO = 0 has dP = 0 and Dr = 0, so dS = 0 whatever its query)
  __shared__ int live_end;
  if (tid == 0) live_end = 0;
  __syncthreads();
  int lend = 0;
  float gacc[8], wacc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) gacc[u] = wacc[u] = 0.f;
  float bacc = 0.f;
  constexpr bool proj = PROJ;
  float wv[8];  // projected gate: this lane's 8 elements of w_h
  if constexpr (proj) {
#pragma unroll
    for (int u = 0; u < 8; ++u) wv[u] = a.gproj[h * HD + 8 * dg + u];
  }
  float ocv[8];
  if (gated) {
    const float* ocp = a.oc + g.pq(b, h, i) + 8 * dg;
#pragma unroll
    for (int u = 0; u < 8; ++u) ocv[u] = ocp[u];
  }
  // the next pass's dO and O_sel rows are loaded before this pass's stores
  uint4 dv_n = make_uint4(0, 0, 0, 0), ov_n = make_uint4(0, 0, 0, 0);
  if (slot < qexist) {
    const long long off = qb + (long long)(blk0 + slot) * qrs + 8 * dg;
    dv_n = ldg16(a.dout + off);
    ov_n = ldg16(a.osel + off);
  }
  for (int s = slot; s < qexist; s += 16) {
    const long long off = qb + (long long)(blk0 + s) * qrs + 8 * dg;
    const uint4 dv = dv_n, ov = ov_n;
    if (s + 16 < qexist) {
      dv_n = ldg16(a.dout + off + 16 * qrs);
      ov_n = ldg16(a.osel + off + 16 * qrs);
    }
    const uint4 qv = proj ? ldg16(a.q + off) : make_uint4(0, 0, 0, 0);  // for the gate only
    // the row is live when one of its 16 lanes sees a non-zero element of dO
    // (either sign of zero counts as zero); the wave holds rows 4w .. 4w+3
    const uint32_t nz = (dv.x | dv.y | dv.z | dv.w) & 0x7fff7fffu;
    if ((__ballot(nz != 0) >> (16 * (slot & 3))) & 0xffffull) lend = s + 1;
    const uint32_t* dw = reinterpret_cast<const uint32_t*>(&dv);
    const uint32_t* ow = reinterpret_cast<const uint32_t*>(&ov);
    float dof[8], of[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      dof[2 * w] = E::lo(dw[w]);
      dof[2 * w + 1] = E::hi(dw[w]);
      of[2 * w] = E::lo(ow[w]);
      of[2 * w + 1] = E::hi(ow[w]);
    }
    float part = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) part += dof[u] * of[u];
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) part += __shfl_xor(part, m, 16);
    if (dg == 0) {
      const long long lr = g.lse_base(b, h) + blk0 + s;
      a.dr[lr] = part;
      const float l = a.lse[lr];
      a.lse2[lr] = l == -INFINITY ? INFINITY : l * LOG2E;  // exp2 domain; empty rows give P = 0
    }
    if (gated) {
      if (proj || a.gate_mode == VSA_GATE_PER_TOKEN) {
        float gt;
        float qf[8];
        if constexpr (proj) {  // the gate again from the query row: sigmoid(<q, w_h> + b_h)
          const uint32_t* qw = reinterpret_cast<const uint32_t*>(&qv);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            qf[2 * w] = E::lo(qw[w]);
            qf[2 * w + 1] = E::hi(qw[w]);
          }
          float z = 0.f;
#pragma unroll
          for (int u = 0; u < 8; ++u) z = __builtin_fmaf(qf[u], wv[u], z);
#pragma unroll
          for (int m = 8; m >= 1; m >>= 1) z += __shfl_xor(z, m, 16);
          z += a.gproj[g.Hq * HD + h];
          gt = 1.f / (1.f + __builtin_amdgcn_exp2f(-z * LOG2E));
        } else {
          gt = E::lo(a.gate[g.gtok_base(b, h) + (long long)(blk0 + s) * g.gtok_rs()]);
        }
        float dgp = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          gacc[u] += gt * dof[u];
          dgp += dof[u] * ocv[u];
        }
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) dgp += __shfl_xor(dgp, m, 16);
        if constexpr (proj) {  // dL/dz = dL/dgate * gate (1 - gate); its sums for dw and db
          const float dl = dgp * gt * (1.f - gt);
#pragma unroll
          for (int u = 0; u < 8; ++u) wacc[u] = __builtin_fmaf(dl, qf[u], wacc[u]);
          if (dg == 0) {
            a.dlogit[g.lse_base(b, h) + blk0 + s] = dl;
            bacc += dl;
          }
        } else if (a.dgate && dg == 0) {
          a.dgate[g.gtok_base(b, h) + (long long)(blk0 + s) * g.gtok_rs()] =
              (uint16_t)(E::pack(dgp, 0.f) & 0xffffu);
        }
      } else {
        const uint4 gv = ldg16(a.gate + off);
        const uint32_t* gw = reinterpret_cast<const uint32_t*>(&gv);
        uint32_t dgw[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          gacc[2 * w] += E::lo(gw[w]) * dof[2 * w];
          gacc[2 * w + 1] += E::hi(gw[w]) * dof[2 * w + 1];
          dgw[w] = E::pack(dof[2 * w] * ocv[2 * w], dof[2 * w + 1] * ocv[2 * w + 1]);
        }
        if (a.dgate) stg16(a.dgate + off, make_uint4(dgw[0], dgw[1], dgw[2], dgw[3]));
      }
    }
  }
  if (dg == 0 && lend) atomicMax(&live_end, lend);
  __syncthreads();
  if (tid == 0) a.qlive[((long long)b * g.Hq + h) * g.Qb + i] = live_end;
  if (!gated) return;
#pragma unroll
  for (int u = 0; u < 8; ++u) red[slot][8 * dg + u] = gacc[u];
  __syncthreads();
  if (tid < HD) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += red[r][tid];
    a.doc[g.pq(b, h, i) + tid] = s;
  }
  if constexpr (!proj) return;
  __syncthreads();  // red is reused for the dw partial sums
#pragma unroll
  for (int u = 0; u < 8; ++u) red[slot][8 * dg + u] = wacc[u];
  __shared__ float bred[16];
  if (dg == 0) bred[slot] = bacc;
  __syncthreads();
  if (tid < HD) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += red[r][tid];
    a.dwp[g.pq(b, h, i) + tid] = s;
  }
  if (tid == 0) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += bred[r];
    a.dbp[((long long)b * g.Hq + h) * g.Qb + i] = s;
  }
}

// [dw | db] of the projected gate: sums of bwd_pre's per-Q-block partials over
// batch entries and Q blocks; one work-group per head, one thread per element.
__global__ __launch_bounds__(HD) void gate_proj_grad_kernel(const Geom g, const float* dwp,
                                                            const float* dbp, float* dtheta) {
  const int h = blockIdx.x, d = threadIdx.x;
  float sw = 0.f, sb = 0.f;
  for (int b = 0; b < g.B; ++b)
    for (int i = 0; i < g.Qb; ++i) {
      const long long r = ((long long)b * g.Hq + h) * g.Qb + i;
      sw += dwp[r * HD + d];
      if (d == 0) sb += dbp[r];
    }
  dtheta[h * HD + d] = sw;
  if (d == 0) dtheta[g.Hq * HD + h] = sb;
}

// ---------------------------------------------------------------------------
// dK / dV (KV-owned)
// ---------------------------------------------------------------------------
// One work-group of 8 waves owns a span of up to 256 keys of a KV block and
// walks every (head of the group, selecting Q block, row chunk). Each wave
// keeps dK^T and dV^T of 32 keys in registers. A span picks the narrowest of
// three shapes that covers its live keys, so no wave sits on absent keys:
//   KS = 8 key slots x 1 row group  (256 keys, 32-row chunks)
//   KS = 4 key slots x 2 row groups (128 keys, 64-row chunks)
//   KS = 2 key slots x 4 row groups ( 64 keys, 128-row chunks)
// Each row group takes 32 rows of a chunk; the row groups' sums are added
// through LDS at the end. One launch covers all three shapes: each work-group
// runs the shape of its own span.
//
// Q / dO chunks (with the chunk rows' lse2 and D terms) go global -> LDS with
// counted direct loads into a ring of NST slots, so NST - 1 chunks are in
// flight while one is computed; the KV-owned list of the current head sits in
// LDS a page at a time.
constexpr int DKDV_NW = 8;
constexpr int DKDV_LIST_CAP = 1024;

// AQ: the variant that also adds each chunk's dQ = dS K into a float
// accumulator with atomics (fewer ring slots: its dS tile takes LDS).
template <int KS, bool AQ = false>
struct DkdvShape {
  static constexpr int NW = DKDV_NW;
  static constexpr int RG = NW / KS;                 // row groups
  static constexpr int KW = 32 * KS;                 // keys of the work-group
  static constexpr int QC = 32 * RG;                 // query rows per chunk
  static constexpr int QT = QC * HD * 2;             // bytes of a QC-row tile
  static constexpr int STAGE = 2 * QT + 2 * QC * 4;  // Q | dO | lse2 | dr
  // ring slots (LDS budget)
  static constexpr int NST = AQ ? (KS == 8 ? 3 : 2) : (KS == 8 ? 4 : KS == 4 ? 3 : 2);
  // direct loads per chunk and wave: Q and dO rows; the first wave of each row
  // group also loads the group's lse2 and dr
  static constexpr int LPC_ROWS = 2 * (QC / 4 / NW);
  static constexpr int LPC = LPC_ROWS + 2;
  static_assert(NW % KS == 0 && (QC / 4) % NW == 0, "whole row groups, equal load shares");
  static_assert((RG - 1) * KS * 64 * 64 * 4 <= NST * STAGE, "row-group reduction fits in the ring");
  static_assert(STAGE % 256 == 0, "slots keep the 256-byte row alignment");
};

// wait until at most `later` chunks of L direct loads each are outstanding
template <int NST, int L>
__device__ __forceinline__ void wait_later(int later) {
  if (NST >= 4 && later >= 2) wait_vm<(NST >= 4 ? 2 : 0) * L>();
  else if (NST >= 3 && later >= 1) wait_vm<(NST >= 3 ? 1 : 0) * L>();
  else wait_vm<0>();
}

__device__ __forceinline__ int dkdv_shape(int live) { return live > 128 ? 8 : live > 64 ? 4 : 2; }

// LDS of one shape, carved from the kernel's buffer: the Q/dO ring, the K
// tile, the V^T columns d >= 16 DKDV_VREG ([ks - VREG][key][lane half]; the
// registers do not hold all eight) and the list page
constexpr int DKDV_VREG = 6;
// dS tile of the atomic-dQ variant: per row group, [key][32 rows] bf16 rows of
// 64 B padded to 72 B (an odd number of 8-byte bank pairs, so the 64 lanes'
// 8-byte writes of one step and the transposed reads spread over the banks)
constexpr int DS_ROW = 72;
constexpr int DS_BYTES = 256 * DS_ROW;  // RG * KW = 256 (key, row group) rows
template <int KS, bool AQ = false>
struct DkdvLds {
  using S = DkdvShape<KS, AQ>;
  static constexpr int KT = (S::NST * S::STAGE + 1023) / 1024 * 1024;
  static constexpr int VX = KT + S::KW * HD * 2;
  static constexpr int LST = VX + (8 - DKDV_VREG) * S::KW * 2 * 16;
  static constexpr int DSB = LST + 2 * DKDV_LIST_CAP * 4;  // Q blocks | their live extents
  static constexpr int CROW = DSB + (AQ ? DS_BYTES : 0);    // row-0 offset of each slot's chunk
  static constexpr int BYTES = CROW + (AQ ? 8 * S::NST : 0);
};
constexpr int imax(int x, int y) { return x > y ? x : y; }
constexpr int DKDV_LDS = imax(DkdvLds<8>::BYTES, imax(DkdvLds<4>::BYTES, DkdvLds<2>::BYTES));
// the atomic-dQ variant runs spans of up to 128 live keys in the 128-key shape
constexpr int DKDV_LDS_AQ = imax(DkdvLds<8, true>::BYTES, DkdvLds<4, true>::BYTES);
static_assert(DKDV_LDS <= 160 * 1024 && DKDV_LDS_AQ <= 160 * 1024, "dK/dV LDS budget");

// Transposed A operand of dQ = dS K read from the dS tile ([key][row], 72-byte
// rows): M index = row (lane % 32), contraction over keys kb .. kb+15 in the
// k-slot order of TrOffs (so it pairs with TrOffs reads of the K tile).
struct DsTr {
  uint32_t o[2];
  __device__ __forceinline__ explicit DsTr(int lane) {
    const TrLane t(lane);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) o[hi] = (t.row_off + 8 * hi) * DS_ROW + t.c_off * 16 + t.half;
  }
  __device__ __forceinline__ uint4 at(const uint8_t* tile, int kb) const {
    const uint2 lo = tr8(tile, (uint32_t)(kb * DS_ROW) + o[0]);
    const uint2 hi = tr8(tile, (uint32_t)(kb * DS_ROW) + o[1]);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
};

// dK / dV of keys k0 .. kend-1 of KV block j (live keys: the first `live`);
// AQ: also dQ += dS K of every chunk, added to a.dqacc with atomics
template <class ET, int KS, bool AQ>
__device__ __forceinline__ void dkdv_span(const BwdArgs& a, uint8_t* smem, int tid, int b, int hk,
                                          int j, int k0, int kend, int nval, int live) {
  using E = Elem<ET>;
  using S = DkdvShape<KS, AQ>;
  using L = DkdvLds<KS, AQ>;
  constexpr int NW = S::NW, RG = S::RG, QC = S::QC, QT = S::QT, STAGE = S::STAGE, KW = S::KW;
  constexpr int NST = S::NST, LPC = S::LPC, LPC_ROWS = S::LPC_ROWS, VREG = DKDV_VREG;
  uint8_t* const ring = smem;  // slot s at ring + s * STAGE
  uint8_t* const Kt = smem + L::KT;
  uint4* const Vx = reinterpret_cast<uint4*>(smem + L::VX);
  int* const lst_i = reinterpret_cast<int*>(smem + L::LST);
  int* const lst_e = lst_i + DKDV_LIST_CAP;
  uint8_t* const dsb = smem + L::DSB;                          // AQ: the chunk's dS
  long long* const crow = reinterpret_cast<long long*>(smem + L::CROW);  // AQ

  const Geom& g = a.g;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave-level values stay scalar
  const int hl = lane >> 5;
  const int kslot = wave % KS, rg = wave / KS;
  const long long krs = g.kv_rs();
  const long long kbase = g.kv_base(b, hk) + (long long)j * g.kv_block * krs;
  const int mykey = k0 + 32 * kslot + (lane & 31);  // key inside the KV block
  const bool key_live = mykey < k0 + live;

  f32x16_t dka[4], dva[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dka[mb][r] = dva[mb][r] = 0.f;

  if (live > 0) {
    // the work-group's K rows stay in LDS for the whole walk (rows past the
    // live keys repeat the last live one and are masked); V^T columns are
    // register B operands (lane: key, d = 16ks + 8hl + 0..7)
    stage_rows<KW, NW>(Kt, wave, lane, a.k + kbase + (long long)k0 * krs, (uint32_t)(krs * 2),
                       min(live, KW) - 1);
    uint4 vr[VREG];
    const long long koff = kbase + (long long)mykey * krs;
    const int vx = (32 * kslot + (lane & 31)) * 2 + hl;  // this lane's slot in Vx
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks >= VREG && rg != 0) continue;  // row group 0 stores the shared columns
      const uint4 v = key_live ? ldg16(a.v + koff + 16 * ks + 8 * hl) : make_uint4(0, 0, 0, 0);
      if (ks < VREG) vr[ks] = v;
      else Vx[(ks - VREG) * KW * 2 + vx] = v;
    }
    const bool wave_keys = 32 * kslot < live;        // this wave has a live key
    const float c2 = g.scale * LOG2E;
    const long long qrs = g.q_rs();
    const uint32_t qrs_bytes = (uint32_t)(qrs * 2);
    const RowOffs ro(lane);
    const TrOffs to(lane);
    const int rb = 32 * rg;  // this wave's rows inside a chunk

    // ---- the list walker: heads of the group, their KV-owned entries, row chunks ----
    // A chunk's loads need only two running offsets (of its row 0 in q / dout
    // and in lse2 / dr), so a fill is a few scalar adds and the direct loads.
    int hh = 0, e0 = 0, cnt = 0, page = 0;  // current head's CSR row and list page
    // a list page: the Q blocks and their live extents
    auto load_list = [&](int hx, int base) {
      const long long qb0 = ((long long)b * g.Hq + hk * g.group + hx) * g.Qb;
      for (int t = tid; t < DKDV_LIST_CAP && base + t < cnt; t += NW * 64) {
        const int si = a.col[e0 + base + t];
        lst_i[t] = si;
        lst_e[t] = a.qlive[qb0 + si];
      }
    };
    auto load_head = [&](int hx) {  // first list page of head hx (all waves; drains loads)
      const long long r = ((long long)b * g.Hq + hk * g.group + hx) * g.KVb + j;
      // uniform, and kept scalar: everything the fills derive from them stays scalar
      e0 = __builtin_amdgcn_readfirstlane(a.row_ptr[r]);
      cnt = __builtin_amdgcn_readfirstlane(a.row_ptr[r + 1]) - e0;
      page = 0;
      __syncthreads();
      load_list(hx, 0);
      __syncthreads();
    };
    // stager: list entry se, rows of its Q block from the next chunk on, and
    // the element offsets of the next chunk's row 0 in q / dout and in lse2 / dr
    int se = 0, left = 0;
    long long cq = 0, cl = 0;
    bool more = true;
    // Rows past a block's live extent have dO = 0 (the padded slots of partial
    // video tiles, where callers pass a zero gradient): their dP and Dr are 0,
    // so dS = 0 and they add exactly nothing to dK and dV; the walk stops there
    // and passes over blocks without a live row.
    auto settle = [&]() {  // from entry se of head hh, find the next entry with live rows
      for (;;) {
        while (se >= cnt) {
          if (++hh >= g.group) {
            more = false;
            return;
          }
          load_head(hh);
          se = 0;
        }
        if (se - page >= DKDV_LIST_CAP) {  // next page (only for lists longer than the cap)
          __syncthreads();
          page = se;
          load_list(hh, page);
          __syncthreads();
        }
        left = min(__builtin_amdgcn_readfirstlane(lst_e[se - page]),
                   g.q_block);  // live rows, never more than exist
        if (left > 0) break;
        ++se;
      }
      const int si = __builtin_amdgcn_readfirstlane(lst_i[se - page]);
      const int h = hk * g.group + hh;
      const long long r0 = (long long)si * g.q_block;
      cq = uniform_i64(g.q_base(b, h) + r0 * qrs);
      cl = uniform_i64(g.lse_base(b, h) + r0);
    };
    load_head(0);
    settle();

    // per slot, 8 bits of `slots`: valid rows of its chunk (1 .. QC), 0 if empty
    uint32_t slots = 0;
    const long long qstep = (long long)QC * qrs;
    auto fill = [&](int s) {
      slots &= ~(0xFFu << (8 * s));
      if (!more) return;
      const int last = min(left, QC) - 1;  // rows past it repeat it
      slots |= (uint32_t)(last + 1) << (8 * s);
      uint8_t* st = ring + s * STAGE;
      if (AQ && tid == 0) crow[s] = cq;
      stage_rows<QC, NW>(st, wave, lane, a.q + cq, qrs_bytes, last);
      stage_rows<QC, NW>(st + QT, wave, lane, a.dout + cq, qrs_bytes, last);
      // the row group's 32 rows of lse2 and dr, loaded by its first wave; rows
      // past the chunk's last repeat it, so no load leaves the block (the lane
      // offset is rebuilt here: kept live over the walk it was spilled, and a
      // reload in the fill waits for every load in flight)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const uint32_t loff = 4u * (uint32_t)min(rb + ln, last);
      const uint32_t lds_l = lds_addr(st + 2 * QT) + 4 * rb;
      if (kslot == 0 && lane < 32) {
        dma4(a.lse2 + cl, loff, lds_l);
        dma4(a.dr + cl, loff, lds_l + 4 * QC);
      }
      left -= QC;
      if (left > 0) {
        cq += qstep;
        cl += QC;
      } else {
        ++se;
        settle();
      }
    };
    auto rem_of = [&](int s) { return (int)((slots >> (8 * s)) & 0xFFu); };

    // one chunk: S = Q K^T and dP = dO V^T, then P and dS, then
    // dV^T += dO^T P and dK^T += Q^T dS
    auto compute = [&](const uint8_t* Qs, int rows_valid) {
      const uint8_t* Ds = Qs + QT;
      const float* lse2 = reinterpret_cast<const float*>(Qs + 2 * QT);
      const float* drs = lse2 + QC;
      // rows rb + 8(r/4) + 4hl + r%4, key column
      f32x16_t sv, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] = dp[r] = 0.f;
      __builtin_amdgcn_iglp_opt(0);  // MFMA / LDS-read interleaving, as in the forward (dK/dV 1 %)
      uint4 nq = ro.at(Qs, rb, 0), nk = ro.at(Kt, 32 * kslot, 0), nd = ro.at(Ds, rb, 0);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const uint4 cq = nq, ck = nk, cd = nd;
        if (ks < 7) {  // the next step's operands are read before this step's MFMAs
          nq = ro.at(Qs, rb, ks + 1);
          nk = ro.at(Kt, 32 * kslot, ks + 1);
          nd = ro.at(Ds, rb, ks + 1);
        }
        // keeps the scheduler from sinking those reads back next to their use
        __builtin_amdgcn_sched_barrier(0);
        sv = E::mfma(cq, ck, sv);
        dp = E::mfma(cd, ks < VREG ? vr[ks] : Vx[(ks - VREG) * KW * 2 + vx], dp);
      }
      const bool partial = rows_valid < rb + 32;  // rows past the Q block get P = 0
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 l4 = *reinterpret_cast<const float4*>(lse2 + rb + 8 * q4 + 4 * hl);
        const float4 d4 = *reinterpret_cast<const float4*>(drs + rb + 8 * q4 + 4 * hl);
        float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
        if (partial) {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (rb + 8 * q4 + 4 * hl + u >= rows_valid) lv[u] = INFINITY;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * q4 + u;
          // a key past the live ones only feeds its own dK / dV column, which
          // the epilogue writes as zero, so it needs no mask here
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], c2, -lv[u]));
          sv[r] = p;
          dp[r] = p * (dp[r] - dv[u]);
        }
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int o = 8 * kt;
        const uint4 pp = make_uint4(E::pack(sv[o], sv[o + 1]), E::pack(sv[o + 2], sv[o + 3]),
                                    E::pack(sv[o + 4], sv[o + 5]), E::pack(sv[o + 6], sv[o + 7]));
        uint4 ps = make_uint4(E::pack(dp[o], dp[o + 1]), E::pack(dp[o + 2], dp[o + 3]),
                              E::pack(dp[o + 4], dp[o + 5]), E::pack(dp[o + 6], dp[o + 7]));
        if constexpr (AQ) {
          // dQ contracts over keys, so a key past the live ones must add
          // nothing there (its own dK column is dropped anyway); the tile
          // stores this wave's 32 keys x 32 rows transposed ([key][row])
          if (!key_live) ps = make_uint4(0, 0, 0, 0);
          uint8_t* dsw = dsb + (rg * KW + 32 * kslot + (lane & 31)) * DS_ROW + 32 * kt + 8 * hl;
          *reinterpret_cast<uint2*>(dsw) = make_uint2(ps.x, ps.y);
          *reinterpret_cast<uint2*>(dsw + 16) = make_uint2(ps.z, ps.w);
        }
        uint4 nv = to.at(Ds, rb + 16 * kt, 0), nk = to.at(Qs, rb + 16 * kt, 0);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const uint4 cv = nv, ck = nk;
          if (mb < 3) {  // the next step's operands are read before this step's MFMAs
            nv = to.at(Ds, rb + 16 * kt, mb + 1);
            nk = to.at(Qs, rb + 16 * kt, mb + 1);
          }
          dva[mb] = E::mfma(cv, pp, dva[mb]);
          dka[mb] = E::mfma(ck, ps, dka[mb]);
        }
      }
    };
    // does this wave have work in a chunk with `rows` valid rows
    auto busy = [&](int rows) { return wave_keys && rows > rb; };

    // AQ, after every wave wrote its dS: this wave's 32-row x 32-d block of the
    // chunk's dQ = dS K (row block qb, d block db, keys k_lo .. of the span's
    // live keys), added to the float accumulator. 256-key spans: two waves per
    // block, one per half of the keys; 128-key spans: one wave per block.
    const int qrb = KS == 8 ? 0 : (wave >> 2), qdb = wave & 3;
    const int k_lo = KS == 8 ? 128 * (wave >> 2) : 0;
    const int k_hi = min(k_lo + (KS == 8 ? 128 : KW), live);
    const uint32_t qrs4 = (uint32_t)(qrs * 4);
    auto dq_part = [&](int rows_valid, long long r0) {
      if (rows_valid <= 32 * qrb || k_lo >= k_hi) return;
      // The lane offsets below are rebuilt here from an opaque copy of the lane
      // id rather than kept live over the walk: the walk's registers are full,
      // and a spilled value reloaded in the fill would wait for every load in
      // flight.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const DsTr dtr(ln);
      // transposed reads of the K tile for this wave's d block (TrOffs at
      // mb = qdb, computed for that block alone: a runtime index into TrOffs
      // would put its table in scratch memory)
      uint32_t kto[2];
      {
        const TrLane t(ln);
#pragma unroll
        for (int hi = 0; hi < 2; ++hi)
          kto[hi] = toff((int)t.row_off + 8 * hi, 4 * qdb + t.c_off) + t.half;
      }
      auto kt_at = [&](int kb) {
        const uint2 lo = tr8(Kt, (uint32_t)(kb * 256) + kto[0]);
        const uint2 hi = tr8(Kt, (uint32_t)(kb * 256) + kto[1]);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
      };
      const uint8_t* dt = dsb + qrb * KW * DS_ROW;
      f32x16_t qa;
#pragma unroll
      for (int r = 0; r < 16; ++r) qa[r] = 0.f;
      // one key step of 16 at a time, the next step's operands read ahead
      uint4 na = dtr.at(dt, k_lo), nb = kt_at(k_lo);
#pragma nounroll
      for (int kb = k_lo; kb < k_hi; kb += 16) {
        const uint4 ca = na, cb = nb;
        if (kb + 16 < k_hi) {
          na = dtr.at(dt, kb + 16);
          nb = kt_at(kb + 16);
        }
        qa = E::mfma(ca, cb, qa);
      }
      // lane: d = 32 qdb + lane % 32; register r: row 32 qrb + 8(r/4) + 4hl + r%4.
      // The address is a uniform base (the chunk's row 0 plus the register's
      // row step) and the lane's 32-bit offset, so no per-row address stays live.
      const int vrow = 32 * qrb + 4 * (ln >> 5);  // the lane's first row
      // byte offset of (row vrow, d = 32 qdb + lane % 32) from the chunk's row 0
      const uint32_t aq_lane = (uint32_t)vrow * qrs4 + 4u * (uint32_t)(32 * qdb + (ln & 31));
      const char* base = reinterpret_cast<const char*>(uniform_ptr(a.dqacc + r0));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int step = 8 * (r >> 2) + (r & 3);
        if (vrow + step < rows_valid) {
          const char* rb_ptr = base + (uint32_t)step * qrs4;
          unsafeAtomicAdd((float*)(rb_ptr + aq_lane), qa[r]);
        }
      }
    };
    // the chunk of slot s1 must have landed; the chunks loaded after it may
    // stay in flight
    auto wait_chunk = [&](int s1) {  // s1: slot of chunk n + 1
      int later = 0;
#pragma unroll
      for (int k = 1; k < NST - 1; ++k) later += rem_of((s1 + k) % NST) != 0;
      if (kslot == 0) wait_later<NST, LPC>(later);
      else wait_later<NST, LPC_ROWS>(later);
    };
    auto next = [&](int s) { return s == NST - 1 ? 0 : s + 1; };

    if (more) {
#pragma unroll
      for (int s = 0; s < NST - 1; ++s) fill(s);
      wait_vm<0>();  // the K tile, V columns and the first slot's rows
      lds_barrier();
      for (int s = 0;;) {
        fill(s == 0 ? NST - 1 : s - 1);  // the slot freed by the previous step
        const int rows = rem_of(s);
        if (busy(rows)) compute(ring + s * STAGE, rows);
        if constexpr (AQ) {
          lds_barrier();  // the chunk's dS tile is complete
          dq_part(rows, crow[s]);
        }
        s = next(s);
        wait_chunk(s);
        lds_barrier();
        if (rem_of(s) == 0) break;
      }
    }

    if (RG > 1) {
      // row groups 1.. hand their sums to row group 0 through the (now idle)
      // ring, one accumulator set at a time: [RG-1][KS][64 values][64 lanes]
      float* red = reinterpret_cast<float*>(ring);
      auto reduce = [&](f32x16_t(&acc)[4]) {
        __syncthreads();
        if (rg > 0) {
          float* w = red + ((rg - 1) * KS + kslot) * 4096 + lane;
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) w[(mb * 16 + r) * 64] = acc[mb][r];
        }
        __syncthreads();
        if (rg == 0) {
#pragma unroll
          for (int g2 = 1; g2 < RG; ++g2) {
            const float* w = red + ((g2 - 1) * KS + kslot) * 4096 + lane;
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[mb][r] += w[(mb * 16 + r) * 64];
          }
        }
      };
      reduce(dka);
      reduce(dva);
    }
  }

  // keys of the span past the work-group's KW (absent or padded): zero gradients
  for (int kk = k0 + KW + (tid >> 4); kk < kend; kk += NW * 4) {
    const long long o = kbase + (long long)kk * krs + 8 * (tid & 15);
    stg16(a.dk + o, make_uint4(0, 0, 0, 0));
    stg16(a.dv + o, make_uint4(0, 0, 0, 0));
  }

  // ---- epilogue: dk = scale * dK + dK_c / valid, dv = dV + dV_c / valid ----
  if (rg != 0 || mykey >= kend) return;
  const long long koff = kbase + (long long)mykey * krs;
  const float* dkc = a.dkc ? a.dkc + g.pk(b, hk, j) : nullptr;
  const float* dvc = a.dvc ? a.dvc + g.pk(b, hk, j) : nullptr;
  const float invn = (key_live && dkc) ? 1.f / (float)nval : 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * mb + 8 * q4 + 4 * hl;
      float kx[4], vx[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        kx[u] = key_live ? g.scale * dka[mb][4 * q4 + u] : 0.f;
        vx[u] = key_live ? dva[mb][4 * q4 + u] : 0.f;
      }
      if (dkc && key_live) {
        const float4 ck = *reinterpret_cast<const float4*>(dkc + d0);
        const float4 cv = *reinterpret_cast<const float4*>(dvc + d0);
        kx[0] += ck.x * invn;
        kx[1] += ck.y * invn;
        kx[2] += ck.z * invn;
        kx[3] += ck.w * invn;
        vx[0] += cv.x * invn;
        vx[1] += cv.y * invn;
        vx[2] += cv.z * invn;
        vx[3] += cv.w * invn;
      }
      *reinterpret_cast<uint2*>(a.dk + koff + d0) =
          make_uint2(E::pack(kx[0], kx[1]), E::pack(kx[2], kx[3]));
      *reinterpret_cast<uint2*>(a.dv + koff + d0) =
          make_uint2(E::pack(vx[0], vx[1]), E::pack(vx[2], vx[3]));
    }
}

// One work item: the span `id` (span-minor order of (b, KV head, KV block,
// span)), in the shape its live keys pick.
template <class ET, bool AQ>
__device__ __forceinline__ void dkdv_item(const BwdArgs& a, uint8_t* smem, int tid, int id) {
  const Geom& g = a.g;
  const int nspan = (g.kv_block + a.span - 1) / a.span;
  const int span = id % nspan;
  id /= nspan;
  const int j = id % g.KVb;
  id /= g.KVb;
  const int hk = id % g.Hkv, b = id / g.Hkv;
  const int k0 = span * a.span;
  const int kend = min(g.kv_exist(b, j), min(g.kv_block, k0 + a.span));  // existing keys < kend
  if (k0 >= kend) return;
  const int nval = g.kv_val(b, j);
  const int live = max(0, min(kend, nval) - k0);  // live keys of the span
  const int shape = dkdv_shape(live);
  if (shape == 8) dkdv_span<ET, 8, AQ>(a, smem, tid, b, hk, j, k0, kend, nval, live);
  else if (AQ || shape == 4) dkdv_span<ET, 4, AQ>(a, smem, tid, b, hk, j, k0, kend, nval, live);
  else dkdv_span<ET, 2, false>(a, smem, tid, b, hk, j, k0, kend, nval, live);
}

// One launch for all three shapes: each work-group picks its span's shape, so
// the memory-bound 64-key spans of partial tiles run next to the MFMA-bound
// 256-key spans instead of after them.
//   PERSIST = false: one work-group per span, in the XCD-aware order.
//   PERSIST = true: a fixed grid (one work-group per CU); each work-group takes
//   the next item of a.lpt_order (longest first within each KV head) from an
//   atomic counter until the list is used up, so long spans start first and
//   short ones fill the tail. Every wave of a work-group reads the same item
//   and they leave the loop together.
template <class ET, bool AQ, bool PERSIST>
__global__ __launch_bounds__(DKDV_NW * 64, 2) void sparse_dkdv_kernel(const BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[AQ ? DKDV_LDS_AQ : DKDV_LDS];
  if constexpr (!PERSIST) {
    const int nspan = (a.g.kv_block + a.span - 1) / a.span;
    dkdv_item<ET, AQ>(a, smem, threadIdx.x, xcd_group(blockIdx.x, gridDim.x, nspan));
  } else {
    __shared__ int next_item;
    for (;;) {
      __syncthreads();  // the previous item is done with the LDS
      if (threadIdx.x == 0) next_item = atomicAdd(a.lpt_counter, 1);
      __syncthreads();
      const int it = next_item;
      if (it >= a.n_items) break;
      // an opaque copy of the thread id per item: values derived from the lane
      // must not be hoisted out of the item loop (the three shapes' copies
      // would then be live together and spill inside the chunk loop)
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      dkdv_item<ET, AQ>(a, smem, tid, a.lpt_order[it]);
    }
  }
}

// ---------------------------------------------------------------------------
// Longest-processing-time order of the dK/dV spans (persistent backward):
// a span's work is estimated as (Q blocks that selected its KV block, over the
// heads of the group) x (chunk steps per Q block of its shape: 8, 4 or 2), cut
// into LPT_LEVELS levels; spans are ordered by KV head (b, hk) first, so the
// grid still sweeps the heads in turn, then by decreasing work. A counting
// sort: histogram, exclusive scan, scatter.
// ---------------------------------------------------------------------------
constexpr int LPT_LEVELS = 1024;

template <int LEVELS = LPT_LEVELS>
__device__ __forceinline__ int lpt_bin(const BwdArgs& a, int id) {
  const Geom& g = a.g;
  const int nspan = (g.kv_block + a.span - 1) / a.span;
  const int span = id % nspan;
  int r = id / nspan;
  const int j = r % g.KVb;
  r /= g.KVb;
  const int hk = r % g.Hkv, b = r / g.Hkv;
  const int k0 = span * a.span;
  const int kend = min(g.kv_exist(b, j), min(g.kv_block, k0 + a.span));
  const int live = max(0, min(kend, g.kv_val(b, j)) - k0);
  long long cnt = 0;
  for (int hh = 0; hh < g.group; ++hh) {
    const long long row = ((long long)b * g.Hq + hk * g.group + hh) * g.KVb + j;
    cnt += a.row_ptr[row + 1] - a.row_ptr[row];
  }
  const int steps = dkdv_shape(live);  // 8, 4 or 2 chunk steps per Q block
  const long long work = live > 0 ? cnt * steps : 0;
  const long long wmax = (long long)g.group * g.Qb * 8;
  const int level = (int)min<long long>(LEVELS - 1, work * (LEVELS - 1) / max(wmax, 1LL));
  return (b * g.Hkv + hk) * LEVELS + (LEVELS - 1 - level);
}

// hist[bin + 1] counts the spans of each bin (hist zeroed before)
__global__ __launch_bounds__(256) void lpt_count_kernel(const BwdArgs a, int32_t* hist) {
  const int id = blockIdx.x * 256 + threadIdx.x;
  if (id < a.n_items) atomicAdd(&hist[lpt_bin(a, id) + 1], 1);
}

// after the scan hist[bin] is the first position of the bin
__global__ __launch_bounds__(256) void lpt_scatter_kernel(const BwdArgs a, int32_t* hist,
                                                           int32_t* order) {
  const int id = blockIdx.x * 256 + threadIdx.x;
  if (id < a.n_items) order[atomicAdd(&hist[lpt_bin(a, id)], 1)] = id;
}

// The same order for small problems in one launch: one work-group histograms
// the bins in LDS (LPT_SMALL_LEVELS levels per KV head), scans them, scatters
// the spans and clears the item counter.
constexpr int LPT_SMALL_LEVELS = 256;
constexpr int LPT_SMALL_BINS = 16384;

__global__ __launch_bounds__(1024) void lpt_small_kernel(const BwdArgs a, int32_t* order,
                                                         int32_t* counter) {
  __shared__ int32_t hist[LPT_SMALL_BINS];
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const int nb = a.g.B * a.g.Hkv * LPT_SMALL_LEVELS, n = a.n_items;
  for (int x = t; x < nb; x += 1024) hist[x] = 0;
  __syncthreads();
  for (int id = t; id < n; id += 1024) atomicAdd(&hist[lpt_bin<LPT_SMALL_LEVELS>(a, id)], 1);
  __syncthreads();
  const int per = (nb + 1023) / 1024, beg = min(t * per, nb), end = min(beg + per, nb);
  int32_t s = 0;
  for (int x = beg; x < end; ++x) s += hist[x];
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int32_t acc = part[t] - s;
  for (int x = beg; x < end; ++x) {
    const int32_t c = hist[x];
    hist[x] = acc;
    acc += c;
  }
  __syncthreads();
  for (int id = t; id < n; id += 1024) order[atomicAdd(&hist[lpt_bin<LPT_SMALL_LEVELS>(a, id)], 1)] = id;
  if (t == 0) *counter = 0;
}

// dq = scale * (the atomically accumulated dS K) + the unpooled compression
// term on valid slots; one work-group per (b, h, Q block), 16 lanes per row.
template <class ET>
__global__ __launch_bounds__(256) void dq_cast_kernel(const BwdArgs a) {
  using E = Elem<ET>;
  const Geom& g = a.g;
  int id = blockIdx.x;
  const int i = id % g.Qb;
  id /= g.Qb;
  const int h = id % g.Hq, b = id / g.Hq;
  const int qlen = g.q_len(b), blk0 = i * g.q_block;
  if (blk0 >= qlen) return;
  const int qexist = min(g.q_block, qlen - blk0);
  const int tid = threadIdx.x, slot = tid >> 4, dg = tid & 15;
  const long long qrs = g.q_rs(), qb = g.q_base(b, h);
  const int nq = a.dqc ? g.q_val(b, i) : 0;
  float cterm[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) cterm[u] = 0.f;
  if (nq > 0) {
    const float* c = a.dqc + g.pq(b, h, i) + 8 * dg;
#pragma unroll
    for (int u = 0; u < 8; ++u) cterm[u] = c[u] / (float)nq;
  }
  float wv[8];  // projected gate: this lane's 8 elements of w_h
#pragma unroll
  for (int u = 0; u < 8; ++u) wv[u] = a.gproj ? a.gproj[h * HD + 8 * dg + u] : 0.f;
  for (int s = slot; s < qexist; s += 16) {
    const long long off = qb + (long long)(blk0 + s) * qrs + 8 * dg;
    const float4 x0 = *reinterpret_cast<const float4*>(a.dqacc + off);
    const float4 x1 = *reinterpret_cast<const float4*>(a.dqacc + off + 4);
    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const bool valid = s < nq;
    const float dl = a.gproj ? a.dlogit[g.lse_base(b, h) + blk0 + s] : 0.f;
    float y[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) y[u] = __builtin_fmaf(dl, wv[u], g.scale * x[u] + (valid ? cterm[u] : 0.f));
    uint32_t w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = E::pack(y[2 * u], y[2 * u + 1]);
    stg16(a.dq + off, make_uint4(w[0], w[1], w[2], w[3]));
  }
}

// ---------------------------------------------------------------------------
// dQ (Q-owned)
// ---------------------------------------------------------------------------
constexpr int KC = KV_CHUNK;

template <class ET, int NW, int NST>
__global__ __launch_bounds__(NW * 64, 2) void sparse_dq_kernel(const BwdArgs a) {
  using E = Elem<ET>;
  const Geom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave-level values stay scalar
  const int hl = lane >> 5, l32 = lane & 31;
  const int nsub = max(1, g.q_block / (32 * NW));  // Q blocks of 8 or 16 rows: one wave
  int id = xcd_group(blockIdx.x, gridDim.x, nsub * XCD_QBLOCKS);
  const int sub = id % nsub;
  id /= nsub;
  const int i = id % g.Qb;
  id /= g.Qb;
  const int h = id % g.Hq, b = id / g.Hq;
  const int qlen = g.q_len(b), blk0 = i * g.q_block;
  if (blk0 >= qlen) return;
  const int qexist = min(g.q_block, qlen - blk0);
  const int myrow = sub * 32 * NW + wave * 32 + l32;
  const bool row_ok = myrow < qexist;
  const long long qrs = g.q_rs();
  const long long qoff = g.q_base(b, h) + (long long)(blk0 + myrow) * qrs;

  // this wave's Q and dO rows: B operands (lane: row l32, d = 16ks + 8hl + 0..7)
  uint4 qr[8], dor[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qr[ks] = row_ok ? ldg16(a.q + qoff + 16 * ks + 8 * hl) : make_uint4(0, 0, 0, 0);
    dor[ks] = row_ok ? ldg16(a.dout + qoff + 16 * ks + 8 * hl) : make_uint4(0, 0, 0, 0);
  }
  const long long lrow = g.lse_base(b, h) + blk0 + myrow;
  const float lse2 = row_ok ? a.lse2[lrow] : INFINITY;
  const float drv = row_ok ? a.dr[lrow] : 0.f;
  const float c2 = g.scale * LOG2E;
  const RowOffs ro(lane);
  const TrOffs to(lane);

  f32x16_t acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;

  const long long rid = ((long long)b * g.Hq + h) * g.Qb + i;
  const int e0 = __builtin_amdgcn_readfirstlane(a.row_ptr[rid]);  // uniform: the walk stays scalar
  const int cnt = __builtin_amdgcn_readfirstlane(a.row_ptr[rid + 1]) - e0;

  // Rows past the block's live extent have dO = 0 (the padded slots of
  // partial video tiles, where callers pass a zero gradient), so dS = 0: a
  // wave made only of them skips the walk's arithmetic (its dq rows are the
  // compression term or zero), and a work-group made only of them skips the walk.
  const int qlive = a.qlive[rid];
  const bool dead = sub * 32 * NW + wave * 32 >= qlive;
  const int walk_cnt = sub * 32 * NW >= qlive ? 0 : cnt;

  walk_kv<NW, NST>(g, b, h / g.group, a.col, e0, walk_cnt, a.k, a.v, wave, lane,
                   [&](const uint8_t* Ks, const uint8_t* Vs, int rem) {
    if (dead) return;
    __builtin_amdgcn_iglp_opt(0);  // MFMA / LDS-read interleaving, as in the forward
    // per half of 32 keys: S^T = K Q^T, dP^T = V dO^T, dS = P * (dP - D), then
    // dQ^T += K^T dS^T over its two key steps of 16
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      // a chunk of at most 32 keys: its second half is all padding, whose
      // dS = 0 adds exactly nothing
      if (hf == 1 && rem <= 32) break;
      f32x16_t sv, pv;
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] = pv[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        sv = E::mfma(ro.at(Ks, 32 * hf, ks), qr[ks], sv);
        pv = E::mfma(ro.at(Vs, 32 * hf, ks), dor[ks], pv);
      }
      // lane holds keys 32hf + 8(r/4) + 4hl + (r%4) of its row; keys past the
      // valid ones get P = 0 through a -inf exponent
      if (rem < KC) {
        const int lim = rem - 32 * hf - 4 * hl;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) >= lim) sv[r] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], c2, -lse2)) * (pv[r] - drv);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int o = 8 * kt;
        const uint4 pb = make_uint4(E::pack(sv[o], sv[o + 1]), E::pack(sv[o + 2], sv[o + 3]),
                                    E::pack(sv[o + 4], sv[o + 5]), E::pack(sv[o + 6], sv[o + 7]));
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[mb] = E::mfma(to.at(Ks, 32 * hf + 16 * kt, mb), pb, acc[mb]);
      }
    }
  });

  if (!row_ok) return;
  const float* dqc = nullptr;
  float invn = 0.f;
  if (a.dqc) {
    const int nq = g.q_val(b, i);
    if (myrow < nq) {
      dqc = a.dqc + g.pq(b, h, i);
      invn = 1.f / (float)nq;
    }
  }
  // projected gate: every row adds dL/dz w_h
  const float dl = a.gproj ? a.dlogit[lrow] : 0.f;
  const float* wh = a.gproj ? a.gproj + h * HD : nullptr;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * mb + 8 * q4 + 4 * hl;
      float x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = g.scale * acc[mb][4 * q4 + u];
      if (dqc) {
        const float4 cq = *reinterpret_cast<const float4*>(dqc + d0);
        x[0] += cq.x * invn;
        x[1] += cq.y * invn;
        x[2] += cq.z * invn;
        x[3] += cq.w * invn;
      }
      if (wh) {
        const float4 w4 = *reinterpret_cast<const float4*>(wh + d0);
        x[0] = __builtin_fmaf(dl, w4.x, x[0]);
        x[1] = __builtin_fmaf(dl, w4.y, x[1]);
        x[2] = __builtin_fmaf(dl, w4.z, x[2]);
        x[3] = __builtin_fmaf(dl, w4.w, x[3]);
      }
      *reinterpret_cast<uint2*>(a.dq + qoff + d0) =
          make_uint2(E::pack(x[0], x[1]), E::pack(x[2], x[3]));
    }
}

template <class ET>
hipError_t launch_pre_t(const PreArgs& a, hipStream_t st) {
  const long long n = (long long)a.g.B * a.g.Hq * a.g.Qb;
  if (n == 0) return hipSuccess;
  if (a.gate_mode == VSA_GATE_PROJECTED) bwd_pre_kernel<ET, true><<<(unsigned)n, 256, 0, st>>>(a);
  else bwd_pre_kernel<ET, false><<<(unsigned)n, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <class ET>
hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const long long n = dkdv_items(g, a.span);
  if (n == 0) return hipSuccess;
  if (a.lpt_order) {
    const unsigned grid = (unsigned)(n < a.persist_grid ? n : a.persist_grid);
    if (a.dqacc) sparse_dkdv_kernel<ET, true, true><<<grid, DKDV_NW * 64, 0, st>>>(a);
    else sparse_dkdv_kernel<ET, false, true><<<grid, DKDV_NW * 64, 0, st>>>(a);
  } else if (a.dqacc) {
    sparse_dkdv_kernel<ET, true, false><<<(unsigned)n, DKDV_NW * 64, 0, st>>>(a);
  } else {
    sparse_dkdv_kernel<ET, false, false><<<(unsigned)n, DKDV_NW * 64, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <class ET>
hipError_t launch_dq_cast_t(const BwdArgs& a, hipStream_t st) {
  const long long n = (long long)a.g.B * a.g.Hq * a.g.Qb;
  if (n == 0) return hipSuccess;
  dq_cast_kernel<ET><<<(unsigned)n, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <class ET>
hipError_t launch_dq_t(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int nw = g.q_block % 256 == 0 ? 8 : g.q_block % 128 == 0 ? 4 : g.q_block % 64 == 0 ? 2 : 1;
  const long long nwg = (long long)g.B * g.Hq * g.Qb * max(1, g.q_block / (32 * nw));
  if (nwg == 0) return hipSuccess;
  if (nw == 8) sparse_dq_kernel<ET, 8, 4><<<(unsigned)nwg, 512, 0, st>>>(a);
  else if (nw == 4) sparse_dq_kernel<ET, 4, 2><<<(unsigned)nwg, 256, 0, st>>>(a);
  else if (nw == 2) sparse_dq_kernel<ET, 2, 2><<<(unsigned)nwg, 128, 0, st>>>(a);
  else sparse_dq_kernel<ET, 1, 2><<<(unsigned)nwg, 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_pre(const PreArgs& a, int dtype, hipStream_t st) {
  return dtype == VSA_BF16 ? launch_pre_t<bf16_tag>(a, st) : launch_pre_t<f16_tag>(a, st);
}
hipError_t launch_sparse_dkdv(const BwdArgs& a, int dtype, hipStream_t st) {
  return dtype == VSA_BF16 ? launch_dkdv_t<bf16_tag>(a, st) : launch_dkdv_t<f16_tag>(a, st);
}
hipError_t launch_sparse_dq(const BwdArgs& a, int dtype, hipStream_t st) {
  return dtype == VSA_BF16 ? launch_dq_t<bf16_tag>(a, st) : launch_dq_t<f16_tag>(a, st);
}
long long dkdv_items(const Geom& g, int span) {
  return (long long)g.B * g.Hkv * g.KVb * ((g.kv_block + span - 1) / span);
}
long long lpt_hist_entries(const Geom& g) { return (long long)g.B * g.Hkv * LPT_LEVELS + 2; }

bool lpt_order_small(const Geom& g, int span) {
  return (long long)g.B * g.Hkv * LPT_SMALL_LEVELS <= LPT_SMALL_BINS && dkdv_items(g, span) <= 16384;
}

hipError_t launch_lpt_order(const BwdArgs& a, int32_t* hist, int32_t* order, hipStream_t st) {
  const long long n = a.n_items, nb = (long long)a.g.B * a.g.Hkv * LPT_LEVELS;
  if (n == 0) return hipSuccess;
  if (lpt_order_small(a.g, a.span)) {  // hist need not be zero: only the counter is used
    lpt_small_kernel<<<1, 1024, 0, st>>>(a, order, a.lpt_counter);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)((n + 255) / 256);
  lpt_count_kernel<<<grid, 256, 0, st>>>(a, hist);
  hipError_t e = launch_exclusive_scan(hist, nb, st);
  if (e != hipSuccess) return e;
  lpt_scatter_kernel<<<grid, 256, 0, st>>>(a, hist, order);
  return hipGetLastError();
}

hipError_t launch_gate_proj_grad(const Geom& g, const float* dwp, const float* dbp, float* dtheta,
                                 hipStream_t st) {
  if (g.Hq == 0) return hipSuccess;
  gate_proj_grad_kernel<<<(unsigned)g.Hq, HD, 0, st>>>(g, dwp, dbp, dtheta);
  return hipGetLastError();
}

hipError_t launch_dq_cast(const BwdArgs& a, int dtype, hipStream_t st) {
  return dtype == VSA_BF16 ? launch_dq_cast_t<bf16_tag>(a, st) : launch_dq_cast_t<f16_tag>(a, st);
}

}  // namespace vsa
