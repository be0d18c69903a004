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
//    also sums gate * dO over the tile (LDS) and forms dgate.
//  * dK/dV: one work-group = NW waves x 32 keys of one KV block; K and V of
//    the wave's keys stay in registers as MFMA B operands for S = Q K^T and
//    dP = dO V^T (lane = key column, 16 query rows per lane); the Q heads of
//    the group and the Q blocks of the KV-owned list are walked in chunks of
//    32 rows, staged in LDS both row-major (for the d contractions) and
//    transposed (for the row contractions dV^T += dO^T P, dK^T += Q^T dS).
//    Accumulators stay in registers; one plain store per element at the end.
//  * dQ: like the forward (Q-owned list, 64-key chunks, S^T and dP^T with
//    lane = query row); dQ^T += K^T dS^T with K^T staged in LDS.
#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace vsa {

namespace {

// ---------------------------------------------------------------------------
// Row term Dr = rowsum(dO * O_sel); gate: dO_c and dgate.
// ---------------------------------------------------------------------------
template <class ET>
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
  float gacc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) gacc[u] = 0.f;
  float ocv[8];
  if (gated) {
    const float* ocp = a.oc + g.pq(b, h, i) + 8 * dg;
#pragma unroll
    for (int u = 0; u < 8; ++u) ocv[u] = ocp[u];
  }
  for (int s = slot; s < qexist; s += 16) {
    const long long off = qb + (long long)(blk0 + s) * qrs + 8 * dg;
    const uint4 dv = ldg16(a.dout + off);
    const uint4 ov = ldg16(a.osel + off);
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
      if (a.gate_mode == VSA_GATE_PER_TOKEN) {
        const float gt = E::lo(a.gate[g.gtok_base(b, h) + (long long)(blk0 + s) * g.gtok_rs()]);
        float dgp = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          gacc[u] += gt * dof[u];
          dgp += dof[u] * ocv[u];
        }
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) dgp += __shfl_xor(dgp, m, 16);
        if (a.dgate && dg == 0)
          a.dgate[g.gtok_base(b, h) + (long long)(blk0 + s) * g.gtok_rs()] =
              (uint16_t)(E::pack(dgp, 0.f) & 0xffffu);
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
}

// ---------------------------------------------------------------------------
// dK / dV (KV-owned)
// ---------------------------------------------------------------------------
// Which 128-key sub-tiles a launch owns: sub-tiles with more than 64 live keys
// go to the wide launch (4 waves x 32 keys), the others (the partial video
// tiles) to a narrow launch over their first 64 keys, where the 4 waves form
// 2 key slots x 2 row groups (each chunk's rows are split, and the two row
// groups' sums are added through LDS at the end), so no wave sits on absent keys.
enum DkdvPart { DKDV_ALL = 0, DKDV_WIDE = 1, DKDV_NARROW = 2 };

template <int NW, int RG, int NBUF>
struct DkdvShape {
  static constexpr int KS = NW / RG;          // key slots (32 keys each)
  static constexpr int KW = 32 * KS;          // keys of the work-group
  static constexpr int QC = 32 * RG;          // query rows per chunk
  static constexpr int QT = QC * HD * 2;      // bytes of a QC-row tile
  static constexpr int STAGE = 2 * QT + 2 * QC * 4;  // Q | dO | lse2 | dr
  static constexpr int LDS = NBUF * STAGE + KW * HD * 2;  // stages, then the K tile
};

template <class ET, int NW, int RG, int NBUF>
__global__ __launch_bounds__(NW * 64, 2) void sparse_dkdv_kernel(const BwdArgs a, int part) {
  using E = Elem<ET>;
  using S = DkdvShape<NW, RG, NBUF>;
  constexpr int QC = S::QC, QT = S::QT, STAGE = S::STAGE, KW = S::KW;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S::LDS];

  const Geom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5;
  const int kslot = wave % S::KS, rg = wave / S::KS;
  const int unit = part == DKDV_ALL ? KW : 128;  // keys per grid sub-tile
  const int nsub = g.kv_block / unit;
  int id = xcd_group(blockIdx.x, gridDim.x, nsub);
  const int sub = id % nsub;
  id /= nsub;
  const int j = id % g.KVb;
  id /= g.KVb;
  const int hk = id % g.Hkv, b = id / g.Hkv;

  const int kexist = g.kv_exist(b, j);
  const int k0 = sub * unit;
  if (k0 >= kexist) return;  // no key of this sub-tile exists
  const int nval = g.kv_val(b, j);
  const int live = max(0, min(unit, nval - k0));  // live keys of the sub-tile
  if (part == DKDV_WIDE && live > 0 && live <= 64) return;
  if (part == DKDV_NARROW && !(live > 0 && live <= 64)) return;
  const long long krs = g.kv_rs();
  const long long kbase = g.kv_base(b, hk) + (long long)j * g.kv_block * krs;
  const int mykey = k0 + 32 * kslot + (lane & 31);  // key inside the KV block
  const bool key_live = mykey < nval;

  f32x16_t dka[4], dva[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dka[mb][r] = dva[mb][r] = 0.f;

  if (live > 0) {
    // the work-group's K rows stay in LDS for the whole walk (rows past the
    // valid keys repeat the last valid one and are masked); V^T columns are
    // register B operands (lane: key, d = 16ks + 8hl + 0..7)
    uint8_t* Kt = smem + NBUF * STAGE;
    const int lastk = min(live, KW) - 1;
    stage_tile<KW, NW>(Kt, wave, lane, [&](int row) {
      return a.k + kbase + (long long)(k0 + min(row, lastk)) * krs;
    });
    uint4 vr[8];
    const long long koff = kbase + (long long)mykey * krs;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      vr[ks] = key_live ? ldg16(a.v + koff + 16 * ks + 8 * hl) : make_uint4(0, 0, 0, 0);
    const float kmask = key_live ? 0.f : -INFINITY;  // added to the exp2 argument
    const float c2 = g.scale * LOG2E;
    const long long qrs = g.q_rs();
    const RowOffs ro(lane);
    const TrOffs to(lane);
    const int rb = 32 * rg;  // this wave's rows inside a chunk

    // one chunk = (head h, Q block i, rows QC*c ..); rows past the block repeat
    // its last row (in bounds) and are masked in the compute
    auto stage = [&](int buf, int h, int i, int c) {
      const int last = g.q_exist(b, i) - c * QC - 1;
      const long long base = g.q_base(b, h) + (long long)(i * g.q_block + c * QC) * qrs;
      uint8_t* st = smem + buf * STAGE;
      stage_tile<QC, NW>(st, wave, lane, [&](int row) { return a.q + base + min(row, last) * qrs; });
      stage_tile<QC, NW>(st + QT, wave, lane,
                         [&](int row) { return a.dout + base + min(row, last) * qrs; });
      const long long lb = g.lse_base(b, h) + i * g.q_block + c * QC;
      if (wave == 0) stage_f32<QC>((float*)(st + 2 * QT), a.lse2 + lb, lane, last);
      if (wave == NW - 1) stage_f32<QC>((float*)(st + 2 * QT) + QC, a.dr + lb, lane, last);
    };

    auto compute = [&](int buf, int rows_valid) {
      const uint8_t* Qs = smem + buf * STAGE;
      const uint8_t* Ds = Qs + QT;
      const float* lse2 = reinterpret_cast<const float*>(Qs + 2 * QT);
      const float* drs = lse2 + QC;
      // S = Q K^T and dP = dO V^T (rows rb + 8(r/4) + 4hl + r%4, key column)
      f32x16_t s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        s = E::mfma(ro.at(Qs, rb, ks), ro.at(Kt, 32 * kslot, ks), s);
        dp = E::mfma(ro.at(Ds, rb, ks), vr[ks], dp);
      }
      const bool partial = rows_valid < rb + 32;  // rows past the Q block get P = 0
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 l4 = *reinterpret_cast<const float4*>(lse2 + rb + 8 * q4 + 4 * hl);
        const float4 d4 = *reinterpret_cast<const float4*>(drs + rb + 8 * q4 + 4 * hl);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
        if (partial) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = 4 * q4 + u;
            const float l = rb + 8 * q4 + 4 * hl + u >= rows_valid ? INFINITY : lv[u];
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c2, -l) + kmask);
            s[r] = p;
            dp[r] = p * (dp[r] - dv[u]);
          }
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = 4 * q4 + u;
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c2, -lv[u]) + kmask);
            s[r] = p;
            dp[r] = p * (dp[r] - dv[u]);
          }
        }
      }
      // dV^T += dO^T P, dK^T += Q^T dS (row steps of 16)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int o = 8 * kt;
        const uint4 pp = make_uint4(E::pack(s[o], s[o + 1]), E::pack(s[o + 2], s[o + 3]),
                                    E::pack(s[o + 4], s[o + 5]), E::pack(s[o + 6], s[o + 7]));
        const uint4 ps = make_uint4(E::pack(dp[o], dp[o + 1]), E::pack(dp[o + 2], dp[o + 3]),
                                    E::pack(dp[o + 4], dp[o + 5]), E::pack(dp[o + 6], dp[o + 7]));
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          dva[mb] = E::mfma(to.at(Ds, rb + 16 * kt, mb), pp, dva[mb]);
          dka[mb] = E::mfma(to.at(Qs, rb + 16 * kt, mb), ps, dka[mb]);
        }
      }
    };

    // walk (head in group, KV-owned entry, row chunk)
    int hh = 0, e = 0, e1 = 0, c = 0, i = 0, nch = 0;
    auto row_of = [&](int hx) { return ((long long)b * g.Hq + hk * g.group + hx) * g.KVb + j; };
    auto settle = [&]() {  // advance (hh, e) to the next entry with rows, from the current one
      while (hh < g.group) {
        if (e < e1) {
          i = a.col[e];
          nch = (g.q_exist(b, i) + QC - 1) / QC;
          if (nch > 0) return;
          ++e;
          continue;
        }
        ++hh;
        if (hh < g.group) {
          const long long r = row_of(hh);
          e = a.row_ptr[r];
          e1 = a.row_ptr[r + 1];
        }
      }
    };
    {
      const long long r = row_of(0);
      e = a.row_ptr[r];
      e1 = a.row_ptr[r + 1];
      settle();
    }
    if (hh < g.group) {
      stage(0, hk * g.group + hh, i, 0);
      wait_vmem();
      __syncthreads();
      int buf = 0;
      while (true) {
        int nhh = hh, ne = e, ne1 = e1, nc = c + 1, ni = i, nnch = nch;
        if (nc >= nch) {
          const int shh = hh, se = e, se1 = e1, si = i, snch = nch;
          ++e;
          nc = 0;
          settle();
          nhh = hh;
          ne = e;
          ne1 = e1;
          ni = i;
          nnch = nch;
          hh = shh;
          e = se;
          e1 = se1;
          i = si;
          nch = snch;
        }
        const bool has_next = nhh < g.group;
        const int rows_valid = g.q_exist(b, i) - c * QC;
        if (NBUF == 2) {
          if (has_next) stage(buf ^ 1, hk * g.group + nhh, ni, nc);
          compute(buf, rows_valid);
          wait_vmem();
          __syncthreads();
        } else {
          compute(0, rows_valid);
          __syncthreads();
          if (has_next) {
            stage(0, hk * g.group + nhh, ni, nc);
            wait_vmem();
            __syncthreads();
          }
        }
        if (!has_next) break;
        hh = nhh;
        e = ne;
        e1 = ne1;
        c = nc;
        i = ni;
        nch = nnch;
        if (NBUF == 2) buf ^= 1;
      }
    }
  }

  int outkey = mykey;
  bool out_live = key_live;
  if (RG == 2) {
    // row group 1 hands its sums to row group 0 through LDS, then writes the
    // zero gradients of the sub-tile's other (padded) keys
    // one accumulator set at a time: [KS waves][64 values][64 lanes] of fp32
    static_assert(S::KS * 64 * 64 * 4 <= S::LDS, "reduction fits in the tiles' LDS");
    float* red = reinterpret_cast<float*>(smem) + kslot * 64 * 64 + lane;
    auto reduce = [&](f32x16_t(&acc)[4]) {
      __syncthreads();
      if (live > 0 && rg == 1) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) red[(mb * 16 + r) * 64] = acc[mb][r];
      }
      __syncthreads();
      if (live > 0 && rg == 0) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[mb][r] += red[(mb * 16 + r) * 64];
      }
    };
    reduce(dka);
    reduce(dva);
    if (rg == 1) {
      outkey = k0 + KW + 32 * kslot + (lane & 31);
      out_live = false;
    }
  }

  // ---- epilogue: dk = scale * dK + dK_c / valid, dv = dV + dV_c / valid ----
  if (outkey >= kexist || outkey >= k0 + unit) return;
  const long long koff = kbase + (long long)outkey * krs;
  const float* dkc = a.dkc ? a.dkc + g.pk(b, hk, j) : nullptr;
  const float* dvc = a.dvc ? a.dvc + g.pk(b, hk, j) : nullptr;
  const float invn = (out_live && dkc) ? 1.f / (float)nval : 0.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * mb + 8 * q4 + 4 * hl;
      float kx[4], vx[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        kx[u] = out_live ? g.scale * dka[mb][4 * q4 + u] : 0.f;
        vx[u] = out_live ? dva[mb][4 * q4 + u] : 0.f;
      }
      if (dkc && out_live) {
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

// ---------------------------------------------------------------------------
// dQ (Q-owned)
// ---------------------------------------------------------------------------
constexpr int KC = 64;             // keys per chunk
constexpr int KTILE = KC * HD * 2;

template <class ET, int NW>
__global__ __launch_bounds__(NW * 64, 2) void sparse_dq_kernel(const BwdArgs a) {
  using E = Elem<ET>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * 2 * KTILE];  // [stage][K | V]

  const Geom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  const int nsub = g.q_block / (32 * NW);
  int id = xcd_group(blockIdx.x, gridDim.x, nsub);
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
  const int hk = h / g.group;
  const long long kvb = g.kv_base(b, hk), krs = g.kv_rs();

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
  const TrLane tl(lane);

  f32x16_t acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;

  const long long rid = ((long long)b * g.Hq + h) * g.Qb + i;
  const int e0 = a.row_ptr[rid], e1 = a.row_ptr[rid + 1];

  auto stage = [&](int buf, int j, int c, int nval) {
    const int t0 = j * g.kv_block + c * KC;
    const int last = nval - c * KC - 1;
    uint8_t* Ks = smem + buf * 2 * KTILE;
    stage_tile<KC, NW>(Ks, wave, lane, [&](int row) {
      return a.k + kvb + (long long)(t0 + min(row, last)) * krs;
    });
    stage_tile<KC, NW>(Ks + KTILE, wave, lane, [&](int row) {
      return a.v + kvb + (long long)(t0 + min(row, last)) * krs;
    });
  };

  if (e0 < e1) {
    int e = e0, c = 0;
    int j = a.col[e];
    int nval = g.kv_val(b, j);
    stage(0, j, 0, nval);
    wait_vmem();
    __syncthreads();
    int buf = 0;
    while (true) {
      int ne = e, nc = c + 1, nj = j, nnval = nval;
      if (nc * KC >= nval) {
        ne = e + 1;
        nc = 0;
        if (ne < e1) {
          nj = a.col[ne];
          nnval = g.kv_val(b, nj);
        }
      }
      const bool has_next = ne < e1;
      if (has_next) stage(buf ^ 1, nj, nc, nnval);

      const uint8_t* Ks = smem + buf * 2 * KTILE;
      const uint8_t* Vs = Ks + KTILE;
      f32x16_t s0, s1, p0, p1;
#pragma unroll
      for (int r = 0; r < 16; ++r) s0[r] = s1[r] = p0[r] = p1[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        s0 = E::mfma(row16(Ks, l32, 2 * ks + hl), qr[ks], s0);
        s1 = E::mfma(row16(Ks, 32 + l32, 2 * ks + hl), qr[ks], s1);
        p0 = E::mfma(row16(Vs, l32, 2 * ks + hl), dor[ks], p0);
        p1 = E::mfma(row16(Vs, 32 + l32, 2 * ks + hl), dor[ks], p1);
      }
      const int rem = nval - c * KC;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float a0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c2, -lse2));
        float a1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c2, -lse2));
        if (rem < KC) {
          const int key = 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key >= rem) a0 = 0.f;
          if (key + 32 >= rem) a1 = 0.f;
        }
        s0[r] = a0 * (p0[r] - drv);
        s1[r] = a1 * (p1[r] - drv);
      }
      // dQ^T += K^T dS^T (key steps of 16)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const f32x16_t& s = (kt < 2) ? s0 : s1;
        const int o = 8 * (kt & 1);
        const uint4 pb = make_uint4(E::pack(s[o], s[o + 1]), E::pack(s[o + 2], s[o + 3]),
                                    E::pack(s[o + 4], s[o + 5]), E::pack(s[o + 6], s[o + 7]));
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[mb] = E::mfma(tr_operand(Ks, tl, 16 * kt, mb), pb, acc[mb]);
      }
      wait_vmem();
      __syncthreads();
      if (!has_next) break;
      e = ne;
      c = nc;
      j = nj;
      nval = nnval;
      buf ^= 1;
    }
  }

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
      *reinterpret_cast<uint2*>(a.dq + qoff + d0) =
          make_uint2(E::pack(x[0], x[1]), E::pack(x[2], x[3]));
    }
}

template <class ET>
hipError_t launch_pre_t(const PreArgs& a, hipStream_t st) {
  const long long n = (long long)a.g.B * a.g.Hq * a.g.Qb;
  if (n == 0) return hipSuccess;
  bwd_pre_kernel<ET><<<(unsigned)n, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <class ET>
hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const long long tiles = (long long)g.B * g.Hkv * g.KVb;
  if (tiles == 0) return hipSuccess;
  if (g.kv_block % 128 == 0) {
    const unsigned n = (unsigned)(tiles * (g.kv_block / 128));
    sparse_dkdv_kernel<ET, 4, 1, 2><<<n, 256, 0, st>>>(a, DKDV_WIDE);
    sparse_dkdv_kernel<ET, 4, 2, 1><<<n, 256, 0, st>>>(a, DKDV_NARROW);
  } else {
    sparse_dkdv_kernel<ET, 2, 1, 2><<<(unsigned)(tiles * (g.kv_block / 64)), 128, 0, st>>>(a, DKDV_ALL);
  }
  return hipGetLastError();
}

template <class ET>
hipError_t launch_dq_t(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int nw = (g.q_block % 128 == 0) ? 4 : (g.q_block % 64 == 0 ? 2 : 1);
  const long long nwg = (long long)g.B * g.Hq * g.Qb * (g.q_block / (32 * nw));
  if (nwg == 0) return hipSuccess;
  if (nw == 4) sparse_dq_kernel<ET, 4><<<(unsigned)nwg, 256, 0, st>>>(a);
  else if (nw == 2) sparse_dq_kernel<ET, 2><<<(unsigned)nwg, 128, 0, st>>>(a);
  else sparse_dq_kernel<ET, 1><<<(unsigned)nwg, 64, 0, st>>>(a);
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

}  // namespace vsa
