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
    if (dg == 0) a.dr[g.lse_base(b, h) + blk0 + s] = part;
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
constexpr int QC = 32;         // query rows per chunk
constexpr int NSTR = HD + 8;   // row-major stride (elements)
constexpr int TSTR = QC + 4;   // transposed stride (elements): 72 B, conflict-free b64 reads
constexpr int KV_STAGE = 2 * QC * NSTR + 2 * HD * TSTR + 2 * QC * 2;  // + lse2, dr (as floats)

template <class ET, int NW>
__global__ __launch_bounds__(NW * 64, 1) void sparse_dkdv_kernel(const BwdArgs a) {
  using E = Elem<ET>;
  constexpr int NT = NW * 64;
  constexpr int TU = (2 * (QC / 4) * (HD / 8)) / NT;  // (4 rows x 8 d) pieces of Q and dO per thread
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * KV_STAGE];

  const Geom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  const int nsub = g.kv_block / (32 * NW);
  int id = xcd_remap(blockIdx.x, gridDim.x);
  const int sub = id % nsub;
  id /= nsub;
  const int j = id % g.KVb;
  id /= g.KVb;
  const int hk = id % g.Hkv, b = id / g.Hkv;

  const int kexist = g.kv_exist(b, j);
  const int k0 = sub * 32 * NW;
  if (k0 >= kexist) return;  // no key of this sub-tile exists
  const int nval = g.kv_val(b, j);
  const int mykey = k0 + wave * 32 + l32;  // key inside the KV block
  const bool key_ok = mykey < kexist, key_live = mykey < nval;
  const long long krs = g.kv_rs();
  const long long koff = g.kv_base(b, hk) + (long long)(j * g.kv_block + mykey) * krs;

  f32x16_t dka[4], dva[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dka[mb][r] = dva[mb][r] = 0.f;

  if (k0 < nval) {
    // B operands: K^T and V^T columns (lane: key l32, d = 16ks + 8hl + 0..7)
    uint4 kr[8], vr[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kr[ks] = key_live ? ldg16(a.k + koff + 16 * ks + 8 * hl) : make_uint4(0, 0, 0, 0);
      vr[ks] = key_live ? ldg16(a.v + koff + 16 * ks + 8 * hl) : make_uint4(0, 0, 0, 0);
    }
    const float c2 = g.scale * LOG2E;
    const long long qrs = g.q_rs();
    uint4 st[TU][4];
    float lst = 0.f;  // lse2 or dr of one staged row (threads 0..63)

    // one chunk = (head h, Q block i, rows 32c .. 32c+31)
    auto load_chunk = [&](int h, int i, int c) {
      const int qex = g.q_exist(b, i);
      const int r0 = c * QC;
      const long long base = g.q_base(b, h) + (long long)(i * g.q_block + r0) * qrs;
#pragma unroll
      for (int u = 0; u < TU; ++u) {
        const int it = tid + u * NT;  // 0..255: first half Q, second half dO
        const int which = it >> 7, w = it & 127, dg = w & 15, rg = w >> 4;
        const uint16_t* src = which ? a.dout : a.q;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int row = 4 * rg + rr;
          st[u][rr] = (r0 + row < qex) ? ldg16(src + base + (long long)row * qrs + 8 * dg)
                                       : make_uint4(0, 0, 0, 0);
        }
      }
      if (tid < 2 * QC) {
        const int row = tid & (QC - 1);
        const long long lb = g.lse_base(b, h) + i * g.q_block + r0 + row;
        if (r0 + row < qex) {
          if (tid < QC) {
            const float l = a.lse[lb];
            lst = l == -INFINITY ? INFINITY : l * LOG2E;
          } else {
            lst = a.dr[lb];
          }
        } else {
          lst = tid < QC ? INFINITY : 0.f;
        }
      }
    };
    auto store_chunk = [&](int buf) {
      uint16_t* base = smem + buf * KV_STAGE;
#pragma unroll
      for (int u = 0; u < TU; ++u) {
        const int it = tid + u * NT;
        const int which = it >> 7, w = it & 127, dg = w & 15, rg = w >> 4;
        uint16_t* nat = base + which * (QC * NSTR);
        uint16_t* tr = base + 2 * QC * NSTR + which * (HD * TSTR);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          *reinterpret_cast<uint4*>(nat + (4 * rg + rr) * NSTR + 8 * dg) = st[u][rr];
        const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&st[u][0]);
        const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&st[u][1]);
        const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&st[u][2]);
        const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&st[u][3]);
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          uint2 even, odd;
          even.x = (r0[w2] & 0xffffu) | (r1[w2] << 16);
          even.y = (r2[w2] & 0xffffu) | (r3[w2] << 16);
          odd.x = (r0[w2] >> 16) | (r1[w2] & 0xffff0000u);
          odd.y = (r2[w2] >> 16) | (r3[w2] & 0xffff0000u);
          *reinterpret_cast<uint2*>(tr + (8 * dg + 2 * w2) * TSTR + 4 * rg) = even;
          *reinterpret_cast<uint2*>(tr + (8 * dg + 2 * w2 + 1) * TSTR + 4 * rg) = odd;
        }
      }
      if (tid < 2 * QC) {
        float* fl = reinterpret_cast<float*>(base + 2 * QC * NSTR + 2 * HD * TSTR);
        fl[tid] = lst;
      }
    };

    // walk (head in group, KV-owned entry, row chunk)
    int hh = 0, e = 0, e1 = 0, c = 0, i = 0, nch = 0;
    auto row_of = [&](int hx) { return ((long long)b * g.Hq + hk * g.group + hx) * g.KVb + j; };
    // advance (hh, e) to the next non-empty position, starting at the current one
    auto settle = [&]() {
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
      load_chunk(hk * g.group + hh, i, 0);
      store_chunk(0);
      __syncthreads();
      int buf = 0;
      while (true) {
        // the chunk after this one
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
        if (has_next) load_chunk(hk * g.group + nhh, ni, nc);

        const uint16_t* base = smem + buf * KV_STAGE;
        const uint16_t* Qn = base;
        const uint16_t* Dn = base + QC * NSTR;
        const uint16_t* Qt = base + 2 * QC * NSTR;
        const uint16_t* Dt = Qt + HD * TSTR;
        const float* lse2 = reinterpret_cast<const float*>(base + 2 * QC * NSTR + 2 * HD * TSTR);
        const float* drs = lse2 + QC;

        // S = Q K^T and dP = dO V^T (rows 8(r/4) + 4hl + r%4, key column l32)
        f32x16_t s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const uint4 aq = *reinterpret_cast<const uint4*>(Qn + l32 * NSTR + 16 * ks + 8 * hl);
          const uint4 ad = *reinterpret_cast<const uint4*>(Dn + l32 * NSTR + 16 * ks + 8 * hl);
          s = E::mfma(aq, kr[ks], s);
          dp = E::mfma(ad, vr[ks], dp);
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 l4 = *reinterpret_cast<const float4*>(lse2 + 8 * q4 + 4 * hl);
          const float4 d4 = *reinterpret_cast<const float4*>(drs + 8 * q4 + 4 * hl);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
          const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = 4 * q4 + u;
            const float p = key_live ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c2, -lv[u])) : 0.f;
            s[r] = p;
            dp[r] = p * (dp[r] - dv[u]);
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
            const int ro = (32 * mb + l32) * TSTR + 16 * kt + 4 * hl;
            const uint2 dlo = *reinterpret_cast<const uint2*>(Dt + ro);
            const uint2 dhi = *reinterpret_cast<const uint2*>(Dt + ro + 8);
            const uint2 qlo = *reinterpret_cast<const uint2*>(Qt + ro);
            const uint2 qhi = *reinterpret_cast<const uint2*>(Qt + ro + 8);
            dva[mb] = E::mfma(make_uint4(dlo.x, dlo.y, dhi.x, dhi.y), pp, dva[mb]);
            dka[mb] = E::mfma(make_uint4(qlo.x, qlo.y, qhi.x, qhi.y), ps, dka[mb]);
          }
        }

        if (has_next) store_chunk(buf ^ 1);
        __syncthreads();
        if (!has_next) break;
        hh = nhh;
        e = ne;
        e1 = ne1;
        c = nc;
        i = ni;
        nch = nnch;
        buf ^= 1;
      }
    }
  }

  // ---- epilogue: dk = scale * dK + dK_c / valid, dv = dV + dV_c / valid ----
  if (!key_ok) return;
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

// ---------------------------------------------------------------------------
// dQ (Q-owned)
// ---------------------------------------------------------------------------
constexpr int KC = 64;
constexpr int KSTR = HD + 8;
constexpr int KTSTR = KC + 4;
constexpr int DQ_STAGE = 2 * KC * KSTR + HD * KTSTR;  // K, V row-major + K^T

template <class ET, int NW>
__global__ __launch_bounds__(NW * 64, 1) void sparse_dq_kernel(const BwdArgs a) {
  using E = Elem<ET>;
  constexpr int NT = NW * 64;
  constexpr int KU = (KC * HD / 8) / NT;
  constexpr int TU = (KC / 4) * (HD / 8) / NT;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * DQ_STAGE];

  const Geom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, l32 = lane & 31;
  const int nsub = g.q_block / (32 * NW);
  int id = xcd_remap(blockIdx.x, gridDim.x);
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
  float lse2 = INFINITY, drv = 0.f;
  if (row_ok) {
    const float l = a.lse[lrow];
    lse2 = l == -INFINITY ? INFINITY : l * LOG2E;
    drv = a.dr[lrow];
  }
  const float c2 = g.scale * LOG2E;

  f32x16_t acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;

  const long long rid = ((long long)b * g.Hq + h) * g.Qb + i;
  const int e0 = a.row_ptr[rid], e1 = a.row_ptr[rid + 1];
  uint4 kst[KU], vst[KU], tst[TU][4];

  auto load_chunk = [&](int j, int c, int nval) {
    const int t0 = j * g.kv_block + c * KC;
    const int rem = nval - c * KC;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int idx = tid + u * NT, key = idx >> 4, dq = idx & 15;
      const bool ok = key < rem;
      const long long off = kvb + (long long)(t0 + key) * krs + 8 * dq;
      kst[u] = ok ? ldg16(a.k + off) : make_uint4(0, 0, 0, 0);
      vst[u] = ok ? ldg16(a.v + off) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      const int it = tid + u * NT, dg = it & 15, kg = it >> 4;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = 4 * kg + rr;
        tst[u][rr] = key < rem ? ldg16(a.k + kvb + (long long)(t0 + key) * krs + 8 * dg)
                               : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_chunk = [&](int buf) {
    uint16_t* Ks = smem + buf * DQ_STAGE;
    uint16_t* Vs = Ks + KC * KSTR;
    uint16_t* Kt = Vs + KC * KSTR;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int idx = tid + u * NT, key = idx >> 4, dq = idx & 15;
      *reinterpret_cast<uint4*>(Ks + key * KSTR + 8 * dq) = kst[u];
      *reinterpret_cast<uint4*>(Vs + key * KSTR + 8 * dq) = vst[u];
    }
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      const int it = tid + u * NT, dg = it & 15, kg = it >> 4;
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&tst[u][0]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&tst[u][1]);
      const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&tst[u][2]);
      const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&tst[u][3]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint2 even, odd;
        even.x = (r0[w] & 0xffffu) | (r1[w] << 16);
        even.y = (r2[w] & 0xffffu) | (r3[w] << 16);
        odd.x = (r0[w] >> 16) | (r1[w] & 0xffff0000u);
        odd.y = (r2[w] >> 16) | (r3[w] & 0xffff0000u);
        *reinterpret_cast<uint2*>(Kt + (8 * dg + 2 * w) * KTSTR + 4 * kg) = even;
        *reinterpret_cast<uint2*>(Kt + (8 * dg + 2 * w + 1) * KTSTR + 4 * kg) = odd;
      }
    }
  };

  if (e0 < e1) {
    int e = e0, c = 0;
    int j = a.col[e];
    int nval = g.kv_val(b, j);
    load_chunk(j, c, nval);
    store_chunk(0);
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
      if (has_next) load_chunk(nj, nc, nnval);

      const uint16_t* Ks = smem + buf * DQ_STAGE;
      const uint16_t* Vs = Ks + KC * KSTR;
      const uint16_t* Kt = Vs + KC * KSTR;
      f32x16_t s0, s1, p0, p1;
#pragma unroll
      for (int r = 0; r < 16; ++r) s0[r] = s1[r] = p0[r] = p1[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int o0 = l32 * KSTR + 16 * ks + 8 * hl, o1 = o0 + 32 * KSTR;
        s0 = E::mfma(*reinterpret_cast<const uint4*>(Ks + o0), qr[ks], s0);
        s1 = E::mfma(*reinterpret_cast<const uint4*>(Ks + o1), qr[ks], s1);
        p0 = E::mfma(*reinterpret_cast<const uint4*>(Vs + o0), dor[ks], p0);
        p1 = E::mfma(*reinterpret_cast<const uint4*>(Vs + o1), dor[ks], p1);
      }
      const int rem = nval - c * KC;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * hl + (r & 3);
        float a0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c2, -lse2));
        float a1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c2, -lse2));
        if (key >= rem) a0 = 0.f;
        if (key + 32 >= rem) a1 = 0.f;
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
        for (int mb = 0; mb < 4; ++mb) {
          const uint16_t* kp = Kt + (32 * mb + l32) * KTSTR + 16 * kt + 4 * hl;
          const uint2 lo = *reinterpret_cast<const uint2*>(kp);
          const uint2 hi = *reinterpret_cast<const uint2*>(kp + 8);
          acc[mb] = E::mfma(make_uint4(lo.x, lo.y, hi.x, hi.y), pb, acc[mb]);
        }
      }
      if (has_next) store_chunk(buf ^ 1);
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
  const int nw = (g.kv_block % 128 == 0) ? 4 : 2;
  const long long nwg = (long long)g.B * g.Hkv * g.KVb * (g.kv_block / (32 * nw));
  if (nwg == 0) return hipSuccess;
  if (nw == 4) sparse_dkdv_kernel<ET, 4><<<(unsigned)nwg, 256, 0, st>>>(a);
  else sparse_dkdv_kernel<ET, 2><<<(unsigned)nwg, 128, 0, st>>>(a);
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
