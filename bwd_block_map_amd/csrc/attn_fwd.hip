// Sparse-branch forward: softmax attention of every Q row over the valid keys
// of the KV blocks its Q block selected, with the natural-log LSE, and the
// gated composition out = O_sel + gate * O_c in the epilogue.
//
// Semantics: FastVideo block_sparse_attn_cute_fwd.py (`_cute_attention`:
// Q-owned block lists, the per-tile valid-token mask of `_build_vbs_mask_mod`,
// LSE returned as [B,H,S]); Ascend op-plugin test page, forward goldens
// (masked row softmax, LSE = logsumexp of the scaled masked scores).
//
// gfx950 design. One work-group = NW waves x 32 rows of one Q block; every
// wave keeps its 32 query rows in registers as MFMA B operands and walks the
// block's KV list in chunks of 64 keys staged through LDS (double-buffered:
// the next chunk's global loads are issued before this chunk's MFMAs and
// written to the other LDS stage after them). Scores are formed transposed,
// S^T = K Q^T with v_mfma_f32_32x32x16, so each lane owns one query row and
// the row max / sum are in-lane plus one exchange with lane ^ 32. P^T feeds
// O^T += V^T P^T directly from registers: the MFMA contraction order is free,
// so the (4 keys, 4 keys) split of each lane's P values is matched by reading
// V^T from LDS at the same key positions. V is transposed once, while it is
// written to LDS. The chunk loop of a KV block stops after ceil(valid/64)
// chunks; only a partial last chunk runs the key mask.
#include "kernels.hpp"

namespace vsa {

namespace {

constexpr int KC = 64;         // keys per chunk
constexpr int KSTR = HD + 8;   // LDS row stride of K (elements): 272 B, conflict-free b128 reads
constexpr int VSTR = KC + 4;   // LDS row stride of V^T (elements): 136 B, conflict-free b64 reads
constexpr int STAGE = KC * KSTR + HD * VSTR;  // elements per LDS stage

template <class ET, int NW>
__global__ __launch_bounds__(NW * 64, 2) void sparse_fwd_kernel(const FwdArgs a) {
  using E = Elem<ET>;
  constexpr int NT = NW * 64;
  constexpr int KU = (KC * HD / 8) / NT;  // 16-byte K pieces per thread
  constexpr int VU = (KC / 4) * (HD / 8) / NT;  // (4 keys x 8 d) V pieces per thread
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

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

  const int qlen = g.q_len(b);
  const int blk0 = i * g.q_block;
  if (blk0 >= qlen) return;  // Q block outside this sequence
  const int qexist = min(g.q_block, qlen - blk0);
  const int myrow = sub * 32 * NW + wave * 32 + l32;  // row inside the Q block
  const bool row_ok = myrow < qexist;
  const long long qrs = g.q_rs();
  const long long qoff = g.q_base(b, h) + (long long)(blk0 + myrow) * qrs;
  const int hk = h / g.group;
  const long long kvb = g.kv_base(b, hk), krs = g.kv_rs();

  // this wave's query rows: B operand of S^T = K Q^T (lane: row l32, d = 16ks + 8hl + 0..7)
  uint4 qr[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qr[ks] = row_ok ? ldg16(a.q + qoff + 16 * ks + 8 * hl) : make_uint4(0, 0, 0, 0);

  const long long rid = ((long long)b * g.Hq + h) * g.Qb + i;
  const int e0 = a.row_ptr[rid], e1 = a.row_ptr[rid + 1];

  const float c2 = g.scale * LOG2E;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;

  uint4 kst[KU];
  uint4 vst[VU][4];

  // global -> registers for chunk c of KV block j (keys >= nval read as zero)
  auto load_chunk = [&](int j, int c, int nval) {
    const int t0 = j * g.kv_block + c * KC;
    const int rem = nval - c * KC;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int idx = tid + u * NT, key = idx >> 4, dq = idx & 15;
      kst[u] = key < rem ? ldg16(a.k + kvb + (long long)(t0 + key) * krs + 8 * dq)
                         : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int it = tid + u * NT, dg = it & 15, kg = it >> 4;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = 4 * kg + rr;
        vst[u][rr] = key < rem ? ldg16(a.v + kvb + (long long)(t0 + key) * krs + 8 * dg)
                               : make_uint4(0, 0, 0, 0);
      }
    }
  };
  // registers -> LDS stage: K row-major, V transposed (V^T[d][key])
  auto store_chunk = [&](int buf) {
    uint16_t* Ks = smem + buf * STAGE;
    uint16_t* Vt = Ks + KC * KSTR;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int idx = tid + u * NT, key = idx >> 4, dq = idx & 15;
      *reinterpret_cast<uint4*>(Ks + key * KSTR + 8 * dq) = kst[u];
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
      const int it = tid + u * NT, dg = it & 15, kg = it >> 4;
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&vst[u][0]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&vst[u][1]);
      const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&vst[u][2]);
      const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&vst[u][3]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // d = 8dg + 2w (low halves) and 8dg + 2w + 1 (high halves)
        uint2 even, odd;
        even.x = (r0[w] & 0xffffu) | (r1[w] << 16);
        even.y = (r2[w] & 0xffffu) | (r3[w] << 16);
        odd.x = (r0[w] >> 16) | (r1[w] & 0xffff0000u);
        odd.y = (r2[w] >> 16) | (r3[w] & 0xffff0000u);
        *reinterpret_cast<uint2*>(Vt + (8 * dg + 2 * w) * VSTR + 4 * kg) = even;
        *reinterpret_cast<uint2*>(Vt + (8 * dg + 2 * w + 1) * VSTR + 4 * kg) = odd;
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
      // the chunk after this one
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

      // ---- this chunk: S^T = K Q^T (2 x 32 keys by 32 rows) ----
      const uint16_t* Ks = smem + buf * STAGE;
      const uint16_t* Vt = Ks + KC * KSTR;
      f32x16_t s0, s1;
#pragma unroll
      for (int r = 0; r < 16; ++r) s0[r] = s1[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const uint4 a0 = *reinterpret_cast<const uint4*>(Ks + l32 * KSTR + 16 * ks + 8 * hl);
        const uint4 a1 =
            *reinterpret_cast<const uint4*>(Ks + (32 + l32) * KSTR + 16 * ks + 8 * hl);
        s0 = E::mfma(a0, qr[ks], s0);
        s1 = E::mfma(a1, qr[ks], s1);
      }
      // lane holds keys 8(r/4) + 4hl + (r%4) (+32 for s1) of its row
      const int rem = nval - c * KC;
      if (rem < KC) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key >= rem) s0[r] = -INFINITY;
          if (key + 32 >= rem) s1[r] = -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      mx = xhalf_max(mx);
      const float mnew = fmaxf(m_run, mx);
      const float msc = mnew == -INFINITY ? 0.f : mnew * c2;
      const float alpha = __builtin_amdgcn_exp2f(m_run * c2 - msc);
      m_run = mnew;
      float lsum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c2, -msc));
        s1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c2, -msc));
        lsum += s0[r] + s1[r];
      }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][r] *= alpha;

      // ---- O^T += V^T P^T: 4 key steps of 16 ----
      uint4 pb[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const f32x16_t& s = (kt < 2) ? s0 : s1;
        const int o = 8 * (kt & 1);
        pb[kt] = make_uint4(E::pack(s[o + 0], s[o + 1]), E::pack(s[o + 2], s[o + 3]),
                            E::pack(s[o + 4], s[o + 5]), E::pack(s[o + 6], s[o + 7]));
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const uint16_t* vp = Vt + (32 * mb + l32) * VSTR + 16 * kt + 4 * hl;
          const uint2 lo = *reinterpret_cast<const uint2*>(vp);
          const uint2 hi = *reinterpret_cast<const uint2*>(vp + 8);
          acc[mb] = E::mfma(make_uint4(lo.x, lo.y, hi.x, hi.y), pb[kt], acc[mb]);
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

  // ---- epilogue ----
  l_run = xhalf_sum(l_run);
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  if (!row_ok) return;
  if (hl == 0)
    a.lse[g.lse_base(b, h) + blk0 + myrow] =
        l_run > 0.f ? m_run * g.scale + __logf(l_run) : -INFINITY;
  float gt = 0.f;
  if (a.gate_mode == VSA_GATE_PER_TOKEN)
    gt = E::lo(a.gate[g.gtok_base(b, h) + (long long)(blk0 + myrow) * g.gtok_rs()]);
  const float* ocp = a.gate_mode != VSA_GATE_NONE ? a.oc + g.pq(b, h, i) : nullptr;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * mb + 8 * q4 + 4 * hl;  // 4 consecutive d of this lane
      float o0 = acc[mb][4 * q4 + 0] * inv, o1 = acc[mb][4 * q4 + 1] * inv;
      float o2 = acc[mb][4 * q4 + 2] * inv, o3 = acc[mb][4 * q4 + 3] * inv;
      if (a.gate_mode != VSA_GATE_NONE) {
        if (a.osel)
          *reinterpret_cast<uint2*>(a.osel + qoff + d0) =
              make_uint2(E::pack(o0, o1), E::pack(o2, o3));
        const float4 oc = *reinterpret_cast<const float4*>(ocp + d0);
        float g0 = gt, g1 = gt, g2 = gt, g3 = gt;
        if (a.gate_mode == VSA_GATE_PER_ELEMENT) {
          const uint2 gv = *reinterpret_cast<const uint2*>(a.gate + qoff + d0);
          g0 = E::lo(gv.x);
          g1 = E::hi(gv.x);
          g2 = E::lo(gv.y);
          g3 = E::hi(gv.y);
        }
        o0 = __builtin_fmaf(g0, oc.x, o0);
        o1 = __builtin_fmaf(g1, oc.y, o1);
        o2 = __builtin_fmaf(g2, oc.z, o2);
        o3 = __builtin_fmaf(g3, oc.w, o3);
      }
      *reinterpret_cast<uint2*>(a.out + qoff + d0) = make_uint2(E::pack(o0, o1), E::pack(o2, o3));
    }
}

template <class ET>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int nw = (g.q_block % 128 == 0) ? 4 : (g.q_block % 64 == 0 ? 2 : 1);
  const long long nwg = (long long)g.B * g.Hq * g.Qb * (g.q_block / (32 * nw));
  if (nwg == 0) return hipSuccess;
  if (nw == 4) sparse_fwd_kernel<ET, 4><<<(unsigned)nwg, 256, 0, st>>>(a);
  else if (nw == 2) sparse_fwd_kernel<ET, 2><<<(unsigned)nwg, 128, 0, st>>>(a);
  else sparse_fwd_kernel<ET, 1><<<(unsigned)nwg, 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_fwd(const FwdArgs& a, int dtype, hipStream_t st) {
  return dtype == VSA_BF16 ? launch_fwd_t<bf16_tag>(a, st) : launch_fwd_t<f16_tag>(a, st);
}

}  // namespace vsa
