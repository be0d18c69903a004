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
// block's KV list in chunks of 64 keys. K and V chunks go global -> LDS with
// direct 16-byte loads (no staging registers) into a ring of NST slots, so
// NST - 1 chunks are in flight while one is computed (kv_walk.hpp). Scores are formed
// transposed, S^T = K Q^T with v_mfma_f32_32x32x16, so each lane owns one
// query row and the row max / sum are in-lane plus one exchange with lane ^ 32.
// P^T stays in registers as the B operand of O^T += V^T P^T; the V^T operand
// comes straight from the row-major V tile through ds_read_b64_tr_b16, in the
// key order that matches the lane's P values. The chunk loop of a KV block
// stops after ceil(valid/64) chunks; only a partial last chunk runs the mask.
#include "kernels.hpp"
#include "kv_walk.hpp"

namespace vsa {

namespace {

constexpr int KC = KV_CHUNK;

template <class ET, int NW, int NST>
__global__ __launch_bounds__(NW * 64, 2) void sparse_fwd_kernel(const FwdArgs a) {
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

  const int qlen = g.q_len(b);
  const int blk0 = i * g.q_block;
  if (blk0 >= qlen) return;  // Q block outside this sequence
  const int qexist = min(g.q_block, qlen - blk0);
  const int myrow = sub * 32 * NW + wave * 32 + l32;  // row inside the Q block
  const bool row_ok = myrow < qexist;
  const long long qrs = g.q_rs();
  const long long qoff = g.q_base(b, h) + (long long)(blk0 + myrow) * qrs;

  // this wave's query rows: B operand of S^T = K Q^T (lane: row l32, d = 16ks + 8hl + 0..7)
  uint4 qr[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qr[ks] = row_ok ? ldg16(a.q + qoff + 16 * ks + 8 * hl) : make_uint4(0, 0, 0, 0);

  const long long rid = ((long long)b * g.Hq + h) * g.Qb + i;
  const int e0 = __builtin_amdgcn_readfirstlane(a.row_ptr[rid]);  // uniform: the walk stays scalar
  const int cnt = __builtin_amdgcn_readfirstlane(a.row_ptr[rid + 1]) - e0;

  const float c2 = g.scale * LOG2E;
  // exp offset of this lane's row in log2 units: it moves only when a chunk's
  // max exceeds it by more than TAU, so P <= 2^TAU and rescaling is rare
  float msc = -1e30f;
  float l_a = 0.f, l_b = 0.f;  // two partial row sums (of the rounded P)
  f32x16_t acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
  const RowOffs ro(lane);
  const TrOffs to(lane);

  // All-zero query rows (video callers zero the padded slots of partial
  // tiles). Rows of one Q block with equal query values (here: all zero, of
  // either sign) go through identical arithmetic over the same block list, so
  // they get identical outputs. The lowest wave whose 32 rows are all zero
  // runs the general path; the work-group's other all-zero waves skip the
  // chunk arithmetic and copy its accumulators, row sum and exp offset at the
  // end.
  __shared__ int zflag[NW];
  __shared__ float zacc[HD + 2];
  uint32_t nzq = 0;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) nzq |= (qr[ks].x | qr[ks].y | qr[ks].z | qr[ks].w) & 0x7fff7fffu;
  const bool zwave = __ballot(nzq != 0) == 0ull;
  if (lane == 0) zflag[wave] = zwave;
  __syncthreads();
  int zfirst = NW, nzw = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int f = zflag[w];
    if (f && zfirst == NW) zfirst = w;
    nzw += f;
  }
  zfirst = __builtin_amdgcn_readfirstlane(zfirst);
  const bool zshare = __builtin_amdgcn_readfirstlane(nzw) > 1;  // uniform over the work-group
  const bool zlead = zwave && wave == zfirst, zskip = zwave && wave != zfirst;

  walk_kv<NW, NST>(g, b, h / g.group, a.col, e0, cnt, a.k, a.v, wave, lane,
                   [&](const uint8_t* Ks, const uint8_t* Vs, int rem) {
    if (zskip) return;
    // LLVM's MFMA / LDS-read interleaving strategy 0 for the chunk body
    // (measured: forward 3 % faster than the default schedule)
    __builtin_amdgcn_iglp_opt(0);
    // ---- S^T = K Q^T (2 x 32 keys by 32 rows) ----
    f32x16_t s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) s0[r] = s1[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      s0 = E::mfma(ro.at(Ks, 0, ks), qr[ks], s0);
      s1 = E::mfma(ro.at(Ks, 32, ks), qr[ks], s1);
    }
    // lane holds keys 8(r/4) + 4hl + (r%4) (+32 for s1) of its row
    if (rem < KC) {
      const int lim = rem - 4 * hl;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r >> 2) + (r & 3);
        if (kk >= lim) s0[r] = -INFINITY;
        if (kk + 32 >= lim) s1[r] = -INFINITY;
      }
    }
    // chunk max of the row: a maximum3 tree, then the other lane half
    float t[11];
#pragma unroll
    for (int u = 0; u < 5; ++u) {
      t[u] = vmax3(s0[3 * u], s0[3 * u + 1], s0[3 * u + 2]);
      t[5 + u] = vmax3(s1[3 * u], s1[3 * u + 1], s1[3 * u + 2]);
    }
    t[10] = vmax(s0[15], s1[15]);
    float mx = vmax3(vmax3(t[0], t[1], t[2]), vmax3(t[3], t[4], t[5]), vmax3(t[6], t[7], t[8]));
    mx = xhalf_max(vmax3(mx, t[9], t[10]));
    constexpr float TAU = 8.f;
    if (mx * c2 > msc + TAU) {  // move the offset to this chunk's max
      const float nm = mx * c2;
      const float alpha = __builtin_amdgcn_exp2f(msc - nm);
      l_a *= alpha;
      l_b *= alpha;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][r] *= alpha;
      msc = nm;
    }

    // ---- P^T, its row sums, and O^T += V^T P^T: 4 key steps of 16 ----
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x16_t& sv = (kt < 2) ? s0 : s1;
      const int o = 8 * (kt & 1);
      float pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) pv[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[o + u], c2, -msc));
      const uint4 pb = make_uint4(E::pack(pv[0], pv[1]), E::pack(pv[2], pv[3]), E::pack(pv[4], pv[5]),
                                  E::pack(pv[6], pv[7]));
      l_a = E::sum2(pb.x, l_a);
      l_b = E::sum2(pb.y, l_b);
      l_a = E::sum2(pb.z, l_a);
      l_b = E::sum2(pb.w, l_b);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] = E::mfma(to.at(Vs, 16 * kt, mb), pb, acc[mb]);
    }
  });

  float l_run = xhalf_sum(l_a + l_b);
  if (zshare) {  // every row of the leading all-zero wave holds the shared result
    if (zlead && l32 == 0) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) zacc[32 * mb + 8 * (r >> 2) + 4 * hl + (r & 3)] = acc[mb][r];
      if (hl == 0) {
        zacc[HD] = l_run;
        zacc[HD + 1] = msc;
      }
    }
    __syncthreads();
    if (zskip) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[mb][r] = zacc[32 * mb + 8 * (r >> 2) + 4 * hl + (r & 3)];
      l_run = zacc[HD];
      msc = zacc[HD + 1];
    }
  }
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  if (!row_ok) return;
  if (hl == 0)  // natural-log LSE: (offset + log2 l) * ln 2
    a.lse[g.lse_base(b, h) + blk0 + myrow] =
        l_run > 0.f ? (msc + __builtin_amdgcn_logf(l_run)) * 0.69314718055994531f : -INFINITY;
  float gt = 0.f;
  if (a.gate_mode == VSA_GATE_PER_TOKEN) {
    gt = E::lo(a.gate[g.gtok_base(b, h) + (long long)(blk0 + myrow) * g.gtok_rs()]);
  } else if (a.gate_mode == VSA_GATE_PROJECTED) {
    // sigmoid(<q row, w_h> + b_h): this lane's 64 elements of the row (d =
    // 16ks + 8hl + 0..7, already in registers), then the other lane half's
    const float* w = a.gproj + h * HD + 8 * hl;
    float z = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const float4 w0 = *reinterpret_cast<const float4*>(w + 16 * ks);
      const float4 w1 = *reinterpret_cast<const float4*>(w + 16 * ks + 4);
      z = __builtin_fmaf(E::lo(qr[ks].x), w0.x, z);
      z = __builtin_fmaf(E::hi(qr[ks].x), w0.y, z);
      z = __builtin_fmaf(E::lo(qr[ks].y), w0.z, z);
      z = __builtin_fmaf(E::hi(qr[ks].y), w0.w, z);
      z = __builtin_fmaf(E::lo(qr[ks].z), w1.x, z);
      z = __builtin_fmaf(E::hi(qr[ks].z), w1.y, z);
      z = __builtin_fmaf(E::lo(qr[ks].w), w1.z, z);
      z = __builtin_fmaf(E::hi(qr[ks].w), w1.w, z);
    }
    z = xhalf_sum(z) + a.gproj[g.Hq * HD + h];
    gt = 1.f / (1.f + __builtin_amdgcn_exp2f(-z * LOG2E));
    if (a.gate_out && hl == 0)
      a.gate_out[g.gtok_base(b, h) + (long long)(blk0 + myrow) * g.gtok_rs()] =
          (uint16_t)(E::pack(gt, 0.f) & 0xffffu);
  }
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
  const int nw = g.q_block % 256 == 0 ? 8 : g.q_block % 128 == 0 ? 4 : g.q_block % 64 == 0 ? 2 : 1;
  const long long nwg = (long long)g.B * g.Hq * g.Qb * max(1, g.q_block / (32 * nw));
  if (nwg == 0) return hipSuccess;
  if (nw == 8) sparse_fwd_kernel<ET, 8, 4><<<(unsigned)nwg, 512, 0, st>>>(a);
  else if (nw == 4) sparse_fwd_kernel<ET, 4, 2><<<(unsigned)nwg, 256, 0, st>>>(a);
  else if (nw == 2) sparse_fwd_kernel<ET, 2, 2><<<(unsigned)nwg, 128, 0, st>>>(a);
  else sparse_fwd_kernel<ET, 1, 2><<<(unsigned)nwg, 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_fwd(const FwdArgs& a, int dtype, hipStream_t st) {
  return dtype == VSA_BF16 ? launch_fwd_t<bf16_tag>(a, st) : launch_fwd_t<f16_tag>(a, st);
}

}  // namespace vsa
