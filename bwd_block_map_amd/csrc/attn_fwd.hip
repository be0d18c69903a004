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
// direct 16-byte loads (no staging registers), double-buffered: the next
// chunk is in flight while this one is computed. Scores are formed
// transposed, S^T = K Q^T with v_mfma_f32_32x32x16, so each lane owns one
// query row and the row max / sum are in-lane plus one exchange with lane ^ 32.
// P^T stays in registers as the B operand of O^T += V^T P^T; the V^T operand
// comes straight from the row-major V tile through ds_read_b64_tr_b16, in the
// key order that matches the lane's P values. The chunk loop of a KV block
// stops after ceil(valid/64) chunks; only a partial last chunk runs the mask.
#include <type_traits>

#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace vsa {

namespace {

constexpr int KC = 64;             // keys per chunk
constexpr int TILE = KC * HD * 2;  // bytes of one 64-row tile
constexpr int LIST_CAP = 1024;     // block-list entries held in LDS at a time

template <int I>
using Slot = std::integral_constant<int, I>;

template <class ET, int NW, int NST>
__global__ __launch_bounds__(NW * 64, 2) void sparse_fwd_kernel(const FwdArgs a) {
  using E = Elem<ET>;
  static_assert(NST == 2 || NST == 4, "stage ring of 2 or 4");
  // K and V tiles of the NST stages as distinct LDS objects: with the stage
  // fixed at compile time the compiler can tell the tiles being filled from
  // the ones being read, and does not wait for the prefetch before reading
  __shared__ __attribute__((aligned(1024))) uint8_t sK0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t sK2[NST > 2 ? TILE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sV2[NST > 2 ? TILE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sK3[NST > 2 ? TILE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sV3[NST > 2 ? TILE : 16];
  __shared__ int lst_j[LIST_CAP];  // a page of this row's block list: block and valid keys
  __shared__ int lst_v[LIST_CAP];

  const Geom& g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: wave-level values stay scalar
  const int hl = lane >> 5, l32 = lane & 31;

  const int nsub = g.q_block / (32 * NW);
  int id = xcd_group(blockIdx.x, gridDim.x, nsub);
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
  const uint32_t krs_bytes = (uint32_t)(krs * 2);

  // this wave's query rows: B operand of S^T = K Q^T (lane: row l32, d = 16ks + 8hl + 0..7)
  uint4 qr[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qr[ks] = row_ok ? ldg16(a.q + qoff + 16 * ks + 8 * hl) : make_uint4(0, 0, 0, 0);

  const long long rid = ((long long)b * g.Hq + h) * g.Qb + i;
  const int e0 = a.row_ptr[rid];
  const int cnt = a.row_ptr[rid + 1] - e0;

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

  // ---- the block list, a page of LIST_CAP entries at a time, in LDS ----
  const int kvlen = g.kv_len(b);
  auto load_page = [&](int base) {
    for (int t = tid; t < LIST_CAP && base + t < cnt; t += NW * 64) {
      const int j = a.col[e0 + base + t];
      const int ex = max(0, min(g.kv_block, kvlen - j * g.kv_block));
      lst_j[t] = j;
      lst_v[t] = g.kv_valid ? min(g.kv_valid[j], ex) : ex;
    }
  };
  if (cnt == 0) goto epilogue;
  load_page(0);
  wait_vm<0>();  // the query rows and the list page have landed
  __syncthreads();

  {
    // stager: the next chunk to load (entry se of the list, chunk sc of block sj)
    int se = 0, sc = 0, page = 0;
    int sj = lst_j[0], snv = lst_v[0];
    bool more = true;
    auto advance = [&]() {
      if (++sc * KC < snv) return;
      sc = 0;
      if (++se >= cnt) {
        more = false;
        return;
      }
      if (se - page >= LIST_CAP) {  // next page (only for lists longer than LIST_CAP)
        __syncthreads();
        page = se;
        load_page(page);
        __syncthreads();
      }
      sj = lst_j[se - page];
      snv = lst_v[se - page];
    };
    // per slot: whether it holds a chunk, and that chunk's number of valid keys
    bool have[NST];
    int rem[NST];
    auto tileK = [&](auto sid) -> uint8_t* {
      constexpr int S = decltype(sid)::value;
      if constexpr (S == 0) return sK0;
      else if constexpr (S == 1) return sK1;
      else if constexpr (S == 2) return sK2;
      else return sK3;
    };
    auto tileV = [&](auto sid) -> uint8_t* {
      constexpr int S = decltype(sid)::value;
      if constexpr (S == 0) return sV0;
      else if constexpr (S == 1) return sV1;
      else if constexpr (S == 2) return sV2;
      else return sV3;
    };
    // load the stager's chunk into slot sid (rows past the valid keys repeat
    // the last valid row: in bounds, and masked out of the softmax)
    auto fill = [&](auto sid) {
      constexpr int S = decltype(sid)::value;
      have[S] = more;
      if (!more) return;
      const long long t0 = kvb + (long long)(sj * g.kv_block + sc * KC) * krs;
      const int left = snv - sc * KC;
      rem[S] = left;
      stage_rows<KC, NW>(tileK(sid), wave, lane, a.k + t0, krs_bytes, left - 1);
      stage_rows<KC, NW>(tileV(sid), wave, lane, a.v + t0, krs_bytes, left - 1);
      advance();
    };
    constexpr int LPC = 2 * rows_loads<KC, NW>();  // direct loads per chunk and wave

    // one chunk: refill the slot freed last step, compute slot sid, wait for the next
    auto step = [&](auto sid) -> bool {
      constexpr int S = decltype(sid)::value;
      fill(Slot<(S + NST - 1) % NST>{});
      const uint8_t* Ks = tileK(sid);
      const uint8_t* Vs = tileV(sid);

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
      if (rem[S] < KC) {
        const int lim = rem[S] - 4 * hl;
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

      // the next slot's chunk must have landed; later chunks may stay in flight
      if constexpr (NST == 4) {
        const int later = (int)have[(S + 2) % NST] + (int)have[(S + 3) % NST];
        if (later == 2) wait_vm<2 * LPC>();
        else if (later == 1) wait_vm<LPC>();
        else wait_vm<0>();
      } else {
        wait_vm<0>();
      }
      lds_barrier();
      return have[(S + 1) % NST];
    };

    // prologue: the first NST - 1 chunks in flight
    fill(Slot<0>{});
    if constexpr (NST == 4) {
      fill(Slot<1>{});
      fill(Slot<2>{});
      const int later = (int)have[1] + (int)have[2];
      if (later == 2) wait_vm<2 * LPC>();
      else if (later == 1) wait_vm<LPC>();
      else wait_vm<0>();
    } else {
      wait_vm<0>();
    }
    lds_barrier();
    if constexpr (NST == 4) {
      while (step(Slot<0>{}) && step(Slot<1>{}) && step(Slot<2>{}) && step(Slot<3>{})) {
      }
    } else {
      while (step(Slot<0>{}) && step(Slot<1>{})) {
      }
    }
  }

epilogue:
  const float l_run = xhalf_sum(l_a + l_b);
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  if (!row_ok) return;
  if (hl == 0)  // natural-log LSE: (offset + log2 l) * ln 2
    a.lse[g.lse_base(b, h) + blk0 + myrow] =
        l_run > 0.f ? (msc + __builtin_amdgcn_logf(l_run)) * 0.69314718055994531f : -INFINITY;
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
  const int nw = g.q_block % 256 == 0 ? 8 : g.q_block % 128 == 0 ? 4 : g.q_block % 64 == 0 ? 2 : 1;
  const long long nwg = (long long)g.B * g.Hq * g.Qb * (g.q_block / (32 * nw));
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
