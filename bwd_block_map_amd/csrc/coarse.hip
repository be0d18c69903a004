// Video-tile pooling, pooled-score top-k selection and the compression branch.
//
// Semantics: FastVideo test_vsa256_backward.py (the VSA entry points select
// `topk` KV tiles per Q tile and compose the sparse output with a gated
// compression output; q_var only changes the compression divisor). The
// reading implemented here: pooled tiles are means over valid slots, the
// coarse score is C = scale <Qc_i, Kc_j> over non-empty KV tiles, top-k keeps
// the largest scores (ties to the lower tile), the compression output is
// O_c = softmax_j(C) V_c, and its gradient returns to the valid slots
// divided by the tile's valid count.
//
// gfx950 design: these steps are small (tens of GFLOP at the largest video
// shape) and run on fp32 VALU. Pooling is one work-group per tile with
// coalesced 16-byte loads and an LDS reduction. The coarse kernels keep a
// block of CR score rows in LDS, stream the pooled K/V tiles once per block,
// select top-k per row with a 4-pass 8-bit radix select (per-wave LDS
// histograms, ties resolved by ascending tile index with ballots) and write
// the map bytes directly.
#include "kernels.hpp"

namespace vsa {

namespace {

template <class ET>
__global__ __launch_bounds__(256) void pool_kernel(const Geom g, const uint16_t* __restrict__ x,
                                                   int is_q, float* __restrict__ out) {
  using E = Elem<ET>;
  __shared__ float red[16][HD];
  const int heads = is_q ? g.Hq : g.Hkv, nb = is_q ? g.Qb : g.KVb;
  int id = blockIdx.x;
  const int blk = id % nb;
  id /= nb;
  const int h = id % heads, b = id / heads;
  const int n = is_q ? g.q_val(b, blk) : g.kv_val(b, blk);
  const long long base = (is_q ? g.q_base(b, h) : g.kv_base(b, h)) +
                         (long long)blk * (is_q ? g.q_block : g.kv_block) * (is_q ? g.q_rs() : g.kv_rs());
  const long long rs = is_q ? g.q_rs() : g.kv_rs();
  const int tid = threadIdx.x, slot = tid >> 4, dg = tid & 15;
  float acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.f;
  for (int r = slot; r < n; r += 16) {
    const uint4 v = ldg16(x + base + (long long)r * rs + 8 * dg);
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&v);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[2 * u] += E::lo(w[u]);
      acc[2 * u + 1] += E::hi(w[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) red[slot][8 * dg + u] = acc[u];
  __syncthreads();
  if (tid < HD) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += red[r][tid];
    const long long o = is_q ? g.pq(b, h, blk) : g.pk(b, h, blk);
    out[o + tid] = n > 0 ? s / (float)n : 0.f;
  }
}

// order-preserving map of fp32 to uint32 (-0 folded onto +0)
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Coarse scores for CR Q tiles, then (optionally) top-k -> map bytes and the
// coarse attention O_c / lse_c. Dynamic LDS: sc[CR][KVb], qcs[CR][HD],
// hist[4][256] and a staging tile of CT pooled K (transposed) or V rows. The
// pooled K and V rows are streamed through the tile with coalesced loads; every
// score and every O_c element keeps its sequential accumulation order over d
// (scores) and over the KV tiles (O_c).
constexpr int CT = 64;               // pooled rows per staging tile
constexpr int CT_LD = CT + 1;        // padded row of the transposed K tile
constexpr int TILE_FLOATS = HD * CT_LD;
constexpr int TILE_LOADS = CT * HD / 4 / 256;  // 16-byte loads per thread for one tile
// CR is a template argument: with a run-time row count every "r < CR" test
// becomes a branch around one FMA and serialises the LDS reads behind it.
template <int CR>
__global__ __launch_bounds__(256) void coarse_fwd_kernel(const CoarseArgs a, int want_topk, int want_gate) {
  extern __shared__ float dsm[];
  const Geom& g = a.g;
  const int KVb = g.KVb;
  float* sc = dsm;
  float* qcs = sc + CR * KVb;
  int* hist = reinterpret_cast<int*>(qcs + CR * HD);
  float* tile = reinterpret_cast<float*>(hist + 4 * 256);
  const int nrb = (g.Qb + CR - 1) / CR;
  int id = blockIdx.x;
  const int rb = id % nrb;
  id /= nrb;
  const int h = id % g.Hq, b = id / g.Hq;
  const int hk = h / g.group;
  const int i0 = rb * CR, nr = min(CR, g.Qb - i0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  for (int t = tid; t < CR * HD; t += 256) {
    const int r = t / HD, d = t % HD;
    qcs[t] = r < nr ? a.qc[g.pq(b, h, i0 + r) + d] : 0.f;
  }
  __syncthreads();
  // scores, CT KV tiles at a time: the tiles' pooled K rows are staged
  // transposed (tile[d][j]); thread (wave w, lane j) forms rows w, w+4, .. of
  // column j, accumulating over d in order
  for (int j0 = 0; j0 < KVb; j0 += CT) {
    __syncthreads();  // the previous tile is consumed
    float4 kv[TILE_LOADS];  // all loads of the tile in flight at once
#pragma unroll
    for (int k = 0; k < TILE_LOADS; ++k) {
      const int t = tid + 256 * k, jj = t / (HD / 4), d4 = t % (HD / 4), j = min(j0 + jj, KVb - 1);
      kv[k] = reinterpret_cast<const float4*>(a.kc + g.pk(b, hk, j))[d4];
    }
#pragma unroll
    for (int k = 0; k < TILE_LOADS; ++k) {
      const int t = tid + 256 * k, jj = t / (HD / 4), d4 = t % (HD / 4);
      tile[(4 * d4 + 0) * CT_LD + jj] = kv[k].x;
      tile[(4 * d4 + 1) * CT_LD + jj] = kv[k].y;
      tile[(4 * d4 + 2) * CT_LD + jj] = kv[k].z;
      tile[(4 * d4 + 3) * CT_LD + jj] = kv[k].w;
    }
    __syncthreads();
    // rows wave + 4u, u < RU (all of them exist when CR is a multiple of 4)
    constexpr int RU = (CR + 3) / 4;
    const int j = j0 + lane;
    float acc[RU];
#pragma unroll
    for (int u = 0; u < RU; ++u) acc[u] = 0.f;
    if (CR % 4 == 0 || wave < CR) {
#pragma unroll 8
      for (int d = 0; d < HD; ++d) {
        const float kv = tile[d * CT_LD + lane];
#pragma unroll
        for (int u = 0; u < RU; ++u) acc[u] = __builtin_fmaf(qcs[(wave + 4 * u) * HD + d], kv, acc[u]);
      }
      if (j < KVb) {
        const bool valid = g.kv_val(b, j) > 0;
#pragma unroll
        for (int u = 0; u < RU; ++u) sc[(wave + 4 * u) * KVb + j] = valid ? g.scale * acc[u] : -INFINITY;
      }
    }
  }
  __syncthreads();

  if (want_topk) {
    int* hw = hist + wave * 256;
    for (int r = wave; r < nr; r += 4) {
      const float* row = sc + r * KVb;
      int nv = 0;
      for (int j0 = 0; j0 < KVb; j0 += 64) {
        const int j = j0 + lane;
        nv += __popcll(__ballot(j < KVb && row[j] != -INFINITY));
      }
      int kk = min(a.topk, nv);
      uint32_t prefix = 0, pmask = 0;
      if (kk > 0) {
        for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
          for (int u = 0; u < 4; ++u) hw[lane * 4 + u] = 0;
          __builtin_amdgcn_wave_barrier();
          for (int j = lane; j < KVb; j += 64) {
            const float f = row[j];
            if (f == -INFINITY) continue;
            const uint32_t u = fkey(f);
            if ((u & pmask) == prefix) atomicAdd(&hw[(u >> shift) & 255u], 1);
          }
          __builtin_amdgcn_wave_barrier();
          // lane L owns bins 255-4L .. 252-4L (descending digit order)
          int cnt[4], tot = 0;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            cnt[u] = hw[255 - 4 * lane - u];
            tot += cnt[u];
          }
          int incl = tot;  // inclusive prefix over lanes
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
          }
          const unsigned long long hit = __ballot(incl >= kk);
          const int L = __ffsll((long long)hit) - 1;
          int above = __shfl(incl - tot, L, 64);  // elements in bins above lane L's
          int digit = 0;
          if (lane == L) {
            int acc = above;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              if (acc + cnt[u] >= kk) {
                digit = 255 - 4 * lane - u;
                above = acc;
                break;
              }
              acc += cnt[u];
            }
          }
          digit = __shfl(digit, L, 64);
          above = __shfl(above, L, 64);
          kk -= above;
          prefix |= (uint32_t)digit << shift;
          pmask |= 0xffu << shift;
          __builtin_amdgcn_wave_barrier();
        }
      }
      // select: keys above the threshold, plus the first kk keys equal to it
      uint8_t* mrow = a.map + (((long long)b * g.Hq + h) * g.Qb + i0 + r) * KVb;
      int taken_eq = 0;
      const unsigned long long below = (1ull << lane) - 1ull;
      for (int j0 = 0; j0 < KVb; j0 += 64) {
        const int j = j0 + lane;
        const float f = j < KVb ? row[j] : -INFINITY;
        const bool valid = f != -INFINITY && a.topk > 0 && nv > 0;
        const uint32_t u = valid ? fkey(f) : 0u;
        const bool eq = valid && u == prefix;
        const unsigned long long be = __ballot(eq);
        const int rank = taken_eq + __popcll(be & below);
        const bool sel = valid && (u > prefix || (eq && rank < kk));
        if (j < KVb) mrow[j] = sel ? 1 : 0;
        taken_eq += __popcll(be);
      }
    }
  }

  if (want_gate) {
    __syncthreads();
    // row softmax in place, lse_c
    for (int r = wave; r < nr; r += 4) {
      float* row = sc + r * KVb;
      float m = -INFINITY;
      for (int j = lane; j < KVb; j += 64) m = fmaxf(m, row[j]);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
      float l = 0.f;
      if (m != -INFINITY)
        for (int j = lane; j < KVb; j += 64) l += __expf(row[j] - m);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off, 64);
      const float inv = l > 0.f ? 1.f / l : 0.f;
      for (int j = lane; j < KVb; j += 64) row[j] = m == -INFINITY ? 0.f : __expf(row[j] - m) * inv;
      if (lane == 0) a.lse_c[((long long)b * g.Hq + h) * g.Qb + i0 + r] = l > 0.f ? m + __logf(l) : -INFINITY;
    }
    __syncthreads();
    // O_c[r][d] = sum_j P[r][j] V_c[j][d], CT pooled V rows at a time (tile[j][d])
    const int d = tid & (HD - 1), half = tid >> 7;
    float acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = 0.f;
    for (int j0 = 0; j0 < KVb; j0 += CT) {
      __syncthreads();  // the previous tile is consumed
      float4 vv[TILE_LOADS];
#pragma unroll
      for (int k = 0; k < TILE_LOADS; ++k) {
        const int t = tid + 256 * k, jj = t / (HD / 4), d4 = t % (HD / 4), j = min(j0 + jj, KVb - 1);
        vv[k] = reinterpret_cast<const float4*>(a.vc + g.pk(b, hk, j))[d4];
      }
#pragma unroll
      for (int k = 0; k < TILE_LOADS; ++k) reinterpret_cast<float4*>(tile)[tid + 256 * k] = vv[k];
      __syncthreads();
      const int nj = min(CT, KVb - j0);
      if (CR == 16 || half * 8 < CR) {
#pragma unroll 4
        for (int jj = 0; jj < nj; ++jj) {
          const float v = tile[jj * HD + d];
#pragma unroll
          for (int u = 0; u < (CR < 8 ? CR : 8); ++u)
            acc[u] = __builtin_fmaf(sc[(half * 8 + u) * KVb + j0 + jj], v, acc[u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = half * 8 + u;
      if (r < nr) a.oc[g.pq(b, h, i0 + r) + d] = acc[u];
    }
  }
}

// Coarse backward, row form: P_c, dS_c for CR2 rows (kept in workspace for the
// column pass) and dQ_c = scale dS_c K_c. For dQ_c the pooled K rows stream
// through an LDS tile with all loads of a tile in flight.
// 8 rows per work-group (CR2): with 4, two work-groups share a CU at 1440 KV
// tiles, but twice as many row blocks then stream every pooled K/V row (6 %
// slower). With more KV tiles than 8 rows of P_c and dS_c fit in LDS, the
// launch takes 4, 2 or 1 rows per work-group.
constexpr int CT2 = 32;                  // pooled K rows per staging tile
constexpr int TILE2_FLOATS = CT2 * HD;
template <int CR2>
__global__ __launch_bounds__(256) void coarse_bwd_rows_kernel(const CoarseArgs a) {
  extern __shared__ float dsm[];
  const Geom& g = a.g;
  const int KVb = g.KVb;
  float* P = dsm;                 // [CR2][KVb]
  float* dS = P + CR2 * KVb;      // [CR2][KVb]
  float* qcs = dS + CR2 * KVb;    // [CR2][HD]
  float* dos = qcs + CR2 * HD;    // [CR2][HD]
  float* lsc = dos + CR2 * HD;    // [CR2]
  float* tile = lsc + CR2;        // [CT2][HD]
  const int nrb = (g.Qb + CR2 - 1) / CR2;
  int id = blockIdx.x;
  const int rb = id % nrb;
  id /= nrb;
  const int h = id % g.Hq, b = id / g.Hq;
  const int hk = h / g.group;
  const int i0 = rb * CR2, nr = min(CR2, g.Qb - i0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int t = tid; t < CR2 * HD; t += 256) {
    const int r = t / HD, d = t % HD;
    qcs[t] = r < nr ? a.qc[g.pq(b, h, i0 + r) + d] : 0.f;
    dos[t] = r < nr ? a.doc[g.pq(b, h, i0 + r) + d] : 0.f;
  }
  if (tid < CR2) lsc[tid] = tid < nr ? a.lse_c[((long long)b * g.Hq + h) * g.Qb + i0 + tid] : -INFINITY;
  __syncthreads();
  for (int j = tid; j < KVb; j += 256) {
    const bool valid = g.kv_val(b, j) > 0;
    float cs[CR2], dp[CR2];
#pragma unroll
    for (int r = 0; r < CR2; ++r) cs[r] = dp[r] = 0.f;
    if (valid) {
      const float4* kp = reinterpret_cast<const float4*>(a.kc + g.pk(b, hk, j));
      const float4* vp = reinterpret_cast<const float4*>(a.vc + g.pk(b, hk, j));
      // unrolled so that the loads of eight steps are in flight together
      // (one step at a time waits out an L2 round trip per 4 elements)
#pragma unroll 8
      for (int d4 = 0; d4 < HD / 4; ++d4) {
        const float4 kv = kp[d4], vv = vp[d4];
#pragma unroll
        for (int r = 0; r < CR2; ++r) {
          const float4 qv = *reinterpret_cast<const float4*>(qcs + r * HD + 4 * d4);
          const float4 ov = *reinterpret_cast<const float4*>(dos + r * HD + 4 * d4);
          cs[r] += qv.x * kv.x + qv.y * kv.y + qv.z * kv.z + qv.w * kv.w;
          dp[r] += ov.x * vv.x + ov.y * vv.y + ov.z * vv.z + ov.w * vv.w;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < CR2; ++r) {
      const float p = (valid && lsc[r] != -INFINITY) ? __expf(g.scale * cs[r] - lsc[r]) : 0.f;
      P[r * KVb + j] = p;
      dS[r * KVb + j] = p == 0.f ? 0.f : dp[r];
    }
  }
  __syncthreads();
  for (int rr = wave; rr < nr; rr += 4) {
    float s = 0.f;
    for (int j = lane; j < KVb; j += 64) s += P[rr * KVb + j] * dS[rr * KVb + j];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    const long long ro = (((long long)b * g.Hq + h) * g.Qb + i0 + rr) * KVb;
    for (int j = lane; j < KVb; j += 64) {
      const float p = P[rr * KVb + j];
      const float ds = p * (dS[rr * KVb + j] - s);
      dS[rr * KVb + j] = ds;
      a.dss[ro + j] = ds;
      a.ps[ro + j] = p;
    }
  }
  // dQ_c[r][d] = scale sum_j dS_c[r][j] K_c[j][d], CT2 pooled K rows at a time (tile[j][d])
  constexpr int RH = CR2 > 1 ? CR2 / 2 : 1;  // rows per half of the work-group
  const int d = tid & (HD - 1), half = tid >> 7;
  const bool rows_here = half * RH < CR2;  // one row: the second half idles
  float acc[RH];
#pragma unroll
  for (int u = 0; u < RH; ++u) acc[u] = 0.f;
  constexpr int KLOADS = CT2 * HD / 4 / 256;
  for (int j0 = 0; j0 < KVb; j0 += CT2) {
    __syncthreads();  // dS is final / the previous tile is consumed
    float4 x[KLOADS];
#pragma unroll
    for (int k = 0; k < KLOADS; ++k) {
      const int t = tid + 256 * k, j = min(j0 + t / (HD / 4), KVb - 1), d4 = t % (HD / 4);
      x[k] = reinterpret_cast<const float4*>(a.kc + g.pk(b, hk, j))[d4];
    }
#pragma unroll
    for (int k = 0; k < KLOADS; ++k) reinterpret_cast<float4*>(tile)[tid + 256 * k] = x[k];
    __syncthreads();
    const int nj = min(CT2, KVb - j0);
    if (rows_here) {
#pragma unroll 4
      for (int jt = 0; jt < nj; ++jt) {
        const float kv = tile[jt * HD + d];
#pragma unroll
        for (int u = 0; u < RH; ++u) acc[u] = __builtin_fmaf(dS[(half * RH + u) * KVb + j0 + jt], kv, acc[u]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < RH; ++u) {
    const int rr = half * RH + u;
    if (rows_here && rr < nr) a.dqc[g.pq(b, h, i0 + rr) + d] = g.scale * acc[u];
  }
}

// Coarse backward, column form: dK_c = scale sum dS_c^T Q_c, dV_c = sum P_c^T dO_c
// over the Q heads of the group (16 KV tiles per work-group, thread = (d, 8
// tiles)). The Q tiles' pooled rows and this block's dS_c / P_c columns are
// staged in LDS CI tiles at a time, all loads of a stage in flight.
constexpr int CC = 16;
constexpr int CI = 32;
__global__ __launch_bounds__(256) void coarse_bwd_cols_kernel(const CoarseArgs a) {
  __shared__ float4 qo[2][CI][HD / 4];  // q_c | dO_c rows
  __shared__ float pd[2][CI][CC];       // dS_c | P_c of this block's columns
  const Geom& g = a.g;
  const int KVb = g.KVb;
  const int ncb = (KVb + CC - 1) / CC;
  int id = blockIdx.x;
  const int cb = id % ncb;
  id /= ncb;
  const int hk = id % g.Hkv, b = id / g.Hkv;
  const int tid = threadIdx.x, d = tid & (HD - 1), half = tid >> 7;
  const int j0 = cb * CC + half * 8;
  float dk[8], dv[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) dk[u] = dv[u] = 0.f;
  constexpr int QLOADS = 2 * CI * HD / 4 / 256, PLOADS = 2 * CI * CC / 256;
  for (int hh = 0; hh < g.group; ++hh) {
    const int h = hk * g.group + hh;
    for (int i0 = 0; i0 < g.Qb; i0 += CI) {
      float4 x[QLOADS];
      float y[PLOADS];
#pragma unroll
      for (int k = 0; k < QLOADS; ++k) {
        const int t = tid + 256 * k, arr = t / (CI * HD / 4), rem = t % (CI * HD / 4);
        const int i = min(i0 + rem / (HD / 4), g.Qb - 1), d4 = rem % (HD / 4);
        x[k] = reinterpret_cast<const float4*>((arr ? a.doc : a.qc) + g.pq(b, h, i))[d4];
      }
#pragma unroll
      for (int k = 0; k < PLOADS; ++k) {
        const int t = tid + 256 * k, arr = t / (CI * CC), rem = t % (CI * CC);
        const int i = min(i0 + rem / CC, g.Qb - 1), j = cb * CC + rem % CC;
        const long long ro = (((long long)b * g.Hq + h) * g.Qb + i) * KVb;
        y[k] = j < KVb ? (arr ? a.ps : a.dss)[ro + j] : 0.f;
      }
      __syncthreads();  // the previous stage is consumed
#pragma unroll
      for (int k = 0; k < QLOADS; ++k) (&qo[0][0][0])[tid + 256 * k] = x[k];
#pragma unroll
      for (int k = 0; k < PLOADS; ++k) (&pd[0][0][0])[tid + 256 * k] = y[k];
      __syncthreads();
      const int ni = min(CI, g.Qb - i0);
      const float* qrow = reinterpret_cast<const float*>(&qo[0][0][0]);
      const float* orow = reinterpret_cast<const float*>(&qo[1][0][0]);
      for (int ii = 0; ii < ni; ++ii) {
        const float q = qrow[ii * HD + d], o = orow[ii * HD + d];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          dk[u] = __builtin_fmaf(pd[0][ii][half * 8 + u], q, dk[u]);
          dv[u] = __builtin_fmaf(pd[1][ii][half * 8 + u], o, dv[u]);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (j0 + u < KVb) {
      a.dkc[g.pk(b, hk, j0 + u) + d] = g.scale * dk[u];
      a.dvc[g.pk(b, hk, j0 + u) + d] = dv[u];
    }
}

__global__ void zero_kernel(uint8_t* p, size_t n) {
  const size_t n16 = n / 16;
  uint4* p16 = reinterpret_cast<uint4*>(p);
  for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < n16;
       t += (size_t)gridDim.x * blockDim.x)
    p16[t] = make_uint4(0, 0, 0, 0);
  const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n - n16 * 16) p[n16 * 16 + t] = 0;
}

}  // namespace

namespace {
size_t rows_lds(int cr2, int KVb) {
  return ((size_t)2 * cr2 * KVb + 2 * cr2 * HD + cr2 + TILE2_FLOATS) * 4;
}
// rows per work-group of the coarse backward: 8 when they fit, else fewer
int coarse_bwd_rows(int KVb) {
  for (int cr = 8; cr > 1; cr >>= 1)
    if (rows_lds(cr, KVb) <= 160 * 1024) return cr;
  return 1;
}
}  // namespace

// LDS of the coarse backward's row pass at its launch shape (above 160 KiB:
// too many KV tiles for these kernels)
size_t coarse_bwd_lds(int KVb) { return rows_lds(coarse_bwd_rows(KVb), KVb); }

int coarse_rows_per_block(int KVb) {
  // scores [CR][KVb] + qc [CR][HD] + 4 histograms + the staging tile. Prefer
  // the largest CR with which two work-groups share a CU's 160 KiB (a single
  // four-wave work-group leaves each SIMD one wave to hide LDS latency with),
  // else the largest that fits at all.
  auto need = [&](int cr) { return ((long long)cr * (KVb + HD) + 4 * 256 + TILE_FLOATS) * 4; };
  for (int cr = 16; cr >= 1; cr >>= 1)
    if (need(cr) <= 80 * 1024) return cr;
  int cr = 16;
  while (cr > 1 && need(cr) > 160 * 1024) cr >>= 1;
  return need(cr) <= 160 * 1024 ? cr : 0;  // 0: KVb too large for these kernels
}

hipError_t launch_pool(const Geom& g, int dtype, const void* q, const void* k, const void* v,
                       float* qc, float* kc, float* vc, hipStream_t st) {
  const unsigned nq = (unsigned)((long long)g.B * g.Hq * g.Qb);
  const unsigned nk = (unsigned)((long long)g.B * g.Hkv * g.KVb);
  auto go = [&](auto tag) {
    using ET = decltype(tag);
    if (nq) pool_kernel<ET><<<nq, 256, 0, st>>>(g, (const uint16_t*)q, 1, qc);
    if (nk) {
      pool_kernel<ET><<<nk, 256, 0, st>>>(g, (const uint16_t*)k, 0, kc);
      pool_kernel<ET><<<nk, 256, 0, st>>>(g, (const uint16_t*)v, 0, vc);
    }
  };
  if (dtype == VSA_BF16) go(bf16_tag{});
  else go(f16_tag{});
  return hipGetLastError();
}

hipError_t launch_coarse_fwd(const CoarseArgs& a, bool want_topk, bool want_gate, hipStream_t st) {
  const Geom& g = a.g;
  const int cr = coarse_rows_per_block(g.KVb);
  const long long n = (long long)g.B * g.Hq * ((g.Qb + cr - 1) / cr);
  if (n == 0) return hipSuccess;
  const size_t lds = ((size_t)cr * (g.KVb + HD) + 4 * 256 + TILE_FLOATS) * 4;
  const int tk = want_topk ? 1 : 0, gt = want_gate ? 1 : 0;
  switch (cr) {
    case 16: coarse_fwd_kernel<16><<<(unsigned)n, 256, lds, st>>>(a, tk, gt); break;
    case 8: coarse_fwd_kernel<8><<<(unsigned)n, 256, lds, st>>>(a, tk, gt); break;
    case 4: coarse_fwd_kernel<4><<<(unsigned)n, 256, lds, st>>>(a, tk, gt); break;
    case 2: coarse_fwd_kernel<2><<<(unsigned)n, 256, lds, st>>>(a, tk, gt); break;
    default: coarse_fwd_kernel<1><<<(unsigned)n, 256, lds, st>>>(a, tk, gt); break;
  }
  return hipGetLastError();
}

hipError_t launch_coarse_bwd(const CoarseArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int cr2 = coarse_bwd_rows(g.KVb);
  const long long nr = (long long)g.B * g.Hq * ((g.Qb + cr2 - 1) / cr2);
  const long long nc = (long long)g.B * g.Hkv * ((g.KVb + CC - 1) / CC);
  if (nr == 0 || nc == 0) return hipSuccess;
  const size_t lds = coarse_bwd_lds(g.KVb);
  if (cr2 == 8) coarse_bwd_rows_kernel<8><<<(unsigned)nr, 256, lds, st>>>(a);
  else if (cr2 == 4) coarse_bwd_rows_kernel<4><<<(unsigned)nr, 256, lds, st>>>(a);
  else if (cr2 == 2) coarse_bwd_rows_kernel<2><<<(unsigned)nr, 256, lds, st>>>(a);
  else coarse_bwd_rows_kernel<1><<<(unsigned)nr, 256, lds, st>>>(a);
  coarse_bwd_cols_kernel<<<(unsigned)nc, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  unsigned grid = (unsigned)std::min<size_t>((n16 + 255) / 256 + 1, 65536);
  zero_kernel<<<grid, 256, 0, st>>>((uint8_t*)p, bytes);
  return hipGetLastError();
}

}  // namespace vsa
