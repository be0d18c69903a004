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
// gfx950 design: pooling is one work-group per tile with coalesced 16-byte
// loads and an LDS reduction. The coarse contractions (scores, O_c, and in the
// backward C, dP_c, dQ_c, dK_c, dV_c) run on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32) with both operands loaded straight into registers,
// 16 bytes per lane. The row kernels keep up to 16 rows of scores in LDS,
// select top-k per row with a 4-pass 8-bit radix select (per-wave LDS
// histograms, ties resolved by ascending tile index with ballots) and write the
// map bytes directly.
#include "kernels.hpp"

namespace vsa {

namespace {

// One launch pools q, k and v: tiles [0, nq) are the Q tiles, the next nk the
// K tiles and the last nk the V tiles (tile wg0 + blockIdx.x).
template <class ET>
__global__ __launch_bounds__(256) void pool_kernel(const Geom g, const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v, float* __restrict__ qc,
                                                   float* __restrict__ kc, float* __restrict__ vc,
                                                   long long wg0) {
  using E = Elem<ET>;
  __shared__ float red[16][HD];
  const long long nq = (long long)g.B * g.Hq * g.Qb, nk = (long long)g.B * g.Hkv * g.KVb;
  const long long t = wg0 + blockIdx.x;
  const bool is_q = t < nq;
  const uint16_t* x = is_q ? q : t < nq + nk ? k : v;
  float* out = is_q ? qc : t < nq + nk ? kc : vc;
  int id = (int)(is_q ? t : (t - nq) % nk);
  const int heads = is_q ? g.Hq : g.Hkv, nb = is_q ? g.Qb : g.KVb;
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
    const uint4 xv = ldg16(x + base + (long long)r * rs + 8 * dg);
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&xv);
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

// The contractions of the coarse branch run on the fp32 matrix cores:
// v_mfma_f32_16x16x4_f32 computes D[16][16] += A[16][4] B[4][16]; lane l
// supplies A[l % 16][l / 16] and B[l / 16][l % 16] and holds
// D[4 (l / 16) + v][l % 16] for v < 4.
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
__device__ __forceinline__ f32x4_t mfma16(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr int NWC = 8;        // waves of the row kernels (two per SIMD)
constexpr int MR = 16;        // rows of one MFMA block
constexpr int HD16 = HD / 16;

// Dot products of pooled rows: lane (r = l % 16, kk = l / 16) holds d = 16 m +
// 4 kk + {0..3} (m < HD / 16) of one row. Any assignment of the d to the MFMA
// steps sums the same products; only the rounding order depends on it.
__device__ __forceinline__ void load_row(float4 (&x)[HD16], const float* row, int kk) {
#pragma unroll
  for (int m = 0; m < HD16; ++m) x[m] = *reinterpret_cast<const float4*>(row + 16 * m + 4 * kk);
}
__device__ __forceinline__ void zero_row(float4 (&x)[HD16]) {
#pragma unroll
  for (int m = 0; m < HD16; ++m) x[m] = make_float4(0.f, 0.f, 0.f, 0.f);
}
// D[i][j] = <X_i, Y_j> for the 16 rows X held by lanes i = l % 16 and the 16
// rows Y held by lanes j = l % 16
__device__ __forceinline__ f32x4_t rowdot16(const float4 (&x)[HD16], const float4 (&y)[HD16]) {
  f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < HD16; ++m) {
    c = mfma16(x[m].x, y[m].x, c);
    c = mfma16(x[m].y, y[m].y, c);
    c = mfma16(x[m].z, y[m].z, c);
    c = mfma16(x[m].w, y[m].w, c);
  }
  return c;
}

// Score rows in LDS: row stride a multiple of 64 floats plus 4, so the MFMA
// operand reads (16 rows x 4 consecutive tiles) and the result writes (4 rows x
// 16 consecutive tiles) touch 64 distinct banks.
__host__ __device__ __forceinline__ int score_ld(int KVb) { return ((KVb + 63) & ~63) + 4; }
// the first LDS area also takes the 4 x 16 x HD partial sums of a row-times-
// matrix product once its rows are consumed
__host__ __device__ __forceinline__ long long row_area(int cr, int KVb) {
  const long long n = (long long)cr * score_ld(KVb);
  return n > 4LL * MR * HD ? n : 4LL * MR * HD;
}

// Out[r][d] = sum_j W[r][j] M[j][d] for the rows r < nr of a 16-row block, W in
// LDS (stride ld), M pooled rows of HD floats (the coarse forward's O_c). Wave w: d half (w & 1) and every
// fourth group of four j (w >> 1); lane (r, kk) feeds W[r][j] as A and M[j][64
// half + 4 r + c] as B of the MFMA whose accumulator c holds d = 64 half + 4 n +
// c. The four partial sums meet in `red` (aliasing W: callers sync first), and
// out(row, d, value) stores the sums in fixed order.
template <class RowPtr, class Out>
__device__ __forceinline__ void rows_times_pooled(const float* W, int ld, int nr, int KVb,
                                                  RowPtr mrow, float* red, Out out) {
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, kk = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave & 1, qj = wave >> 1;
  f32x4_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nst = (KVb + 3) / 4;
  const bool row_ok = r < nr;
  // RB steps per batch, the next batch's loads issued before this batch's
  // MFMAs (steps past the end add W = 0 times a clamped row)
  constexpr int RB = 8;
  float4 mb[RB], mn[RB];
  auto load = [&](int t0, float4 (&m)[RB]) {
#pragma unroll
    for (int e = 0; e < RB; ++e) {
      const int j = min(4 * (t0 + 4 * e) + kk, KVb - 1);
      m[e] = *reinterpret_cast<const float4*>(mrow(j) + 64 * half + 4 * r);
    }
  };
  auto step = [&](int t0, const float4 (&m)[RB]) {
#pragma unroll
    for (int e = 0; e < RB; ++e) {
      const int j = 4 * (t0 + 4 * e) + kk;
      const float w = (row_ok && j < KVb) ? W[r * ld + j] : 0.f;
      acc[0] = mfma16(w, m[e].x, acc[0]);
      acc[1] = mfma16(w, m[e].y, acc[1]);
      acc[2] = mfma16(w, m[e].z, acc[2]);
      acc[3] = mfma16(w, m[e].w, acc[3]);
    }
  };
  if (qj < nst) load(qj, mb);
  for (int t0 = qj; t0 < nst; t0 += 8 * RB) {
    const int t1 = t0 + 4 * RB, t2 = t0 + 8 * RB;
    if (t1 < nst) load(t1, mn);
    step(t0, mb);
    if (t2 < nst) load(t2, mb);
    if (t1 < nst) step(t1, mn);
  }
  __syncthreads();  // W consumed
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[(qj * MR + 4 * kk + v) * HD + 64 * half + 4 * r + c] = acc[c][v];
  __syncthreads();
  for (int t = tid; t < nr * HD; t += NWC * 64) {
    const int row = t / HD, d = t % HD;
    const float* x = red + row * HD + d;
    out(row, d, ((x[0] + x[MR * HD]) + x[2 * MR * HD]) + x[3 * MR * HD]);
  }
}

// Coarse scores for CR Q tiles, then (optionally) top-k -> map bytes and the
// coarse attention O_c / lse_c. Dynamic LDS: sc[CR][score_ld] (at least the
// 4 x 16 x HD partial sums of O_c) and hist[NWC][256]. Each wave forms 16 x 16
// score blocks on the matrix cores with its Q rows and the block's pooled K rows
// in registers (loaded straight from global memory, 16 bytes per lane); top-k is
// a 4-pass 8-bit radix select per row; O_c = P_c V_c reads P_c from LDS and the
// pooled V rows from global memory.
// CR is a template argument so that the per-row stores unroll.
template <int CR>
__global__ __launch_bounds__(NWC * 64) void coarse_fwd_kernel(const CoarseArgs a, int want_topk, int want_gate) {
  extern __shared__ float dsm[];
  const Geom& g = a.g;
  const int KVb = g.KVb, LD = score_ld(KVb);
  float* sc = dsm;
  int* hist = reinterpret_cast<int*>(dsm + row_area(CR, KVb));
  const int nrb = (g.Qb + CR - 1) / CR;
  int id = blockIdx.x;
  const int rb = id % nrb;
  id /= nrb;
  const int h = id % g.Hq, b = id / g.Hq;
  const int hk = h / g.group;
  const int i0 = rb * CR, nr = min(CR, g.Qb - i0);
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, kk = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // scores: wave w takes the 16-tile column blocks w, w + NWC, ...
  float4 qx[HD16];
  if (r < nr) load_row(qx, a.qc + g.pq(b, h, i0 + r), kk);
  else zero_row(qx);
  // the next block's K rows are loaded while this block's MFMAs run
  const int nblk = (KVb + 15) / 16;
  auto kload = [&](int cb, float4 (&ky)[HD16]) {
    load_row(ky, a.kc + g.pk(b, hk, min(cb * 16 + r, KVb - 1)), kk);
  };
  auto scores = [&](int cb, const float4 (&ky)[HD16]) {
    const int j = cb * 16 + r;
    const f32x4_t c = rowdot16(qx, ky);
    if (j < KVb) {
      const bool valid = g.kv_val(b, j) > 0;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (4 * kk + v < CR) sc[(4 * kk + v) * LD + j] = valid ? g.scale * c[v] : -INFINITY;
    }
  };
  float4 ka[HD16], kb[HD16];
  if (wave < nblk) kload(wave, ka);
  for (int cb = wave; cb < nblk; cb += 2 * NWC) {
    const int c1 = cb + NWC, c2 = cb + 2 * NWC;
    if (c1 < nblk) kload(c1, kb);
    scores(cb, ka);
    if (c2 < nblk) kload(c2, ka);
    if (c1 < nblk) scores(c1, kb);
  }
  __syncthreads();

  if (want_topk) {
    int* hw = hist + wave * 256;
    for (int rr = wave; rr < nr; rr += NWC) {
      const float* row = sc + rr * LD;
      int nv = 0;
      for (int j0 = 0; j0 < KVb; j0 += 64) {
        const int j = j0 + lane;
        nv += __popcll(__ballot(j < KVb && row[j] != -INFINITY));
      }
      int kth = min(a.topk, nv);
      uint32_t prefix = 0, pmask = 0;
      if (kth > 0) {
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
          const unsigned long long hit = __ballot(incl >= kth);
          const int L = __ffsll((long long)hit) - 1;
          int above = __shfl(incl - tot, L, 64);  // elements in bins above lane L's
          int digit = 0;
          if (lane == L) {
            int acc = above;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              if (acc + cnt[u] >= kth) {
                digit = 255 - 4 * lane - u;
                above = acc;
                break;
              }
              acc += cnt[u];
            }
          }
          digit = __shfl(digit, L, 64);
          above = __shfl(above, L, 64);
          kth -= above;
          prefix |= (uint32_t)digit << shift;
          pmask |= 0xffu << shift;
          __builtin_amdgcn_wave_barrier();
        }
      }
      // select: keys above the threshold, plus the first kth keys equal to it
      uint8_t* mrow = a.map + (((long long)b * g.Hq + h) * g.Qb + i0 + rr) * KVb;
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
        const bool sel = valid && (u > prefix || (eq && rank < kth));
        if (j < KVb) mrow[j] = sel ? 1 : 0;
        taken_eq += __popcll(be);
      }
    }
  }

  if (want_gate) {
    __syncthreads();
    // row softmax in place, lse_c
    for (int rr = wave; rr < nr; rr += NWC) {
      float* row = sc + rr * LD;
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
      if (lane == 0) a.lse_c[((long long)b * g.Hq + h) * g.Qb + i0 + rr] = l > 0.f ? m + __logf(l) : -INFINITY;
    }
    __syncthreads();
    // O_c = P_c V_c
    rows_times_pooled(sc, LD, nr, KVb, [&](int j) { return a.vc + g.pk(b, hk, j); }, sc,
                      [&](int row, int d, float o) { a.oc[g.pq(b, h, i0 + row) + d] = o; });
  }
}

// Coarse backward, row form, 16 Q tiles per work-group. The scores are formed
// transposed on the matrix cores, C^T = K_c Q_c^T and dP^T = V_c dO_c^T, so
// lane (r, kk) ends with row r at tiles j = 16 cb + 4 kk + v (v < 4), exactly
// the A operand of a product over j. In the same sweep it takes P = exp(C -
// lse_c), W = P dP, the row sum s = sum_j W, and accumulates U = W K_c and
// Z = P K_c; dQ_c = scale (U - s Z) = scale dS_c K_c with dS_c = P (dP - s).
// P and W go to the workspace with s per row; the column pass forms dS_c =
// W - s P from them. Dynamic LDS: the q_c and dO_c rows (B operands of the
// scores), then the waves' partial U, Z and s.
constexpr int QLD = HD + 4;  // padded pooled row: conflict-free 16-byte reads
__global__ __launch_bounds__(NWC * 64) void coarse_bwd_rows_kernel(const CoarseArgs a) {
  extern __shared__ float dsm[];
  float* qs = dsm;                       // [MR][QLD]
  float* os = qs + MR * QLD;             // [MR][QLD]
  float* red = dsm;                      // after the sweep: [NWC][2][MR][HD]
  float* ssum = dsm + NWC * 2 * MR * HD; // [NWC][MR]
  const Geom& g = a.g;
  const int KVb = g.KVb;
  const int nrb = (g.Qb + MR - 1) / MR;
  int id = blockIdx.x;
  const int rb = id % nrb;
  id /= nrb;
  const int h = id % g.Hq, b = id / g.Hq;
  const int hk = h / g.group;
  const int i0 = rb * MR, nr = min(MR, g.Qb - i0);
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, kk = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long rowbase = ((long long)b * g.Hq + h) * g.Qb + i0;

  for (int t = tid; t < MR * HD / 4; t += NWC * 64) {
    const int row = t / (HD / 4), d = 4 * (t % (HD / 4));
    const bool ok = row < nr;
    *reinterpret_cast<float4*>(qs + row * QLD + d) =
        ok ? *reinterpret_cast<const float4*>(a.qc + g.pq(b, h, i0 + row) + d) : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(os + row * QLD + d) =
        ok ? *reinterpret_cast<const float4*>(a.doc + g.pq(b, h, i0 + row) + d) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();
  const bool row_ok = r < nr;
  const float lse_r = row_ok ? a.lse_c[rowbase + r] : -INFINITY;
  float* prow = row_ok ? a.ps + (rowbase + r) * KVb : nullptr;   // used only for rows that exist
  float* wrow = row_ok ? a.dss + (rowbase + r) * KVb : nullptr;
  const bool vec_store = (KVb & 3) == 0;

  f32x4_t U[2][4], Z[2][4];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int c = 0; c < 4; ++c) U[h2][c] = Z[h2][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float sacc = 0.f;
  const int nblk = (KVb + 15) / 16;
  auto kvload = [&](int cb, float4 (&ky)[HD16], float4 (&vy)[HD16]) {
    const int jc = min(cb * 16 + r, KVb - 1);
    load_row(ky, a.kc + g.pk(b, hk, jc), kk);
    load_row(vy, a.vc + g.pk(b, hk, jc), kk);
  };
  for (int cb = wave; cb < nblk; cb += NWC) {
    float4 ky[HD16], vy[HD16];
    kvload(cb, ky, vy);
    // this block's K rows as the B operand of U and Z (tile 16 cb + 4 kk + v,
    // d = 64 h2 + 4 r + {0..3}), loaded while the scores run
    float4 kd[4][2];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        kd[v][h2] = *reinterpret_cast<const float4*>(
            a.kc + g.pk(b, hk, min(cb * 16 + 4 * kk + v, KVb - 1)) + 64 * h2 + 4 * r);
    f32x4_t c = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < HD16; ++m) {
      const float4 q = *reinterpret_cast<const float4*>(qs + r * QLD + 16 * m + 4 * kk);
      const float4 o = *reinterpret_cast<const float4*>(os + r * QLD + 16 * m + 4 * kk);
      c = mfma16(ky[m].x, q.x, c);
      c = mfma16(ky[m].y, q.y, c);
      c = mfma16(ky[m].z, q.z, c);
      c = mfma16(ky[m].w, q.w, c);
      dp = mfma16(vy[m].x, o.x, dp);
      dp = mfma16(vy[m].y, o.y, dp);
      dp = mfma16(vy[m].z, o.z, dp);
      dp = mfma16(vy[m].w, o.w, dp);
    }
    const int j0 = cb * 16 + 4 * kk;
    float pv[4], wv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = j0 + v;
      const bool valid = j < KVb && lse_r != -INFINITY && g.kv_val(b, j) > 0;
      const float p = valid ? __expf(g.scale * c[v] - lse_r) : 0.f;
      pv[v] = p;
      wv[v] = p == 0.f ? 0.f : p * dp[v];
      sacc += wv[v];
    }
    if (row_ok) {
      if (vec_store && j0 + 3 < KVb) {
        *reinterpret_cast<float4*>(prow + j0) = make_float4(pv[0], pv[1], pv[2], pv[3]);
        *reinterpret_cast<float4*>(wrow + j0) = make_float4(wv[0], wv[1], wv[2], wv[3]);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (j0 + v < KVb) {
            prow[j0 + v] = pv[v];
            wrow[j0 + v] = wv[v];
          }
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        U[h2][0] = mfma16(wv[v], kd[v][h2].x, U[h2][0]);
        U[h2][1] = mfma16(wv[v], kd[v][h2].y, U[h2][1]);
        U[h2][2] = mfma16(wv[v], kd[v][h2].z, U[h2][2]);
        U[h2][3] = mfma16(wv[v], kd[v][h2].w, U[h2][3]);
        Z[h2][0] = mfma16(pv[v], kd[v][h2].x, Z[h2][0]);
        Z[h2][1] = mfma16(pv[v], kd[v][h2].y, Z[h2][1]);
        Z[h2][2] = mfma16(pv[v], kd[v][h2].z, Z[h2][2]);
        Z[h2][3] = mfma16(pv[v], kd[v][h2].w, Z[h2][3]);
      }
  }
  sacc += __shfl_xor(sacc, 16, 64);
  sacc += __shfl_xor(sacc, 32, 64);
  __syncthreads();  // q_c, dO_c consumed: the area takes the partial sums
  if (kk == 0) ssum[wave * MR + r] = sacc;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int o = (4 * kk + v) * HD + 64 * h2 + 4 * r + c;
        red[(wave * 2 + 0) * MR * HD + o] = U[h2][c][v];
        red[(wave * 2 + 1) * MR * HD + o] = Z[h2][c][v];
      }
  __syncthreads();
  if (tid < nr) {
    float sr = 0.f;
    for (int w = 0; w < NWC; ++w) sr += ssum[w * MR + tid];
    a.csum[rowbase + tid] = sr;
  }
  for (int t = tid; t < nr * HD; t += NWC * 64) {
    const int row = t / HD, d = t % HD;
    float sr = 0.f, u = 0.f, z = 0.f;
    for (int w = 0; w < NWC; ++w) {
      sr += ssum[w * MR + row];
      u += red[(w * 2 + 0) * MR * HD + t];
      z += red[(w * 2 + 1) * MR * HD + t];
    }
    a.dqc[g.pq(b, h, i0 + row) + d] = g.scale * (u - sr * z);
  }
}

// Coarse backward, column form: dK_c = scale sum dS_c^T Q_c and dV_c = sum
// P_c^T dO_c over the Q tiles of every head of the group. A work-group owns 32
// KV tiles (two 16-row MFMA blocks per wave); wave w computes dK_c (w even) or
// dV_c (w odd) for the d half w >> 1, lane (r, kk) feeding dS_c[i][j] = W - s_i
// P (or P_c) as A and Q_c[i][64 half + 4 r + c] (or dO_c) as B, four tiles i
// per step.
constexpr int CCOL = 32;
__global__ __launch_bounds__(256) void coarse_bwd_cols_kernel(const CoarseArgs a) {
  const Geom& g = a.g;
  const int KVb = g.KVb;
  const int ncb = (KVb + CCOL - 1) / CCOL;
  int id = blockIdx.x;
  const int cb = id % ncb;
  id /= ncb;
  const int hk = id % g.Hkv, b = id / g.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, kk = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int is_v = wave & 1, half = wave >> 1;
  const float* A = is_v ? a.ps : a.dss;
  const float* X = is_v ? a.doc : a.qc;
  const int j0 = cb * CCOL;
  f32x4_t acc[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[u][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bool ok0 = j0 + r < KVb, ok1 = j0 + 16 + r < KVb;
  const int nst = (g.Qb + 3) / 4;
  for (int hh = 0; hh < g.group; ++hh) {
    const int h = hk * g.group + hh;
    const long long rowbase = ((long long)b * g.Hq + h) * g.Qb;
#pragma unroll 8
    for (int t = 0; t < nst; ++t) {
      const int i = 4 * t + kk, ic = min(i, g.Qb - 1);
      const float4 x = *reinterpret_cast<const float4*>(X + g.pq(b, h, ic) + 64 * half + 4 * r);
      const float* arow = A + (rowbase + ic) * KVb + j0 + r;
      float a0 = (i < g.Qb && ok0) ? arow[0] : 0.f;
      float a1 = (i < g.Qb && ok1) ? arow[16] : 0.f;
      if (!is_v) {  // dS_c = W - s P
        const float* prow = a.ps + (rowbase + ic) * KVb + j0 + r;
        const float si = a.csum[rowbase + ic];
        a0 = (i < g.Qb && ok0) ? a0 - si * prow[0] : 0.f;
        a1 = (i < g.Qb && ok1) ? a1 - si * prow[16] : 0.f;
      }
      acc[0][0] = mfma16(a0, x.x, acc[0][0]);
      acc[0][1] = mfma16(a0, x.y, acc[0][1]);
      acc[0][2] = mfma16(a0, x.z, acc[0][2]);
      acc[0][3] = mfma16(a0, x.w, acc[0][3]);
      acc[1][0] = mfma16(a1, x.x, acc[1][0]);
      acc[1][1] = mfma16(a1, x.y, acc[1][1]);
      acc[1][2] = mfma16(a1, x.z, acc[1][2]);
      acc[1][3] = mfma16(a1, x.w, acc[1][3]);
    }
  }
  float* out = is_v ? a.dvc : a.dkc;
  const float f = is_v ? 1.f : g.scale;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = j0 + 16 * u + 4 * kk + v;
      if (j < KVb) {
        float* o = out + g.pk(b, hk, j) + 64 * half + 4 * r;
        *reinterpret_cast<float4*>(o) =
            make_float4(f * acc[u][0][v], f * acc[u][1][v], f * acc[u][2][v], f * acc[u][3][v]);
      }
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
size_t fwd_lds(int cr, int KVb) { return (size_t)(row_area(cr, KVb) + NWC * 256) * 4; }
constexpr size_t ROWS_LDS = (size_t)(NWC * 2 * MR * HD + NWC * MR) * 4;
static_assert(2 * MR * QLD <= NWC * 2 * MR * HD, "pooled rows fit the partial-sum area");
}  // namespace

// LDS of the coarse backward's row pass (independent of the KV tile count)
size_t coarse_bwd_lds(int) { return ROWS_LDS; }

// Q tiles per work-group of the coarse forward: the most (up to one 16-row MFMA
// block) whose score rows fit in LDS; 0: KVb too large for these kernels.
int coarse_rows_per_block(int KVb) {
  for (int cr = 16; cr >= 1; cr >>= 1)
    if (fwd_lds(cr, KVb) <= 160 * 1024) return cr;
  return 0;
}

hipError_t launch_pool(const Geom& g, int dtype, const void* q, const void* k, const void* v,
                       float* qc, float* kc, float* vc, hipStream_t st) {
  const long long nq = (long long)g.B * g.Hq * g.Qb, nk = (long long)g.B * g.Hkv * g.KVb;
  const long long n = nq + 2 * nk;
  constexpr long long CHUNK = 1LL << 30;  // work-groups per launch
  auto go = [&](auto tag) {
    using ET = decltype(tag);
    for (long long b0 = 0; b0 < n; b0 += CHUNK)
      pool_kernel<ET><<<(unsigned)std::min(CHUNK, n - b0), 256, 0, st>>>(
          g, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, qc, kc, vc, b0);
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
  const size_t lds = fwd_lds(cr, g.KVb);
  const int tk = want_topk ? 1 : 0, gt = want_gate ? 1 : 0;
  switch (cr) {
    case 16: coarse_fwd_kernel<16><<<(unsigned)n, NWC * 64, lds, st>>>(a, tk, gt); break;
    case 8: coarse_fwd_kernel<8><<<(unsigned)n, NWC * 64, lds, st>>>(a, tk, gt); break;
    case 4: coarse_fwd_kernel<4><<<(unsigned)n, NWC * 64, lds, st>>>(a, tk, gt); break;
    case 2: coarse_fwd_kernel<2><<<(unsigned)n, NWC * 64, lds, st>>>(a, tk, gt); break;
    default: coarse_fwd_kernel<1><<<(unsigned)n, NWC * 64, lds, st>>>(a, tk, gt); break;
  }
  return hipGetLastError();
}

hipError_t launch_coarse_bwd(const CoarseArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const long long nr = (long long)g.B * g.Hq * ((g.Qb + MR - 1) / MR);
  const long long nc = (long long)g.B * g.Hkv * ((g.KVb + CCOL - 1) / CCOL);
  if (nr == 0 || nc == 0) return hipSuccess;
  coarse_bwd_rows_kernel<<<(unsigned)nr, NWC * 64, ROWS_LDS, st>>>(a);
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
