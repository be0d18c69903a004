// Block map -> CSR index of the live (Q block, KV block) pairs.
//
// FastVideo block_sparse_attn_cute_fwd.py: `_map_to_index` turns the boolean
// map into per-row block lists, `_build_sparse_tensors` drops KV tiles with no
// valid token and builds the backward's KV-owned lists from the transposed map.
// Here both directions are CSR (nnz-sized instead of dense [.., KVb, Qb]):
// count -> exclusive scan -> fill, all deterministic, columns ascending.
#include "kernels.hpp"

namespace vsa {

// Q-owned count: one wave per row (b, h, i); lanes read 64 consecutive map
// bytes per step and a ballot counts the live ones.
__global__ __launch_bounds__(256) void index_count_q(Geom g, const uint8_t* __restrict__ map,
                                                     int32_t* __restrict__ row_ptr) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long rows = (long long)g.B * g.Hq * g.Qb;
  if (row >= rows) return;
  const int i = (int)(row % g.Qb);
  const long long bh = row / g.Qb;
  const int h = (int)(bh % g.Hq), b = (int)(bh / g.Hq);
  const uint8_t* m = map + b * g.map_bstride + ((long long)h * g.Qb + i) * g.KVb;
  const bool qok = i < g.nqb(b);
  const int nk = g.nkb(b);
  int cnt = 0;
  for (int j0 = 0; j0 < g.KVb; j0 += 64) {
    const int j = j0 + lane;
    const bool live = qok && j < nk && m[j] != 0 && g.kv_val(b, j) > 0;
    cnt += __popcll(__ballot(live));
  }
  if (lane == 0) row_ptr[row + 1] = cnt;
}

// Q-owned fill: same walk, each live entry written at its rank in the row.
__global__ __launch_bounds__(256) void index_fill_q(Geom g, const uint8_t* __restrict__ map,
                                                    const int32_t* __restrict__ row_ptr,
                                                    int32_t* __restrict__ col, long long cap) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long rows = (long long)g.B * g.Hq * g.Qb;
  if (row >= rows) return;
  const int i = (int)(row % g.Qb);
  const long long bh = row / g.Qb;
  const int h = (int)(bh % g.Hq), b = (int)(bh / g.Hq);
  const uint8_t* m = map + b * g.map_bstride + ((long long)h * g.Qb + i) * g.KVb;
  const bool qok = i < g.nqb(b);
  const int nk = g.nkb(b);
  long long pos = row_ptr[row];
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int j0 = 0; j0 < g.KVb; j0 += 64) {
    const int j = j0 + lane;
    const bool live = qok && j < nk && m[j] != 0 && g.kv_val(b, j) > 0;
    const unsigned long long bal = __ballot(live);
    const long long at = pos + __popcll(bal & below);
    if (live && at < cap) col[at] = j;
    pos += __popcll(bal);
  }
}

// KV-owned count / fill: a work-group takes 64 columns (b, h, j) and its four
// waves split each column's rows i into four segments; lanes of a wave read
// 64 consecutive map bytes of one row per step. The fill places a segment
// after the live entries of the segments above it, so the columns stay in
// ascending row order.
constexpr int KV_SEG = 4;
__device__ __forceinline__ int kv_seg_count(const Geom& g, const uint8_t* __restrict__ map, long long t,
                                            int seg, int* nq_out, const uint8_t** m_out, int* i0,
                                            int* i1) {
  const int j = (int)(t % g.KVb);
  const long long bh = t / g.KVb;
  const int h = (int)(bh % g.Hq), b = (int)(bh / g.Hq);
  const bool col_ok = j < g.nkb(b) && g.kv_val(b, j) > 0;
  const int nq = col_ok ? g.nqb(b) : 0;
  const int per = (nq + KV_SEG - 1) / KV_SEG;
  *i0 = min(seg * per, nq);
  *i1 = min(*i0 + per, nq);
  *m_out = map + b * g.map_bstride + (long long)h * g.Qb * g.KVb + j;
  *nq_out = nq;
  int cnt = 0;
  for (int i = *i0; i < *i1; ++i) cnt += (*m_out)[(long long)i * g.KVb] != 0;
  return cnt;
}

__global__ __launch_bounds__(256) void index_count_kv(Geom g, const uint8_t* __restrict__ map,
                                                      int32_t* __restrict__ row_ptr) {
  __shared__ int part[KV_SEG][64];
  const int lane = threadIdx.x & 63, seg = threadIdx.x >> 6;
  const long long t = (long long)blockIdx.x * 64 + lane;
  const long long rows = (long long)g.B * g.Hq * g.KVb;
  int nq = 0, i0 = 0, i1 = 0;
  const uint8_t* m = nullptr;
  part[seg][lane] = t < rows ? kv_seg_count(g, map, t, seg, &nq, &m, &i0, &i1) : 0;
  __syncthreads();
  if (seg == 0 && t < rows) row_ptr[t + 1] = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
}

__global__ __launch_bounds__(256) void index_fill_kv(Geom g, const uint8_t* __restrict__ map,
                                                     const int32_t* __restrict__ row_ptr,
                                                     int32_t* __restrict__ col, long long cap) {
  __shared__ int part[KV_SEG][64];
  const int lane = threadIdx.x & 63, seg = threadIdx.x >> 6;
  const long long t = (long long)blockIdx.x * 64 + lane;
  const long long rows = (long long)g.B * g.Hq * g.KVb;
  int nq = 0, i0 = 0, i1 = 0;
  const uint8_t* m = nullptr;
  part[seg][lane] = t < rows ? kv_seg_count(g, map, t, seg, &nq, &m, &i0, &i1) : 0;
  __syncthreads();
  if (t >= rows) return;
  long long pos = row_ptr[t];
  for (int s2 = 0; s2 < seg; ++s2) pos += part[s2][lane];
  for (int i = i0; i < i1; ++i)
    if (m[(long long)i * g.KVb] != 0) {
      if (pos < cap) col[pos] = i;
      ++pos;
    }
}

// In-place exclusive scan of the counts row_ptr[1..rows] by one work-group:
// every thread sums a contiguous segment, the segment sums are scanned in LDS,
// then each thread rewrites its segment.
__global__ __launch_bounds__(1024) void index_scan(int32_t* __restrict__ row_ptr, long long rows) {
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const long long per = (rows + 1023) / 1024;
  const long long beg = t * per, end = min(beg + per, rows);
  int32_t s = 0;
  for (long long r = beg; r < end; ++r) s += row_ptr[r + 1];
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int32_t acc = part[t] - s;  // exclusive prefix of this segment
  for (long long r = beg; r < end; ++r) {
    acc += row_ptr[r + 1];
    row_ptr[r + 1] = acc;
  }
  if (t == 0) row_ptr[0] = 0;
}

// Small maps in one launch (the three launches above cost more than the work
// for, e.g., a [2, 8, 32, 32] map): one work-group stages the map in LDS with
// coalesced loads, counts every row there (a thread per row), scans the counts,
// writes row_ptr and fills col. Same CSR as the three-kernel path. Launched
// with two work-groups it builds both directions at once: work-group 1 the
// KV-owned index into (row_ptr1, col1).
constexpr int SMALL_ROWS = 8192;       // rows whose counts fit in LDS
constexpr int SMALL_MAP = 64 * 1024;   // map bytes staged in LDS

__global__ __launch_bounds__(1024) void index_small(Geom g, const uint8_t* __restrict__ map,
                                                    int kv_owned0, int32_t* __restrict__ row_ptr0,
                                                    int32_t* __restrict__ col0,
                                                    int32_t* __restrict__ row_ptr1,
                                                    int32_t* __restrict__ col1, long long cap) {
  const int kv_owned = blockIdx.x ? 1 : kv_owned0;
  int32_t* __restrict__ row_ptr = blockIdx.x ? row_ptr1 : row_ptr0;
  int32_t* __restrict__ col = blockIdx.x ? col1 : col0;
  __shared__ uint8_t mp[SMALL_MAP];
  __shared__ int32_t start[SMALL_ROWS];
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const int nr = kv_owned ? g.KVb : g.Qb;
  const int rows = g.B * g.Hq * nr;
  const int per_b = g.Hq * g.Qb * g.KVb;
  const int staged = (g.map_bstride ? g.B : 1) * per_b;
  for (int x = t; x < staged; x += 1024) mp[x] = map[(x / per_b) * g.map_bstride + x % per_b];
  __syncthreads();
  // the live entries of row r in ascending column order: fn(column)
  auto walk = [&](int r, auto&& fn) {
    const int x = r % nr, bh = r / nr;
    const int h = bh % g.Hq, b = bh / g.Hq;
    const uint8_t* m = mp + (g.map_bstride ? b : 0) * per_b + h * g.Qb * g.KVb;
    if (!kv_owned) {
      if (x >= g.nqb(b)) return;
      const int nk = g.nkb(b);
      for (int j = 0; j < nk; ++j)
        if (m[x * g.KVb + j] != 0 && g.kv_val(b, j) > 0) fn(j);
    } else {
      if (x >= g.nkb(b) || g.kv_val(b, x) == 0) return;
      const int nq = g.nqb(b);
      for (int i = 0; i < nq; ++i)
        if (m[i * g.KVb + x] != 0) fn(i);
    }
  };
  for (int r = t; r < rows; r += 1024) {
    int c = 0;
    walk(r, [&](int) { ++c; });
    start[r] = c;
  }
  __syncthreads();
  // exclusive scan: contiguous segments per thread, their sums scanned in LDS
  const int per = (rows + 1023) / 1024, beg = min(t * per, rows), end = min(beg + per, rows);
  int32_t s = 0;
  for (int r = beg; r < end; ++r) s += start[r];
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int32_t acc = part[t] - s;
  for (int r = beg; r < end; ++r) {
    const int32_t c = start[r];
    start[r] = acc;
    acc += c;
  }
  __syncthreads();
  for (int r = t; r < rows; r += 1024) {
    row_ptr[r] = start[r];
    long long pos = start[r];
    walk(r, [&](int c) {
      if (pos < cap) col[pos] = c;
      ++pos;
    });
  }
  if (t == 0) row_ptr[rows] = part[1023];
}

// a[1 .. n] holds counts; afterwards a[0] = 0 and a[r] = the sum of the first r
hipError_t launch_exclusive_scan(int32_t* a, long long n, hipStream_t st) {
  index_scan<<<1, 1024, 0, st>>>(a, n);
  return hipGetLastError();
}

hipError_t launch_index(const Geom& g, const uint8_t* map, int kv_owned, int32_t* row_ptr,
                        int32_t* col, long long cap, hipStream_t st) {
  const long long rows = (long long)g.B * g.Hq * (kv_owned ? g.KVb : g.Qb);
  if (rows == 0) {  // only row_ptr[0] = 0
    index_scan<<<1, 1024, 0, st>>>(row_ptr, 0);
    return hipGetLastError();
  }
  const long long staged = (g.map_bstride ? g.B : 1LL) * g.Hq * g.Qb * g.KVb;
  if (rows <= SMALL_ROWS && staged <= SMALL_MAP) {
    index_small<<<1, 1024, 0, st>>>(g, map, kv_owned, row_ptr, col, nullptr, nullptr, cap);
  } else if (!kv_owned) {
    const unsigned grid = (unsigned)((rows + 3) / 4);
    index_count_q<<<grid, 256, 0, st>>>(g, map, row_ptr);
    index_scan<<<1, 1024, 0, st>>>(row_ptr, rows);
    index_fill_q<<<grid, 256, 0, st>>>(g, map, row_ptr, col, cap);
  } else {
    const unsigned grid = (unsigned)((rows + 63) / 64);
    index_count_kv<<<grid, 256, 0, st>>>(g, map, row_ptr);
    index_scan<<<1, 1024, 0, st>>>(row_ptr, rows);
    index_fill_kv<<<grid, 256, 0, st>>>(g, map, row_ptr, col, cap);
  }
  return hipGetLastError();
}

hipError_t launch_index_both(const Geom& g, const uint8_t* map, int32_t* q_rp, int32_t* q_col,
                             int32_t* kv_rp, int32_t* kv_col, long long cap, hipStream_t st) {
  const long long rq = (long long)g.B * g.Hq * g.Qb, rk = (long long)g.B * g.Hq * g.KVb;
  const long long staged = (g.map_bstride ? g.B : 1LL) * g.Hq * g.Qb * g.KVb;
  if (rq > 0 && rk > 0 && rq <= SMALL_ROWS && rk <= SMALL_ROWS && staged <= SMALL_MAP) {
    index_small<<<2, 1024, 0, st>>>(g, map, 0, q_rp, q_col, kv_rp, kv_col, cap);
    return hipGetLastError();
  }
  const hipError_t e = launch_index(g, map, 0, q_rp, q_col, cap, st);
  return e != hipSuccess ? e : launch_index(g, map, 1, kv_rp, kv_col, cap, st);
}

}  // namespace vsa
