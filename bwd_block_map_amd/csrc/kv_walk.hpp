// Chunked walk over the KV blocks one Q block selected (one row of the
// Q-owned CSR index), shared by the forward and the dQ kernels.
//
// The selected blocks are visited in index order, each in chunks of 64 keys;
// the last chunk of a block stops at its valid-key count, so a partial video
// tile costs one chunk. K and V chunks go global -> LDS with direct loads into
// a ring of NST slots (NST - 1 chunks in flight while one is computed). The
// direct loads are counted per wave and each step waits only for the slot it
// needs next. The block list itself (block id and valid keys) sits in LDS, a
// page of KV_LIST_CAP entries at a time, so the walk issues no dependent
// global loads.
#pragma once

#include "lds_tiles.hpp"

namespace vsa {

constexpr int KV_CHUNK = 64;                // keys per chunk
constexpr int KV_TILE = KV_CHUNK * HD * 2;  // bytes of one 64-row tile
constexpr int KV_LIST_CAP = 1024;           // block-list entries held in LDS at a time

// compute(Ks, Vs, rem): one chunk, with its K and V tiles in LDS (rows past the
// valid keys repeat the last valid row) and rem = its valid keys (1 .. 64).
// Every wave of the work-group calls walk_kv with the same arguments. All
// global loads the caller issued before are complete when compute first runs.
template <int NW, int NST, class F>
__device__ __forceinline__ void walk_kv(const Geom& g, int b, int hk, const int32_t* col, int e0,
                                        int cnt, const uint16_t* kp, const uint16_t* vp, int wave,
                                        int lane, F&& compute) {
  static_assert(NST >= 2 && NST <= 4, "ring of 2 to 4 slots");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NST][2][KV_TILE];  // [slot][K | V]
  __shared__ int lst_j[KV_LIST_CAP];
  __shared__ int lst_v[KV_LIST_CAP];
  if (cnt <= 0) return;

  const int tid = wave * 64 + lane;
  const long long kvb = uniform_i64(g.kv_base(b, hk)), krs = g.kv_rs();
  const uint32_t krs_bytes = (uint32_t)(krs * 2);
  auto load_page = [&](int base) {
    for (int t = tid; t < KV_LIST_CAP && base + t < cnt; t += NW * 64) {
      const int j = col[e0 + base + t];
      lst_j[t] = j;
      lst_v[t] = g.kv_val(b, j);
    }
  };
  load_page(0);
  wait_vm<0>();  // the caller's loads and the list page have landed
  __syncthreads();

  // stager: the next chunk to load: entry se of the list, `left` keys of its
  // block from that chunk on, and the element offset of the chunk's row 0.
  // All of it is wave-uniform and kept scalar, so a fill is a few scalar adds
  // and the direct loads.
  int se = 0, page = 0, left = 0;
  long long cur = 0;
  bool more = true;
  auto enter = [&]() {  // entry se (on the current page) becomes the stager's block
    const int j = __builtin_amdgcn_readfirstlane(lst_j[se - page]);
    left = __builtin_amdgcn_readfirstlane(lst_v[se - page]);  // >= 1 for a listed block
    cur = uniform_i64(kvb + (long long)j * g.kv_block * krs);
  };
  enter();
  auto advance = [&]() {
    left -= KV_CHUNK;
    if (left > 0) {
      cur += (long long)KV_CHUNK * krs;
      return;
    }
    if (++se >= cnt) {
      more = false;
      return;
    }
    if (se - page >= KV_LIST_CAP) {  // next page (only for lists longer than the cap)
      __syncthreads();
      page = se;
      load_page(page);
      __syncthreads();
    }
    enter();
  };
  // per slot, 8 bits of `slots`: valid keys of its chunk (1 .. 64), 0 if empty
  uint32_t slots = 0;
  auto fill = [&](int s) {
    slots &= ~(0xFFu << (8 * s));
    if (!more) return;
    slots |= (uint32_t)min(left, KV_CHUNK) << (8 * s);
    stage_rows<KV_CHUNK, NW>(ring[s][0], wave, lane, kp + cur, krs_bytes, left - 1);
    stage_rows<KV_CHUNK, NW>(ring[s][1], wave, lane, vp + cur, krs_bytes, left - 1);
    advance();
  };
  auto rem_of = [&](int s) { return (int)((slots >> (8 * s)) & 0xFFu); };
  constexpr int LPC = 2 * rows_loads<KV_CHUNK, NW>();  // direct loads per chunk and wave
  // wait until the chunk of slot s (the next one to compute) has landed; the
  // chunks of the slots after it may stay in flight
  auto wait_for = [&](int s) {
    int later = 0;
#pragma unroll
    for (int k = 1; k < NST - 1; ++k) later += rem_of((s + k) % NST) != 0;
    if (NST >= 4 && later >= 2) wait_vm<(NST >= 4 ? 2 : 0) * LPC>();
    else if (NST >= 3 && later >= 1) wait_vm<(NST >= 3 ? 1 : 0) * LPC>();
    else wait_vm<0>();
    lds_barrier();
  };

#pragma unroll
  for (int s = 0; s < NST - 1; ++s) fill(s);
  wait_for(0);
  for (int s = 0;;) {
    // refill the slot freed by the previous step, then compute slot s
    const int sf = s == 0 ? NST - 1 : s - 1;
    fill(sf);
    compute((const uint8_t*)ring[s][0], (const uint8_t*)ring[s][1], rem_of(s));
    s = s == NST - 1 ? 0 : s + 1;
    wait_for(s);
    if (rem_of(s) == 0) break;
  }
}

}  // namespace vsa
