// LDS tiles of 16-bit rows of HD = 128 elements (256 B = 16 chunks of 16 B)
// for the MFMA kernels, filled by direct global->LDS loads and read either
// row-wise (an MFMA operand whose contraction runs along d) or transposed
// with ds_read_b64_tr_b16 (an operand whose contraction runs along the rows).
//
// Swizzle: chunk c of row r is stored at chunk c ^ swz(r), with swz swapping
// the two low 2-bit fields of r. Then 16 consecutive rows read at one chunk hit
// 16 distinct chunk slots (row-wise 16-byte reads), and the transposed read of
// 4 consecutive rows x 4 consecutive chunks also hits 16 distinct slots.
#pragma once

#include "common.hpp"

namespace vsa {

typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// byte offset of chunk c of row r inside a tile
__device__ __forceinline__ uint32_t toff(int r, int c) {
  return (uint32_t)(r * 256 + ((c ^ swz(r)) << 4));
}

// LDS address (byte offset) of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct global -> LDS load of 16 bytes per lane: lane i fills lds + 16 i from
// base + voff. Issued from inline asm so that the compiler does not track it:
// its own tracking of these loads merges LDS buffers at loop heads and then
// waits for every prefetch before any LDS read. Callers wait with wait_vm and
// synchronise with lds_barrier. M0 carries the LDS base; no other instruction
// in these kernels reads M0, so setting it here clobbers nothing.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// base and lds are wave-uniform; readfirstlane states that to the compiler
// (it folds away when they already live in scalar registers)
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// a wave-uniform 64-bit integer, stated as such (keeps derived values scalar)
__device__ __forceinline__ long long uniform_i64(long long x) {
  const uint64_t v = (uint64_t)x;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (long long)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(uniform_ptr(base)),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "m0", "memory");
}
// the same with 4 bytes per lane (lane i fills lds + 4 i)
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(uniform_ptr(base)),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "m0", "memory");
}
#pragma clang diagnostic pop

// Stage RT rows of a tile whose row r lives at base + min(r, last) * rs_bytes:
// the base is uniform and each lane adds a 32-bit offset computed with a 24-bit
// multiply (row < 256; the C ABI keeps a row stride below 2^24 bytes, fewer
// than 65536 heads in the token-major layouts, so the offset stays below 2^32),
// which keeps the address arithmetic to two 24-bit integer ops.
template <int RT, int NW>
__device__ __forceinline__ void stage_rows(uint8_t* tile, int wave, int lane, const uint16_t* base,
                                           uint32_t rs_bytes, int last) {
  constexpr int P = RT / 4;  // wave instructions of the tile
  const uint32_t t0 = lds_addr(tile);
#pragma unroll
  for (int k = 0; k < (P + NW - 1) / NW; ++k) {
    const int p = wave + k * NW;
    if (P % NW == 0 || p < P) {
      const int row = 4 * p + (lane >> 4);
      const uint32_t c = (uint32_t)((lane & 15) ^ swz(row));
      const uint32_t off = (uint32_t)__umul24((uint32_t)min(row, last), rs_bytes) + 16u * c;
      dma16(base, off, t0 + p * 1024);
    }
  }
}

// Direct loads one wave issues for an RT-row tile (when every wave issues the same number).
template <int RT, int NW>
constexpr int rows_loads() {
  static_assert((RT / 4) % NW == 0, "waves issue equal shares");
  return RT / 4 / NW;
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (loads complete in order; the other counters are left alone).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Work-group barrier for LDS tiles filled by direct loads. __syncthreads()
// carries a release fence that on this target drains every outstanding global
// load, which would also wait for the chunks prefetched further ahead. Here
// each wave first retires its own LDS reads and writes (the direct loads it
// must have landed are waited for by the caller with wait_vm), the empty asm
// statements keep the compiler from moving memory operations across, and the
// hardware barrier does the rest.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-lane byte offsets of the row-wise operand reads. A wave reads rows
// R + (lane & 31) (R a multiple of 16, so the swizzle depends on the lane
// only) at chunk 2ks + (lane >> 5): offset = R*256 + o[ks].
struct RowOffs {
  uint32_t o[8];
  __device__ __forceinline__ explicit RowOffs(int lane) {
    const int r = lane & 31, hl = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) o[ks] = toff(r, 2 * ks + hl);
  }
  __device__ __forceinline__ uint4 at(const uint8_t* tile, int R, int ks) const {
    return *reinterpret_cast<const uint4*>(tile + R * 256 + o[ks]);
  }
};

__device__ __forceinline__ uint2 tr8(const uint8_t* tile, uint32_t off) {
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(tile + off));
  return __builtin_bit_cast(uint2, v);
}

// Transposed A operand of a 32x32x16 MFMA whose M index is d (32*mb + lane%32)
// and whose contraction runs over tile rows rb .. rb+15, in the lane order the
// transposed accumulators use: k-slot e (0..3) of lane half hl is row
// rb + 4hl + e, k-slot 4 + e is row rb + 8 + 4hl + e. ds_read_b64_tr_b16 works
// on 16-lane groups: source lane 4e + i reads 4 elements (d = D0 + 4i .. +3) of
// row e; result lane 4i + c receives element c of the four rows.
struct TrLane {
  uint32_t row_off;  // (4hl + e) rows, as a row index
  int c_off;         // 2g + (i >> 1)
  uint32_t half;     // 8 * (i & 1) bytes
  __device__ __forceinline__ explicit TrLane(int lane) {
    const int s = lane & 15, e = s >> 2, i = s & 3, g = (lane >> 4) & 1, hl = lane >> 5;
    row_off = (uint32_t)(4 * hl + e);
    c_off = 2 * g + (i >> 1);
    half = 8u * (uint32_t)(i & 1);
  }
};

// Per-lane byte offsets of the transposed operand reads: rows rb + {0..15}
// with rb a multiple of 16, so for each (low / high row group, mb) the offset
// is rb*256 + o[hi][mb].
struct TrOffs {
  uint32_t o[2][4];
  __device__ __forceinline__ explicit TrOffs(int lane) {
    const TrLane t(lane);
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        o[hi][mb] = toff((int)t.row_off + 8 * hi, 4 * mb + t.c_off) + t.half;
  }
  __device__ __forceinline__ uint4 at(const uint8_t* tile, int rb, int mb) const {
    const uint2 lo = tr8(tile, (uint32_t)(rb * 256) + o[0][mb]);
    const uint2 hi = tr8(tile, (uint32_t)(rb * 256) + o[1][mb]);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
};

}  // namespace vsa
