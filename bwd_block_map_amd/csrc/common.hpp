// Shared device definitions of the gfx950 block-sparse attention kernels:
// element types, MFMA wrappers, the problem geometry and small helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vsa.h"

namespace vsa {

constexpr int HD = 128;  // head dimension the kernels are built for

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

struct bf16_tag {};
struct f16_tag {};

// Per element-type operations: the 32x32x16 MFMA (fp32 accumulate), packing
// of two fp32 values with round-to-nearest-even, and widening one element.
template <class T>
struct Elem;

template <>
struct Elem<bf16_tag> {
  static __device__ __forceinline__ f32x16_t mfma(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float x, float y) {
    f32x2_t v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  }
  // acc + lo + hi of a packed pair, in fp32 (v_dot2c_f32_bf16 against (1, 1))
  static __device__ __forceinline__ float sum2(uint32_t p, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p),
                                           __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
  }
  static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
};

template <>
struct Elem<f16_tag> {
  static __device__ __forceinline__ f32x16_t mfma(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float x, float y) {
    f32x2_t v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  }
  static __device__ __forceinline__ float sum2(uint32_t p, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, p),
                                  __builtin_bit_cast(f16x2_t, 0x3c003c00u), acc, false);
  }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
};

// Problem geometry as the kernels see it (a copy of vsa_problem's sizes plus
// device pointers), with the row addressing of the three layouts.
struct Geom {
  int layout, B, Hq, Hkv, Sq, Skv, q_block, kv_block, Qb, KVb, group;
  const int32_t* q_valid;
  const int32_t* kv_valid;
  long long qv_bs, kvv_bs;  // entries between batch entries of the counts (0: shared)
  const int32_t* cu_q;
  const int32_t* cu_kv;
  float scale;
  long long map_bstride;

  __device__ __forceinline__ int q_len(int b) const {
    return layout == VSA_TND ? cu_q[b + 1] - cu_q[b] : Sq;
  }
  __device__ __forceinline__ int kv_len(int b) const {
    return layout == VSA_TND ? cu_kv[b + 1] - cu_kv[b] : Skv;
  }
  // blocks covered by sequence b (never more than the map's extent)
  __device__ __forceinline__ int nqb(int b) const {
    return min(Qb, (q_len(b) + q_block - 1) / q_block);
  }
  __device__ __forceinline__ int nkb(int b) const {
    return min(KVb, (kv_len(b) + kv_block - 1) / kv_block);
  }
  __device__ __forceinline__ int q_exist(int b, int i) const {
    return max(0, min(q_block, q_len(b) - i * q_block));
  }
  __device__ __forceinline__ int kv_exist(int b, int j) const {
    return max(0, min(kv_block, kv_len(b) - j * kv_block));
  }
  // valid rows / keys of a block: the tile count when given, never more than exist
  __device__ __forceinline__ int q_val(int b, int i) const {
    const int e = q_exist(b, i);
    return q_valid ? min(q_valid[b * qv_bs + i], e) : e;
  }
  __device__ __forceinline__ int kv_val(int b, int j) const {
    const int e = kv_exist(b, j);
    return kv_valid ? min(kv_valid[b * kvv_bs + j], e) : e;
  }
  // element offset of row 0 of (b, head) and the distance between rows
  __device__ __forceinline__ long long q_base(int b, int h) const {
    if (layout == VSA_BHSD) return ((long long)b * Hq + h) * Sq * HD;
    if (layout == VSA_BSHD) return (long long)b * Sq * Hq * HD + (long long)h * HD;
    return (long long)cu_q[b] * Hq * HD + (long long)h * HD;
  }
  __device__ __forceinline__ long long q_rs() const {
    return layout == VSA_BHSD ? HD : (long long)Hq * HD;
  }
  __device__ __forceinline__ long long kv_base(int b, int hk) const {
    if (layout == VSA_BHSD) return ((long long)b * Hkv + hk) * Skv * HD;
    if (layout == VSA_BSHD) return (long long)b * Skv * Hkv * HD + (long long)hk * HD;
    return (long long)cu_kv[b] * Hkv * HD + (long long)hk * HD;
  }
  __device__ __forceinline__ long long kv_rs() const {
    return layout == VSA_BHSD ? HD : (long long)Hkv * HD;
  }
  // lse / row-term arrays: [B,Hq,Sq] or [Hq,Tq]; rows of a head are contiguous
  __device__ __forceinline__ long long lse_base(int b, int h) const {
    if (layout == VSA_TND) return (long long)h * Sq + cu_q[b];
    return ((long long)b * Hq + h) * Sq;
  }
  // one gate per (token, head): [B,Hq,Sq] (BHSD) or [B,Sq,Hq] (BSHD)
  __device__ __forceinline__ long long gtok_base(int b, int h) const {
    if (layout == VSA_BHSD) return ((long long)b * Hq + h) * Sq;
    return (long long)b * Sq * Hq + h;
  }
  __device__ __forceinline__ long long gtok_rs() const { return layout == VSA_BHSD ? 1 : Hq; }
  // pooled arrays: [B,Hq,Qb,HD] and [B,Hkv,KVb,HD]
  __device__ __forceinline__ long long pq(int b, int h, int i) const {
    return (((long long)b * Hq + h) * Qb + i) * HD;
  }
  __device__ __forceinline__ long long pk(int b, int hk, int j) const {
    return (((long long)b * Hkv + hk) * KVb + j) * HD;
  }
};

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void stg16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// Maximum without the NaN quieting of fmaxf (which costs one extra
// instruction per operand): NaN propagates, v_maximum3_f32 takes three inputs.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }

// max / sum of a value and its copy in lane l ^ 32
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Work-group order. The hardware deals consecutive work-group ids round-robin
// to the 8 XCDs (each with its own L2), so consecutive ids run on different
// XCDs at the same time. Keep that sweep (all XCDs work through the same head
// together, so the Infinity Cache holds one head's operands), but hand each
// group of G consecutive logical ids to one XCD, so the work-groups that read
// the same tile (the sub-tiles of one block) share an L2.
//
// The Q-owned kernels also keep XCD_QBLOCKS neighbouring Q blocks on one XCD:
// spatially local selections (neighbouring video tiles choosing overlapping
// KV tiles) then meet in L2. Measured at 720p with a band selection (Q block i
// takes the 144 KV blocks around i): forward -8.5 %, dQ -4.6 %; with random
// selections no change.
constexpr int XCD_QBLOCKS = 16;
__device__ __forceinline__ int xcd_group(int p, int n, int G) {
  constexpr int X = 8;
  const int full = n / (X * G) * (X * G);
  if (p >= full) return p;  // ragged tail: keep the hardware order
  const int q = p / X;
  return ((q / G) * X + p % X) * G + q % G;
}

constexpr float LOG2E = 1.4426950408889634f;

}  // namespace vsa
