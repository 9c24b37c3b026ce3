// Device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "params.h"

namespace xattn {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.69314718055994530942f;

// Pool row (physical page * page_size + slot) of key t of a request whose logical
// pages start at page_base in the batch's page table.
__device__ __forceinline__ int64_t kv_row(const AttnParams& p, int page_base, int t) {
  int lp, slot;
  if (p.page_shift >= 0) {
    lp = t >> p.page_shift;
    slot = t & (p.page_size - 1);
  } else {
    lp = t / p.page_size;
    slot = t - lp * p.page_size;
  }
  const int64_t page = p.pages ? static_cast<int64_t>(p.pages[page_base + lp])
                               : static_cast<int64_t>(page_base) + lp;
  return page * p.page_size + slot;
}

// Element offset of (pool row, kv head, dim 0) in a [rows][hkv][d] pool.
__device__ __forceinline__ int64_t kv_offset(int64_t row, int hkv, int hk, int d) {
  return (row * hkv + hk) * d;
}

// Last key (inclusive) query token qi of a request may see; -1 when none.
// The queries are the last qo_len positions of the request's kv_len keys.
__device__ __forceinline__ int last_visible(int mask, int block, int qo_len, int kv_len, int qi) {
  if (kv_len <= 0) return -1;
  if (mask == 0) return kv_len - 1;
  const int pos = kv_len - qo_len + qi;
  if (mask == 1) return min(pos, kv_len - 1);
  const int64_t end = (static_cast<int64_t>(pos) / block + 1) * block;
  return static_cast<int>(min(end, static_cast<int64_t>(kv_len))) - 1;
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Round two floats to bf16 (nearest even) and pack them, a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = static_cast<__bf16>(a);
  v[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float a) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));
}

// Sum over the 8 lanes of an aligned group (DPP: quad swaps, then the half-row mirror).
__device__ __forceinline__ float sum8(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  return x;
}

// exp2 of x with the hardware instruction (x = -inf gives 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Dot product of two packed bf16 pairs accumulated into c (fp32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float shfl_xor_f(float x, int m) { return __shfl_xor(x, m, 64); }

}  // namespace xattn
