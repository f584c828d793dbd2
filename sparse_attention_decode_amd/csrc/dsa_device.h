// Device helpers shared by the DSA kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kBlock = 64;  // tokens per pool block (the only block size built)

// Kernel-side view of the pool layout.
struct PoolView {
  const uint8_t* base;
  int64_t row_bytes, lat_off, lat_scale_off, ikey_off, ikey_scale_off;
  int64_t tokens;  // num_blocks * block size: bound on physical token rows
};

// Order-preserving 32-bit key of an fp32 score: a larger score gives a larger key; -0 maps to the
// key of +0 so the two tie.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Workgroup barrier over LDS only: waits for this wave's LDS operations, not its global loads or
// stores (__syncthreads waits for those too).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16x16x128 FP8 x FP8 MFMA (E4M3 operands, fp32 accumulate).  Operand layout, lane l,
// group g = l / 16: row/col l % 16; bytes 0..15 hold K [16g, 16g+16), bytes 16..31 hold
// K [64+16g, 64+16g+16).  Result lane l: rows 4g..4g+3, col l % 16.
__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16x16x128 FP8 (A) x FP4 E2M1 (B) MFMA with E8M0 block scales.  B operand lane l holds
// K [32g, 32g+32) of column l % 16 in its first 16 bytes (element 2j = low nibble of byte j);
// the scale of row/col m and K block kb is taken from lane m + 16 kb (E8M0, 127 = 1.0).
__device__ __forceinline__ v4f mfma_fp8_fp4(v8i a, v8i b, v4f c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, scale_a, 0, scale_b);
}

// 16x16x32 bf16 MFMA: A lane l row l % 16, K [8g, 8g+8); B lane l col l % 16, same K.
__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 fp16 MFMA, same operand layout as the bf16 one.
__device__ __forceinline__ v4f mfma_f16(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// fp32 -> fp16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// E4M3 byte -> fp32.
__device__ __forceinline__ float fp8_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(byte, false)[0];
}

// Wave-wide (64-lane) inclusive prefix sum.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

// Sums / maxima over lane pairs (l, l ^ 16) and (l, l ^ 32) in VALU: permlane16/32_swap(x, x)
// returns the two halves of each 32 / 64-lane group side by side, so adding (or taking the max
// of) the pair gives every lane the pair's result (both lanes of a pair get the same bits).
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}

}  // namespace dsa
