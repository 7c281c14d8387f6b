// Device-side helpers shared by the gfx950 kernels: vector types, bf16/fp16
// conversion, CDNA4 MFMA wrappers and wave64 cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace diffattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, b);
}
// Two fp32 -> packed bf16x2 (lo = a, hi = b), round-to-nearest-even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
// Two fp32 -> packed fp16x2 (lo = a, hi = b), round-to-nearest-even.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
// Packed bf16x2 -> packed fp16x2.  Exact for |x| in the fp16 normal range
// [2^-14, 65504]; smaller magnitudes become fp16 subnormals (abs error < 2^-25).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16x2(bf16lo_to_f32(w), bf16hi_to_f32(w));
}

// v_perm_b32 byte select: result byte i = selector byte i picks from {hi:lo} = {a:b}
// (bytes 0-3 from b, 4-7 from a).
__device__ __forceinline__ uint32_t perm_b32(uint32_t a, uint32_t b, uint32_t sel) {
  return __builtin_amdgcn_perm(a, b, sel);
}
// lo halves of x and y -> {y.lo : x.lo}  (x.lo in bits 0-15)
__device__ __forceinline__ uint32_t pack_lo16(uint32_t x, uint32_t y) {
  return perm_b32(y, x, 0x05040100u);
}
// hi halves of x and y -> {y.hi : x.hi}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t x, uint32_t y) {
  return perm_b32(y, x, 0x07060302u);
}

// D = A(16x32) * B(32x16) + C, bf16 inputs, fp32 accumulate (CDNA4).
// Lane l holds A row (l % 16) and B column (l % 16), eight k values each (k
// group l / 16); D row 4*(l/16)+i, column l % 16 in element i.
__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Reductions across the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float max_across_rows(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float sum_across_rows(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ __forceinline__ float sum_within_row16(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}
__device__ __forceinline__ float max_within_row16(float x) {
  x = fmaxf(x, __shfl_xor(x, 1));
  x = fmaxf(x, __shfl_xor(x, 2));
  x = fmaxf(x, __shfl_xor(x, 4));
  x = fmaxf(x, __shfl_xor(x, 8));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Logistic function in fp32: 1 / (1 + 2^(-x log2 e)).  For x >= 40 it is exactly 1.0f.
__device__ __forceinline__ float sigmoid_f32(float x) {
  return 1.0f / (1.0f + exp2f(-x * kLog2e));
}

__device__ __forceinline__ u32x4 ldg128(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void stg128(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// Register-allocation hint: the value lives in accumulation registers here.
__device__ __forceinline__ void pin_agpr(f32x4& v) { asm volatile("" : "+a"(v)); }

// Wave-uniform "any lane" vote.
__device__ __forceinline__ bool wave_any(bool p) { return __any(p); }

}  // namespace diffattn
