// Device-side helpers shared by the gfx950 kernels: vector types, bf16/fp16
// conversion, CDNA4 MFMA wrappers and wave64 cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace diffattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
// D = A(32x16) * B(16x32) + C, bf16 inputs, fp32 accumulate (CDNA4).
// Lane l holds A row (l % 32) and B column (l % 32), eight k values each (k
// group l / 32); D row 8*(i/4) + 4*(l/32) + i%4, column l % 32 in element i.
__device__ __forceinline__ f32x16 mfma32_bf16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Reductions across the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48),
// with the gfx950 row-swap permutes.  permlane32_swap(x, x) returns
// {x[l mod 32], x[l mod 32 + 32]} in every lane l, and permlane16_swap(x, x)
// returns {x[l'], x[l' + 16]} with l' = l with bit 4 cleared, so each step
// combines a lane with its partner one row-pair (or one row) away.
__device__ __forceinline__ float max_across_rows(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_across_rows(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Sum over each row of 16 lanes with DPP lane permutations (VALU only, no LDS
// round trip): lane ^ 1, lane ^ 2, then the mirrored quad of each half-row and
// the mirrored half of the row.  Every lane of the row gets the row's sum.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xb1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_mov<0x4e>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}
// Sum over all 64 lanes (every lane gets it), in a fixed order.
__device__ __forceinline__ float wave_sum(float x) { return sum_across_rows(row16_sum(x)); }
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

// Sum of the eight bf16 values of a packed 16-byte fragment, added to acc, with
// the dot-product unit (v_dot2c_f32_bf16 against {1, 1}).
__device__ __forceinline__ float sum_bf16x8(const u32x4& p, float acc) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  const s16x2 ones = __builtin_bit_cast(s16x2, 0x3f803f80u);
  // (each word goes through a scalar copy: bit-casting a vector element
  // directly would reinterpret the vector's first word)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = p[j];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(s16x2, w), ones, acc, false);
  }
  return acc;
}
// Sum of the eight fp16 values of a packed 16-byte fragment, added to acc.
__device__ __forceinline__ float sum_f16x8(const u32x4& p, float acc) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  const f16x2 ones = __builtin_bit_cast(f16x2, 0x3c003c00u);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t w = p[j];
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), ones, acc, false);
  }
  return acc;
}
// Eight packed bf16 values times s, rounded back to bf16 (nearest even).
__device__ __forceinline__ u32x4 scale_bf16x8(const u32x4& q, float s) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r[j] = pack_bf16x2(bf16lo_to_f32(q[j]) * s, bf16hi_to_f32(q[j]) * s);
  return r;
}

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

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each 16-lane row
// of the wave, lane j supplies the address of an 8-byte chunk; the 16 chunks
// form a 4 x 16 matrix of 16-bit values whose row r is the chunks of lanes
// 4r..4r+3 in order.  Lane c receives column c: {M[0][c], M[1][c], M[2][c], M[3][c]}.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds_addr) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<void*>(lds_addr)));
  return __builtin_bit_cast(u32x2, v);
}

// Direct global->LDS copy of 16 bytes per lane (gfx950 buffer_load_dwordx4 ...
// lds): lane l's bytes land at lds_base + 16 * l.  `base` is wave-uniform and
// becomes a raw buffer resource (scalar registers, no range limit); `byte_off`
// is the per-lane 32-bit offset.  The buffer form rather than
// global_load_lds: the compiler counts a pending global (flat-encoded) LDS
// load against the LDS wait counter as well, and then makes every later LDS
// read wait for all outstanding LDS reads, so no read can be kept in flight
// behind the MFMAs while a tile is loading.
constexpr int kBufferRsrcWord3 = 0x00020000;
__device__ __forceinline__ void dma16(const void* base, uint32_t byte_off, void* lds_base) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0xffffffff, kBufferRsrcWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)(lds_base), 16, (int)byte_off, 0, 0, 0);
}

// Register-allocation hint: the value lives in accumulation registers here.
__device__ __forceinline__ void pin_agpr(f32x4& v) { asm volatile("" : "+a"(v)); }

// Wave-uniform "any lane" vote.
__device__ __forceinline__ bool wave_any(bool p) { return __any(p); }

}  // namespace diffattn
