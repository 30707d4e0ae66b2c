// Device-side building blocks for gfx950 (CDNA4): vector types, MFMA wrappers, the LDS
// tile swizzle and small wave helpers. Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace da {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWave = 64;

// ---------------------------------------------------------------------------- MFMA
// 32x32x16 bf16 -> f32. Lane l supplies A[l%32][8*(l/32) + e] and B[8*(l/32) + e][l%32]
// (e = 0..7); accumulator element 4*i + j of lane l is C[8*i + 4*(l/32) + j][l%32].
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// 32x32x2 f32 -> f32. Lane l supplies A[l%32][l/32] and B[l/32][l%32]; same C layout.
__device__ __forceinline__ f32x16 mfma32x32x2(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------- LDS tiles
// A bf16 tile of R rows x D columns is stored row-major in 16-byte chunks, chunk c of row r
// at physical chunk c ^ swz_key<D>(r). For D = 128 (16 chunks, rows 256 B apart) the key is
// a bijection on 0..15 over any 16 consecutive rows (32 lanes reading one logical chunk of
// consecutive rows spread over all banks) and gives 4 consecutive rows disjoint 4-chunk
// groups (the transposed 8-byte reads of 4 rows x 4 chunks hit 16 distinct bank groups).
template <int D>
__device__ __forceinline__ int swz_key(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (row >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int swz_byte(int row, int chunk) {
  return row * (D * 2) + ((chunk ^ swz_key<D>(row)) << 4);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const char* base, int byte_off) {
  return *reinterpret_cast<const bf16x8*>(base + byte_off);
}

// Word 3 of a gfx9-family raw buffer resource (32-bit data format, no swizzle or stride).
constexpr int kBufferWord3 = 0x00020000;

// LDS byte address of a shared-memory object (a constant once the kernel's LDS is laid out).
__device__ __forceinline__ int lds_addr(const void* p) {
  return (int)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// gfx950 transposed LDS read: within each 16-lane group, output lane i, slot s receives
// element (i % 4) of the 8 bytes addressed by lane 4*s + i/4 of the same group.
__device__ __forceinline__ bf16x4 lds_read_tr16(const char* base, int byte_off) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) char*)
                                                     (base) + byte_off));
  return __builtin_bit_cast(bf16x4, r);
}

// ---------------------------------------------------------------------------- helpers
__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// float -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Read-only, wave-uniform loads through the scalar cache.
__device__ __forceinline__ int32_t sload(const int32_t* base, int idx) {
  return ((const __attribute__((address_space(4))) int32_t*)(base))[idx];
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace da
