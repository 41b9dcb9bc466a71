// Device-side helpers shared by the gfx950 kernels of the LatentMoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// bfloat16 is the high half of an IEEE float32.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float relu_sq(float v) {
  float r = v > 0.f ? v : 0.f;
  return r * r;
}

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies row
// l%16 of A and column l%16 of B, eight consecutive k each (k block l/16);
// lane l receives D rows 4*(l/16)+v, v = 0..3, of column l%16.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x4, fp32) * B(4x16, fp32); lane l supplies
// A[l%16][l/16] and B[l/16][l%16]; output layout as above.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Streaming load (each weight byte is used once): non-temporal hint.
__device__ __forceinline__ bf16x8 load8_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
  for (int i = 0; i < 8; ++i) z[i] = static_cast<__bf16>(0.0f);
  return z;
}

// Four fp32 values rounded to bfloat16 (relu^2 first for the second form).
__device__ __forceinline__ u16x4 pack4_bf16(f32x4 v) {
  u16x4 o;
  o[0] = f32_to_bf16(v[0]);
  o[1] = f32_to_bf16(v[1]);
  o[2] = f32_to_bf16(v[2]);
  o[3] = f32_to_bf16(v[3]);
  return o;
}
__device__ __forceinline__ u16x4 pack4_bf16_relu_sq(f32x4 v) {
  f32x4 a;
  a[0] = relu_sq(v[0]);
  a[1] = relu_sq(v[1]);
  a[2] = relu_sq(v[2]);
  a[3] = relu_sq(v[3]);
  return pack4_bf16(a);
}

// Store four consecutive fp32 values as bfloat16 (8-byte store).
__device__ __forceinline__ void store4_bf16(uint16_t* p, f32x4 v) {
  *reinterpret_cast<u16x4*>(p) = pack4_bf16(v);
}

// The same with the non-temporal hint.
__device__ __forceinline__ void store4_bf16_nt(uint16_t* p, f32x4 v) {
  __builtin_nontemporal_store(pack4_bf16(v), reinterpret_cast<u16x4*>(p));
}

__device__ __forceinline__ void store4_bf16_relu_sq(uint16_t* p, f32x4 v) {
  *reinterpret_cast<u16x4*>(p) = pack4_bf16_relu_sq(v);
}

__device__ __forceinline__ void store4_bf16_relu_sq_nt(uint16_t* p, f32x4 v) {
  __builtin_nontemporal_store(pack4_bf16_relu_sq(v), reinterpret_cast<u16x4*>(p));
}

// Work tile of the grouped expert GEMMs: rows [row0, row0 + nrows) of the
// expert-sorted slot list all belong to `expert`; the expert's tiles are
// tiles [first, first + count) of the list.
struct Tile {
  int32_t expert, row0, nrows, first, count, pad0, pad1, pad2;
};

}  // namespace lmoe
