// Device helpers for MXFP4 (block-scaled FP4) weights, shared by the
// weight-streaming and the LDS-tiled expert GEMMs.  Layout (lmoe_quantize_mxfp4):
// two E2M1 codes per byte, element 2i in the low nibble; one scale byte per 32
// consecutive k, value 2^(byte - 127).
#pragma once
#include "lmoe_device.h"

namespace lmoe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Eight bf16 weights from one code word (bytes b0..b3, two elements each),
// decoded exactly by v_cvt_scalef32_pk_bf16_fp4 (element 0 = low nibble).
__device__ __forceinline__ bf16x8 mx_decode8(uint32_t word, float scale) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// 2^(byte - 127) as a float (byte 0 is the subnormal 2^-127).
__device__ __forceinline__ float mx_scale(uint32_t byte) {
  return byte ? __uint_as_float(byte << 23) : __uint_as_float(0x00400000u);
}

}  // namespace lmoe
