// Device-side helpers shared by the libk8v4 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace k8v4 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Cross-lane exchange within a wave64 (ds_bpermute based).
__device__ __forceinline__ float lane_xor(float x, int m) { return __shfl_xor(x, m, 64); }
__device__ __forceinline__ int lane_xor(int x, int m) { return __shfl_xor(x, m, 64); }
__device__ __forceinline__ float lane_get(float x, int src) { return __shfl(x, src, 64); }

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;  // v_cvt_f16_f32: round to nearest even, keeps -0 and subnormals
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t as_u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Four int8 codes (two's complement) -> two f16x2 holding code + 1152
// (exact): the byte is offset to code + 128 and placed under the exponent
// pattern 0x64 of 1024.
__device__ __forceinline__ void i8x4_to_f16_biased(uint32_t w, uint32_t &lo, uint32_t &hi) {
  const uint32_t u = w ^ 0x80808080u;
  lo = perm(0x64646464u, u, 0x04010400u);
  hi = perm(0x64646464u, u, 0x04030402u);
}

// Byte offset, inside the 144 * P byte q4_0 tile of one (page, KV head), of
// the fp16 scale of block b of slot s: the nibble bytes fill the first
// 128 * P bytes (slot s at 128 s); the scales follow in groups of 16 slots,
// 256 bytes per group laid out [block][slot % 16].
__host__ __device__ __forceinline__ size_t q4_scale_off(int P, int slot, int b) {
  return (size_t)128 * P + (size_t)(slot >> 4) * 256 + (size_t)b * 32 + (size_t)(slot & 15) * 2;
}

__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Walsh-Hadamard transform of the 256 values held 4 per lane (lane l holds
// dims 4l..4l+3): butterflies in ascending stride order 1, 2 (in-lane),
// then 4..128 across lanes, each output one fp32 add or subtract (lower
// index: a + b, upper index: a - b), then * 1/16.
__device__ __forceinline__ void fwht256_lane4(float y[4], int lane) {
#pragma clang fp contract(off)
  float a, b;
  a = y[0]; b = y[1]; y[0] = a + b; y[1] = a - b;
  a = y[2]; b = y[3]; y[2] = a + b; y[3] = a - b;
  a = y[0]; b = y[2]; y[0] = a + b; y[2] = a - b;
  a = y[1]; b = y[3]; y[1] = a + b; y[3] = a - b;
  for (int m = 1; m < 64; m <<= 1) {
    const bool upper = (lane & m) != 0;
    for (int i = 0; i < 4; i++) {
      const float p = lane_xor(y[i], m);
      y[i] = upper ? (p - y[i]) : (y[i] + p);
    }
  }
  for (int i = 0; i < 4; i++) y[i] = y[i] * 0.0625f;
}

}  // namespace k8v4
