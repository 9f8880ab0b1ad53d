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

// x of lane (lane ^ M), M a power of two below 64, with every lane of the
// wave active.  VALU only, no trip through the LDS crossbar: DPP inside
// rows of 16 (quad_perm for 1 and 2; row_ror:n, which reads lane
// (i - n) mod 16, for 4 and 8) and gfx950's permlane swaps across rows and
// halves: swapping a value with itself leaves the lower row (half) in the
// first result and the upper one in the second.
template <int M>
__device__ __forceinline__ int lane_xor(int x) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "lane_xor: M");
  const int lane = __lane_id();
  if constexpr (M == 1) {
    return __builtin_amdgcn_mov_dpp(x, 0xb1, 0xf, 0xf, false);  // quad_perm [1, 0, 3, 2]
  } else if constexpr (M == 2) {
    return __builtin_amdgcn_mov_dpp(x, 0x4e, 0xf, 0xf, false);  // quad_perm [2, 3, 0, 1]
  } else if constexpr (M == 4) {
    const int up = __builtin_amdgcn_mov_dpp(x, 0x124, 0xf, 0xf, false);  // row_ror:4, lane i - 4
    const int dn = __builtin_amdgcn_mov_dpp(x, 0x12c, 0xf, 0xf, false);  // row_ror:12, lane i + 4
    return (lane & 4) ? up : dn;
  } else if constexpr (M == 8) {
    return __builtin_amdgcn_mov_dpp(x, 0x128, 0xf, 0xf, false);  // row_ror:8
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    return (int)((lane & 16) ? r[0] : r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    return (int)((lane & 32) ? r[0] : r[1]);
  }
}
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
  return __builtin_bit_cast(float, lane_xor<M>(__builtin_bit_cast(int, x)));
}
// Butterfly reductions over all 64 lanes and over the 16 lanes of one
// 16-lane group (lanes sharing lane / 16).
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, lane_xor<32>(x));
  x = fmaxf(x, lane_xor<16>(x));
  x = fmaxf(x, lane_xor<8>(x));
  x = fmaxf(x, lane_xor<4>(x));
  x = fmaxf(x, lane_xor<2>(x));
  return fmaxf(x, lane_xor<1>(x));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += lane_xor<32>(x);
  x += lane_xor<16>(x);
  x += lane_xor<8>(x);
  x += lane_xor<4>(x);
  x += lane_xor<2>(x);
  return x + lane_xor<1>(x);
}
// sum over the 4 lanes l, l ^ 16, l ^ 32, l ^ 48
__device__ __forceinline__ float sum_lg(float x) {
  x += lane_xor<16>(x);
  return x + lane_xor<32>(x);
}
__device__ __forceinline__ float max_lg(float x) {
  x = fmaxf(x, lane_xor<16>(x));
  return fmaxf(x, lane_xor<32>(x));
}
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

// one cross-lane butterfly of stride 4 M dims (lane stride M)
// (lower index: a + b, upper index: a - b, formed as b + (-a) on the upper
// lane, which IEEE addition rounds exactly like b - a; the sign flip is one
// xor, so a stage is one cross-lane move and one add per value)
template <int M>
__device__ __forceinline__ float fwht_pair(float y, uint32_t neg) {
#pragma clang fp contract(off)
  if constexpr (M == 16 || M == 32) {
    // swapping y with itself leaves the lower row (half) in the first
    // result and the upper one in the second, in every lane: lower lanes
    // form lo + hi, upper lanes lo + (-hi)
    const auto r = M == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false)
                           : __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1] ^ neg);
  } else {
    return lane_xor<M>(y) + __uint_as_float(__float_as_uint(y) ^ neg);
  }
}

template <int M>
__device__ __forceinline__ void fwht_stage(float y[4], int lane) {
  const uint32_t neg = (lane & M) ? 0x80000000u : 0u;
  for (int i = 0; i < 4; i++) y[i] = fwht_pair<M>(y[i], neg);
}

// the same stage on 8 values (two rows of 4)
template <int M>
__device__ __forceinline__ void fwht_stage8(float y[8], int lane) {
  const uint32_t neg = (lane & M) ? 0x80000000u : 0u;
  for (int i = 0; i < 8; i++) y[i] = fwht_pair<M>(y[i], neg);
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
  fwht_stage<1>(y, lane);
  fwht_stage<2>(y, lane);
  fwht_stage<4>(y, lane);
  fwht_stage<8>(y, lane);
  fwht_stage<16>(y, lane);
  fwht_stage<32>(y, lane);
  for (int i = 0; i < 4; i++) y[i] = y[i] * 0.0625f;
}

// The inverse rotation of the attention output, split in two factors
// (H = H_hi H_lo, the butterflies of strides 64 and 128, and of strides
// 1 .. 32; the factors commute, and the output needs it only to within its
// tolerance, not bit for bit):
//   fwht_hi_x2: strides 64 and 128 (lane strides 16 and 32) on two rows of
//     4 dims per lane, no scaling -- applied to each split partial;
//   fwht_lo16: strides 1 .. 32 and the 1/16 scale on a 64-dim slice held by
//     the 16 lanes of one row (lane l: dims 4l .. 4l + 3 of the slice) --
//     applied once to each combined output slice.
__device__ __forceinline__ void fwht_hi_x2(float y[4], float z[4], int lane) {
  float w[8] = {y[0], y[1], y[2], y[3], z[0], z[1], z[2], z[3]};
  fwht_stage8<16>(w, lane);
  fwht_stage8<32>(w, lane);
  for (int i = 0; i < 4; i++) {
    y[i] = w[i];
    z[i] = w[4 + i];
  }
}
__device__ __forceinline__ void fwht_hi(float y[4], int lane) {
  fwht_stage<16>(y, lane);
  fwht_stage<32>(y, lane);
}
__device__ __forceinline__ void fwht_lo16(float y[4], int lane) {
#pragma clang fp contract(off)
  float a, b;
  a = y[0]; b = y[1]; y[0] = a + b; y[1] = a - b;
  a = y[2]; b = y[3]; y[2] = a + b; y[3] = a - b;
  a = y[0]; b = y[2]; y[0] = a + b; y[2] = a - b;
  a = y[1]; b = y[3]; y[1] = a + b; y[3] = a - b;
  fwht_stage<1>(y, lane);
  fwht_stage<2>(y, lane);
  fwht_stage<4>(y, lane);
  fwht_stage<8>(y, lane);
  for (int i = 0; i < 4; i++) y[i] = y[i] * 0.0625f;
}

}  // namespace k8v4
