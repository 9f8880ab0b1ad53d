// Quantizer rules of the k8v4 cache, one wave per (token, KV head) with 4
// dims per lane ("#120 --kv k8v4: hybrid KV cache -- INT8 K + Hadamard-
// rotated Q4_0 V (816 B/cell)", What/How): shared by the append kernel and
// the fused append of the decode kernel, so both write the same bytes.
// Every quantizer step is one IEEE fp32 operation rounded as written (the
// functions disable contraction locally, so x * r + 8.5 is never fused).
#pragma once

#include "device.hpp"

namespace k8v4 {

__device__ __forceinline__ void load4(const void *base, int dtype, size_t idx, float x[4]) {
  if (dtype == 0) {
    const u32x2 w = *reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint16_t *>(base) + idx);
    x[0] = f16_bits_to_f32((uint16_t)(w.x & 0xffff));
    x[1] = f16_bits_to_f32((uint16_t)(w.x >> 16));
    x[2] = f16_bits_to_f32((uint16_t)(w.y & 0xffff));
    x[3] = f16_bits_to_f32((uint16_t)(w.y >> 16));
  } else {
    const f32x4 w = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(base) + idx);
    x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
  }
}

// INT8 rule on the 4 values of this lane; lanes 0-31 form group 0 (dims
// 0..127), lanes 32-63 group 1.  Returns 4 packed codes and the scale.
__device__ __forceinline__ uint32_t quant_k(const float x[4], float &d_out) {
#pragma clang fp contract(off)
  float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
  amax = fmaxf(amax, lane_xor<16>(amax));
  amax = fmaxf(amax, lane_xor<8>(amax));
  amax = fmaxf(amax, lane_xor<4>(amax));
  amax = fmaxf(amax, lane_xor<2>(amax));
  amax = fmaxf(amax, lane_xor<1>(amax));
  const float d = amax / 127.0f;                 // correctly rounded division
  const float r = (d != 0.0f) ? 1.0f / d : 0.0f;
  uint32_t packed = 0;
  for (int i = 0; i < 4; i++) {
    float q = __builtin_rintf(x[i] * r);         // v_rndne_f32: nearest, ties to even
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    packed |= ((uint32_t)(int)q & 0xffu) << (8 * i);
  }
  d_out = d;
  return packed;
}

// Q4_0 rule on a 32-block spread over 8 lanes (4 values each).  Returns the
// 4 codes of this lane packed as bytes and the fp16 scale bits.
__device__ __forceinline__ uint32_t quant_q4(const float y[4], int lane, uint16_t &d16) {
#pragma clang fp contract(off)
  // value of largest magnitude, first index on ties
  int bi = 0;
  float bm = fabsf(y[0]);
  for (int i = 1; i < 4; i++) {
    const float a = fabsf(y[i]);
    if (a > bm) { bm = a; bi = i; }
  }
  float bv = y[bi];
  int bidx = 4 * (lane & 7) + bi;
  auto take = [&](float om, float ov, int oi) {
    if (om > bm || (om == bm && oi < bidx)) { bm = om; bv = ov; bidx = oi; }
  };
  take(lane_xor<1>(bm), lane_xor<1>(bv), lane_xor<1>(bidx));
  take(lane_xor<2>(bm), lane_xor<2>(bv), lane_xor<2>(bidx));
  take(lane_xor<4>(bm), lane_xor<4>(bv), lane_xor<4>(bidx));
  const float d = bv / -8.0f;
  const float r = (d != 0.0f) ? 1.0f / d : 0.0f;
  uint32_t codes = 0;
  for (int i = 0; i < 4; i++) {
    const float t = y[i] * r;
    const float u = t + 8.5f;
    int c = (int)u;                              // v_cvt_i32_f32 truncates toward zero
    c = c > 15 ? 15 : c;
    codes |= (uint32_t)c << (8 * i);
  }
  // d is pinned as its own value first: otherwise the compiler may fold the
  // multiply by -1/8 and the conversion into one mixed fma (x * y + 0),
  // which turns the -0 scale of an all-zero block into +0
  float dp = d;
  asm volatile("" : "+v"(dp));
  d16 = f32_to_f16_bits(dp);
  return codes;
}

// Byte of codes 4 lane .. 4 lane + 3 of head-cell `cell` in the K-code run:
// every 16 head-cells form a 4 KB block [dim quarter][cell % 16][64 codes],
// so the attention kernels' 16-byte operand loads (16 cells x 64 dims per
// instruction) each read 1 KB of consecutive bytes.  (The page size is a
// multiple of 16, so a block never straddles two (page, head) tiles.)
__device__ __forceinline__ size_t k_code_off(size_t cell, int lane) {
  return (cell >> 4) * 4096 + (size_t)(lane >> 4) * 1024 + (cell & 15) * 64 + (size_t)(lane & 15) * 4;
}

// fp16 format: K and V of every 16 head-cells are 8 KB blocks laid out as
// the attention kernel's MFMA operands (c = cell % 16):
//   K element d at (cell/16)*8192 + (d/32)*1024 + ((d%32)/8)*256 + c*16 + (d%8)*2
//   V element d at (cell/16)*8192 + ((d%16)/2)*1024 + (c/4)*256 + (d/16)*16
//                  + (d%2)*8 + (c%4)*2
// so every 16-byte load per lane of 16 cells reads 1 KB of consecutive bytes.
__device__ __forceinline__ size_t f16_k_off(size_t cell, int lane) {  // elements 4 lane .. 4 lane + 3
  const int d = 4 * lane;
  return (cell >> 4) * 8192 + (size_t)(d >> 5) * 1024 + (size_t)((d & 31) >> 3) * 256 + (cell & 15) * 16 +
         (size_t)(d & 7) * 2;
}
__device__ __forceinline__ size_t f16_v_off(size_t cell, int d) {
  const size_t c = cell & 15;
  return (cell >> 4) * 8192 + (size_t)((d & 15) >> 1) * 1024 + (c >> 2) * 256 + (size_t)(d >> 4) * 16 +
         (size_t)(d & 1) * 8 + (c & 3) * 2;
}
// one head's 256 values, 4 per lane (dims 4 lane ..), rounded to fp16
__device__ __forceinline__ void store_f16_k(uint8_t *run, size_t cell, int lane, const float x[4]) {
  uint16_t h[4];
  for (int e = 0; e < 4; e++) h[e] = f32_to_f16_bits(x[e]);
  *reinterpret_cast<u32x2 *>(run + f16_k_off(cell, lane)) =
      u32x2{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
}
__device__ __forceinline__ void store_f16_v(uint8_t *run, size_t cell, int lane, const float x[4]) {
  for (int e = 0; e < 4; e++)
    *reinterpret_cast<uint16_t *>(run + f16_v_off(cell, 4 * lane + e)) = f32_to_f16_bits(x[e]);
}

// INT8 half of one head: fp32 scales [cell][2]; codes in the K-code layout
// (KLAYOUT) or as a plain [cell][256] row (the int8 format's V)
template <bool KLAYOUT>
__device__ __forceinline__ void store_int8(uint8_t *codes_run, uint8_t *scales_run, size_t cell, int lane,
                                           uint32_t codes, float d) {
  *reinterpret_cast<uint32_t *>(codes_run + (KLAYOUT ? k_code_off(cell, lane) : cell * 256 + 4 * lane)) = codes;
  if ((lane & 31) == 0) reinterpret_cast<float *>(scales_run)[cell * 2 + (lane >> 5)] = d;
}

// Q4_0 half of one head into its (page, head) tile: byte i of a block =
// code[i] | code[i+16] << 4; lanes j < 4 of the block hold elements
// 4j..4j+3, lane j + 4 holds elements 16 + 4j..
__device__ __forceinline__ void store_q4(uint8_t *run, size_t tile, int P, int slot, int lane, uint32_t codes,
                                         uint16_t d16) {
  const uint32_t hi = (uint32_t)lane_xor<4>((int)codes);
  const int b = lane >> 3, j = lane & 7;
  uint8_t *vt = run + tile * 144 * P;
  if (j < 4) *reinterpret_cast<uint32_t *>(vt + (size_t)slot * 128 + b * 16 + 4 * j) = codes | (hi << 4);
  if (j == 0) *reinterpret_cast<uint16_t *>(vt + q4_scale_off(P, slot, b)) = d16;
}

}  // namespace k8v4
