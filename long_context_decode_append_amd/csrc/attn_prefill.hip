// Causal prefill-chunk attention over a paged pool, for gfx950.
//
// Computes, for n_new queries at positions [pos0, pos0 + n_new), the same
// attention as decode ("#120 --kv k8v4: hybrid KV cache -- INT8 K +
// Hadamard-rotated Q4_0 V (816 B/cell)", How: one fused attention serves
// decode, verify and prefill), row i attending cells [0, pos0 + i].  The
// pool may hold any of the four formats (k8v4; int8 K and V; rotated q4_0
// K and V, scored against the rotated query; fp16 K and V).
//
// Here Q.K^T and P.V are dense contractions (every K/V tile serves all
// query rows of a workgroup), so both run on the matrix cores with the
// 32 x 32 x 16 fp16 MFMA (fp32 accumulation).  A call is two kernels:
//   * staging: one workgroup per (32-cell tile, KV head) loads the tile's
//     raw pages once and writes its image to the workspace -- K [cell][dim]
//     as fp16 values already multiplied by softmax scale x log2 e (INT8
//     code * group scale, q4_0 (code - 8) * d16, fp16 as stored; formed in
//     fp32 and rounded once), V transposed [dim][cell] as (code - 8) * d16
//     or code * d, its cells ordered so that the P.V B-operand of a lane
//     (8 cells) is one 16-byte read.  Every attention workgroup of a KV head
//     reads the same tiles, so this is the dequantization they would
//     otherwise each repeat, and its scores need no scaling;
//   * attention: workgroup = 4 waves, one per SIMD, each owning 32 query
//     rows (4 positions x 8 GQA heads of one KV head; fp32 queries add an
//     MFMA on the fp16 rounding remainder), 128 rows per workgroup.  Five
//     32 KB LDS image buffers (the whole LDS): tile t + 3 is copied in with
//     direct global-to-LDS loads (no registers, no VALU) while tile t's P.V
//     and tile t + 1's Q.K^T run; one barrier per two tiles;
//   * S^T = K.Q^T puts a lane's query row in the column the P.V A-operand
//     needs, so P never leaves registers; online softmax in base 2 against a
//     lazily moved reference max; the causal mask only from the first tile
//     some row does not see whole; each tile step is hand-ordered (operand
//     reads eight MFMAs ahead, VALU work beside the MFMAs);
//   * epilogue: O / l and (rotated V) the inverse Walsh-Hadamard transform
//     in registers: a lane holds one dim of each 32-dim tile, so strides
//     1 .. 16 are cross-lane butterflies and 32 .. 128 in-register ones.
#include "device.hpp"
#include "launch.hpp"

namespace k8v4 {

constexpr int kPfWaves = 4;
constexpr int kPfTile = 32;                   // cells per tile
constexpr int kPfBufs = 5;                    // LDS tile buffers of the attention kernel
constexpr float kPfLazy = 8.0f;               // log2 headroom of the lazy softmax reference

// position of cell c (0..31) in the V order: the P.V B-operand of k-step s,
// lane half h takes cells 16 s + 8 a + 4 h + b (a in {0, 1}, b in 0..3) --
// the cells of that lane's scores -- stored side by side at 16 s + 8 h + 4 a
// + b (bits 2 and 3 of c swapped), so one 16-byte read fetches them
__device__ __forceinline__ int v_pos(int c) { return (c & 19) | ((c & 4) << 1) | ((c & 8) >> 1); }

// A staged tile (the LDS image the attention kernel computes from, copied
// there unchanged), fp16, in 16-byte chunks of 8 elements:
//   K: chunk (j, c) = dims 8 j .. 8 j + 7 of cell c, at chunk 32 j + c;
//   V: chunk (j, d) = dim d of the cells at V positions 8 j .. 8 j + 7, at
//      chunk 256 j + d.
// An operand read (16 bytes per lane) then has the 16 lanes of each LDS pass
// on 16 consecutive chunks -- every bank once, with no padding -- and the
// operands of a tile lie at fixed offsets from a lane's first one.
__device__ __forceinline__ int k_off(int c, int d) { return ((d >> 3) * kPfTile + c) * 8 + (d & 7); }
// V element of dim d at V position p, and of dim d and cell c
__device__ __forceinline__ int v_off_pos(int d, int p) { return ((p >> 3) * 256 + d) * 8 + (p & 7); }
__device__ __forceinline__ int v_off(int d, int c) { return v_off_pos(d, v_pos(c)); }
constexpr int kKElems = kPfTile * 256, kVElems = 256 * kPfTile;
constexpr int kPfImageBytes = 2 * (kKElems + kVElems);  // 32 KB
static_assert(kPfImageBytes % 1024 == 0, "whole 1 KB copy units");

struct PrefillArgs {
  const uint8_t *run[4];  // the pool's runs (format-dependent, as the header lays them out)
  const int32_t *pt;
  const void *q;
  float *out;
  int n_pages, P, H;
  int n_q_heads;
  int pos0, n_new;
  float scale2;           // softmax scale * log2(e)
  uint8_t *img;           // tile images [kv head][tile][kPfImageBytes] (the workspace)
  int n_tiles;            // tiles staged per KV head: ceil((pos0 + n_new) / 32)
};

// (x & m) | c in one VALU op (the compiler splits it when both are literals)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}

// Raw pages of one tile, in the registers of the thread that dequantizes
// them.  Work unit u in [0, 512), two per thread (u = tid and tid + 256); a
// unit's cells lie in half u / 256 of the tile, so every load of a wave
// reads one half (a wave-uniform base plus a fixed lane offset).  With
// i = u % 256:
//   INT8 K: 16 codes of cell 16 (u / 256) + i / 16, dims 16 (i % 16) ..
//   q4_0 K: bytes 8 (i % 2) .. + 7 of block (i % 16) / 2 of the same cell and
//           that block's fp16 scale
//   q4_0 V: bytes 4 (i / 64) .. + 3 of block (i / 8) % 8 of cells 2 j and
//           2 j + 1 of the half, j = i % 8, and the two blocks' scales
//   INT8 V: codes of dims 8 ((i / 8) % 32) .. + 7 of the same two cells, and
//           the two cells' scales of that 128-dim group
//   fp16 K: dims 16 (i % 16) .. + 15 of cell 16 (u / 256) + i / 16
//   fp16 V: 32 consecutive bytes of the half: chunks 2i and 2i + 1 of its
//           8 KB block, each 4 cells x 2 dims
//   INT8 K scale: that of the unit's cell and 128-dim group
// The loads are unconditional (every address lies in the pool: a half past
// the visible cells reads the last visible half again, a cell past them lies
// in its half's page); the values of cells past the visible ones are zeroed
// when stored, so the loads can be issued a tile ahead and consumed a tile
// later.
struct PfRaw {
  u32x4 k;          // INT8 K: 16 codes; q4_0 K: .x .y nibble bytes, .z scale; fp16 K: dims 0 .. 7
  u32x4 k2;         // fp16 K: dims 8 .. 15 of the unit
  float ks;         // INT8 K: the unit's group scale as stored
  u32x2 va, vb;     // V of the two cells (q4_0: .x only)
  uint32_t vd;      // q4_0 V: the two fp16 scales (lo: first cell)
  float vsa, vsb;   // INT8 V: the two cells' scales
  u32x4 v16[2];     // fp16 V: the unit's two 16-byte chunks
};

// Per tile: the physical (page, head) tile of each 16-cell half (P is a
// multiple of 16 and tiles start at multiples of 32, so a half never
// straddles a page) and the slot of its first cell; wave-uniform.
struct PfHalves {
  int tile[2];
  int slot0[2];
  int bad;  // bit i: half i's page-table entry is out of range (page 0 is read instead)
  int P;
  // first cell of half hf in the pool's cell order (a select: hf varies by lane)
  __device__ __forceinline__ size_t cell(int hf) const {
    return hf ? (size_t)tile[1] * P + slot0[1] : (size_t)tile[0] * P + slot0[0];
  }
  __device__ __forceinline__ int tile_of(int hf) const { return hf ? tile[1] : tile[0]; }
  __device__ __forceinline__ int slot_of(int hf) const { return hf ? slot0[1] : slot0[0]; }
};

__device__ __forceinline__ PfHalves pf_halves(const PrefillArgs &a, int g, int c0, int n_cells) {
  PfHalves h;
  h.P = a.P;
  h.bad = 0;
  // a half past the visible cells reads the last visible half again (no
  // branch: the page-table entries past the visible cells are never read)
  const int c_max = (n_cells - 1) & ~15;
  for (int i = 0; i < 2; i++) {
    const int c = min(c0 + 16 * i, c_max);
    const int pidx = (int)((unsigned)c / (unsigned)a.P);
    int page = a.pt[pidx];
    const bool bad = page < 0 || page >= a.n_pages;
    h.bad |= (bad && c0 + 16 * i < n_cells) ? (1 << i) : 0;
    page = bad ? 0 : page;
    h.tile[i] = page * a.H + g;
    h.slot0[i] = c - pidx * a.P;
  }
  return h;
}

template <int FMT, int HF>
__device__ __forceinline__ void pf_load(const PrefillArgs &a, const PfHalves &hv, int tid, PfRaw &r) {
  const int i = tid;  // unit u = tid + 256 HF
  const size_t cell0 = (size_t)hv.tile[HF] * a.P + hv.slot0[HF];  // first cell of the half, pool order
  if (FMT == KV_FMT_F16) {
    // fp16 blocks: 8 KB per 16 cells in each of K and V, the layout the
    // decode kernel loads as MFMA operands
    const int m = i & 15;
    const uint8_t *kb = a.run[0] + cell0 * 512;
    const uint32_t ko = (uint32_t)((m >> 1) * 1024 + (m & 1) * 512 + ((i >> 4) & 15) * 16);
    r.k = *reinterpret_cast<const u32x4 *>(kb + ko);
    r.k2 = *reinterpret_cast<const u32x4 *>(kb + ko + 256);
    const uint8_t *vb = a.run[2] + cell0 * 512;
    r.v16[0] = *reinterpret_cast<const u32x4 *>(vb + 32u * (uint32_t)i);
    r.v16[1] = *reinterpret_cast<const u32x4 *>(vb + 32u * (uint32_t)i + 16u);
    return;
  }
  const uint8_t *tile_base = a.run[0] + (size_t)hv.tile[HF] * 144 * a.P;  // q4_0 K tile of the half
  if (FMT != KV_FMT_Q4_0) {
    // K-code run: 4 KB per 16 cells, [dim quarter][cell % 16][64 codes];
    // a wave's 64 units read four 256-byte stretches
    const int m = i & 15;
    const uint32_t ko = (uint32_t)((m >> 2) * 1024 + ((i >> 4) & 15) * 64 + 16 * (m & 3));
    r.k = *reinterpret_cast<const u32x4 *>(a.run[0] + cell0 * 256 + ko);
  } else {
    const int b = (i & 15) >> 1, hh = i & 1, c = (i >> 4) & 15;
    const uint8_t *kt = tile_base + (size_t)hv.slot0[HF] * 128;
    const u32x2 w = *reinterpret_cast<const u32x2 *>(kt + (uint32_t)(c * 128 + 16 * b + 8 * hh));
    r.k.x = w.x;
    r.k.y = w.y;
    r.k.z = *reinterpret_cast<const uint16_t *>(tile_base + q4_scale_off(a.P, hv.slot0[HF], 0) +
                                                (uint32_t)(b * 32 + c * 2));
  }
  if (FMT != KV_FMT_Q4_0)  // [cell][group] floats in pool order
    r.ks = reinterpret_cast<const float *>(a.run[1])[(cell0 + ((i >> 4) & 15)) * 2 + ((i & 15) >> 3)];
  const int j = i & 7;  // cells 2 j, 2 j + 1 of the half
  if (FMT != KV_FMT_INT8) {
    const int b = (i >> 3) & 7, qq = i >> 6;
    const uint8_t *vt = a.run[2] + (size_t)hv.tile[HF] * 144 * a.P;
    const uint8_t *vs = vt + (size_t)hv.slot0[HF] * 128;
    const uint32_t vo = (uint32_t)(2 * j * 128 + 16 * b + 4 * qq);
    r.va.x = *reinterpret_cast<const uint32_t *>(vs + vo);
    r.vb.x = *reinterpret_cast<const uint32_t *>(vs + vo + 128);
    // the two cells' block-b scales are one aligned word
    r.vd = *reinterpret_cast<const uint32_t *>(vt + q4_scale_off(a.P, hv.slot0[HF], 0) + (uint32_t)(b * 32 + 4 * j));
  } else {
    const int dg = (i >> 3) & 31;  // dims 8 dg .. 8 dg + 7, scale group dg / 16
    const uint8_t *vc = a.run[2] + cell0 * 256;
    const float *vsc = reinterpret_cast<const float *>(a.run[3]) + cell0 * 2;
    r.va = *reinterpret_cast<const u32x2 *>(vc + (uint32_t)(2 * j * 256 + 8 * dg));
    r.vb = *reinterpret_cast<const u32x2 *>(vc + (uint32_t)((2 * j + 1) * 256 + 8 * dg));
    r.vsa = vsc[(2 * j) * 2 + (dg >> 4)];
    r.vsb = vsc[(2 * j + 1) * 2 + (dg >> 4)];
  }
}

// Four nibble bytes -> the 4 low-nibble and the 4 high-nibble values
// (code - 8) * d, as fp16 pairs in byte order
__device__ __forceinline__ void q4_word_to_f16(uint32_t w, f16x2 d, uint32_t lo[2], uint32_t hi[2]) {
  const f16x2 c1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2 c72 = {(_Float16)72.0f, (_Float16)72.0f};
  for (int p = 0; p < 2; p++) {
    // [byte 2p, 0, byte 2p + 1, 0]
    const uint32_t x = perm(0u, w, (0x0cu << 24) | ((2u * p + 1u) << 16) | (0x0cu << 8) | (2u * p));
    lo[p] = as_u32((as_f16x2(and_or(x, 0x000F000Fu, 0x64006400u)) - c1032) * d);
    hi[p] = as_u32((as_f16x2(and_or(x, 0x00F000F0u, 0x54005400u)) - c72) * d);
  }
}

// an fp16 pair times f, formed in fp32 and rounded once
__device__ __forceinline__ uint32_t f16x2_scaled(uint32_t w, float f) {
  const f16x2 h = as_f16x2(w);
  const f16x2 y = {(_Float16)((float)h[0] * f), (_Float16)((float)h[1] * f)};
  return as_u32(y);
}

// Dequantize work unit u of the tile at c0 into its tile image (K times
// softmax scale x log2 e at k_off, V at v_off).  Cells
// at or past n_cells store zero K and V; the K of a half whose page-table
// entry is out of range (bad) is NaN, so rows that reach it return NaN and
// rows that stop before it mask it.
template <int FMT, int HF>
__device__ __forceinline__ void pf_store(const PfRaw &r, int tid, int c0, int n_cells, bool bad, float scale2,
                                         _Float16 *lk, _Float16 *lv) {
  const int u = tid + 256 * HF, i = tid;
  const int cl = u >> 4;
  const bool k_ok = c0 + cl < n_cells;
  const float kf_nan = __builtin_nanf("");
  if (FMT == KV_FMT_F16) {
    // K: dims 16 (u % 16) .. + 15 of cell u / 16; V: chunk (uu, lq, nn)
    // holds dims 16 nn + 2 uu (+1) of cells 4 lq .. 4 lq + 3 of its half,
    // which sit side by side in a V chunk (v_pos)
    const float f = !k_ok ? 0.f : bad ? kf_nan : scale2;
    const uint32_t kw[8] = {r.k.x, r.k.y, r.k.z, r.k.w, r.k2.x, r.k2.y, r.k2.z, r.k2.w};
    uint32_t kf[8];
    for (int e = 0; e < 8; e++) kf[e] = f16x2_scaled(kw[e], f);
    *reinterpret_cast<u32x4 *>(lk + k_off(cl, 16 * (u & 15))) = u32x4{kf[0], kf[1], kf[2], kf[3]};
    *reinterpret_cast<u32x4 *>(lk + k_off(cl, 16 * (u & 15) + 8)) = u32x4{kf[4], kf[5], kf[6], kf[7]};
    const int vh = u >> 8, idx = u & 255;
    const int uu = idx >> 5, lq = (idx >> 3) & 3;
    const int cq = c0 + 16 * vh + 4 * lq;
    const uint32_t m01 = (cq < n_cells ? 0x0000ffffu : 0u) | (cq + 1 < n_cells ? 0xffff0000u : 0u);
    const uint32_t m23 = (cq + 2 < n_cells ? 0x0000ffffu : 0u) | (cq + 3 < n_cells ? 0xffff0000u : 0u);
    for (int q = 0; q < 2; q++) {
      const int d = 16 * (2 * (idx & 7) + q) + 2 * uu;
      *reinterpret_cast<u32x2 *>(lv + v_off(d, 16 * vh + 4 * lq)) = u32x2{r.v16[q].x & m01, r.v16[q].y & m23};
      *reinterpret_cast<u32x2 *>(lv + v_off(d + 1, 16 * vh + 4 * lq)) = u32x2{r.v16[q].z & m01, r.v16[q].w & m23};
    }
    return;
  }
  if (FMT != KV_FMT_Q4_0) {
    // INT8 K -> code * scale * scale2 (the codes are exact in fp16 on the
    // way): dims 16 (u % 16) .. + 15 of cell u / 16
    const f16x2 c1152 = {(_Float16)1152.0f, (_Float16)1152.0f};
    const float f = !k_ok ? 0.f : bad ? kf_nan : r.ks * scale2;
    uint32_t kf[8];
    const uint32_t kw[4] = {r.k.x, r.k.y, r.k.z, r.k.w};
    for (int i = 0; i < 4; i++) {
      uint32_t lo, hi;
      i8x4_to_f16_biased(kw[i], lo, hi);
      kf[2 * i] = f16x2_scaled(as_u32(as_f16x2(lo) - c1152), f);
      kf[2 * i + 1] = f16x2_scaled(as_u32(as_f16x2(hi) - c1152), f);
    }
    *reinterpret_cast<u32x4 *>(lk + k_off(cl, 16 * (u & 15))) = u32x4{kf[0], kf[1], kf[2], kf[3]};
    *reinterpret_cast<u32x4 *>(lk + k_off(cl, 16 * (u & 15) + 8)) = u32x4{kf[4], kf[5], kf[6], kf[7]};
  } else {
    // q4_0 K -> (code - 8) * d16 * scale2: elements 8hh .. 8hh + 7 (low
    // nibbles) and 16 + 8hh .. (high nibbles) of block b (code - 8 is exact
    // in fp16 on the way)
    const int b = (u & 15) >> 1, hh = u & 1;
    const float f = !k_ok ? 0.f : bad ? kf_nan : f16_bits_to_f32((uint16_t)(r.k.z & 0xFFFFu)) * scale2;
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    uint32_t lo[4], hi[4];
    q4_word_to_f16(r.k.x, one, lo, hi);
    q4_word_to_f16(r.k.y, one, lo + 2, hi + 2);
    for (int e = 0; e < 4; e++) {
      lo[e] = f16x2_scaled(lo[e], f);
      hi[e] = f16x2_scaled(hi[e], f);
    }
    *reinterpret_cast<u32x4 *>(lk + k_off(cl, 32 * b + 8 * hh)) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    *reinterpret_cast<u32x4 *>(lk + k_off(cl, 32 * b + 16 + 8 * hh)) = u32x4{hi[0], hi[1], hi[2], hi[3]};
  }
  const int cp = 8 * HF + (i & 7);  // cells 2 cp, 2 cp + 1 of the tile
  const bool ok_a = c0 + 2 * cp < n_cells, ok_b = c0 + 2 * cp + 1 < n_cells;
  if (FMT != KV_FMT_INT8) {
    // q4_0 V -> (code - 8) * d16, transposed [dim][cell]; byte i of the block
    // holds element i (low nibble) and element 16 + i (high nibble); a cell
    // past the visible ones gets scale 0 (its slot may hold any bits)
    const f16x2 c1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const f16x2 c72 = {(_Float16)72.0f, (_Float16)72.0f};
    const int b = (i >> 3) & 7, qq = i >> 6;
    const f16x2 dd = as_f16x2(r.vd & ((ok_a ? 0x0000FFFFu : 0u) | (ok_b ? 0xFFFF0000u : 0u)));
    for (int e = 0; e < 4; e++) {
      // [a.byte, 0, b.byte, 0] for byte e of each cell: elements 4qq + e
      // (low nibbles) and 16 + 4qq + e (high nibbles)
      const uint32_t sel = (0x0cu << 24) | ((4u + e) << 16) | (0x0cu << 8) | (uint32_t)e;
      const uint32_t x = perm(r.vb.x, r.va.x, sel);
      const uint32_t lo = as_u32((as_f16x2(and_or(x, 0x000F000Fu, 0x64006400u)) - c1032) * dd);
      const uint32_t hi = as_u32((as_f16x2(and_or(x, 0x00F000F0u, 0x54005400u)) - c72) * dd);
      *reinterpret_cast<uint32_t *>(lv + v_off(32 * b + 4 * qq + e, 2 * cp)) = lo;
      *reinterpret_cast<uint32_t *>(lv + v_off(32 * b + 16 + 4 * qq + e, 2 * cp)) = hi;
    }
  } else {
    // INT8 V -> code * d rounded to fp16, transposed [dim][cell]
    const int dg = (i >> 3) & 31;
    const float sa = ok_a ? r.vsa : 0.f, sb = ok_b ? r.vsb : 0.f;
    const uint32_t wa[2] = {r.va.x, r.va.y}, wb[2] = {r.vb.x, r.vb.y};
    for (int e = 0; e < 8; e++) {
      const float xa = (float)(int8_t)(wa[e >> 2] >> (8 * (e & 3))) * sa;
      const float xb = (float)(int8_t)(wb[e >> 2] >> (8 * (e & 3))) * sb;
      const f16x2 pr = {(_Float16)xa, (_Float16)xb};
      *reinterpret_cast<uint32_t *>(lv + v_off(8 * dg + e, 2 * cp)) = as_u32(pr);
    }
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// value of the lane whose id is src (a cross-lane read through the LDS
// crossbar; used outside the per-tile path only)
__device__ __forceinline__ float lane_at(float x, int src) { return __shfl(x, src, 64); }

// instruction classes of the scheduling-group hints
// Staging: one workgroup per (tile, KV head) loads the tile's raw pages and
// writes its image (the dequantization every attention workgroup of that
// head would otherwise repeat).  Cells at or past n_cells = pos0 + n_new
// are zero.
template <int FMT>
__global__ __launch_bounds__(256) void prefill_stage_kernel(const PrefillArgs a) {
  const int t = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int c0 = t * kPfTile, n_cells = a.pos0 + a.n_new;
  const PfHalves hv = pf_halves(a, g, c0, n_cells);
  PfRaw r0, r1;
  pf_load<FMT, 0>(a, hv, tid, r0);
  pf_load<FMT, 1>(a, hv, tid, r1);
  uint8_t *im = a.img + ((size_t)g * a.n_tiles + t) * kPfImageBytes;
  _Float16 *lk = reinterpret_cast<_Float16 *>(im), *lv = lk + kKElems;
  pf_store<FMT, 0>(r0, tid, c0, n_cells, hv.bad & 1, a.scale2, lk, lv);
  pf_store<FMT, 1>(r1, tid, c0, n_cells, (hv.bad >> 1) & 1, a.scale2, lk, lv);
}

template <bool QF32, int FMT>
__global__ __launch_bounds__(kPfWaves * 64, 1) void attn_prefill_kernel(const PrefillArgs a) {
  constexpr int kPos = kPfWaves * 32 / kGqa;          // query positions per workgroup
  constexpr bool kRotV = FMT == KV_FMT_Q4_0 || FMT == KV_FMT_K8V4;
  __shared__ __attribute__((aligned(16))) uint8_t lds_img[kPfBufs * kPfImageBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, h = lane >> 5;
  const int g = blockIdx.y;
  const int qb0 = blockIdx.x * kPos;                  // first query (chunk-relative)
  const int q_last = min(qb0 + kPos, a.n_new) - 1;    // last valid query of the block
  const int n_cells = a.pos0 + q_last + 1;            // cells any row of the block sees
  const int wpos0 = qb0 + 4 * wave;                   // this wave's first query position

  // ---- queries.  Row R = col of the wave: position wpos0 + R / 8, head
  // 8 g + R % 8.  B operand of S^T = K.Q^T for k-step kk (16 dims): lane
  // (col, h) holds dims 16 kk + 8 h .. + 7 of row col.  q4_0 scores against
  // rotated keys, so the row is rotated first (q~ = H q / 16): dim bit 3 is
  // the lane half, the others are in registers.
  const int qi = wpos0 + (col >> 3);
  const bool qvalid = qi <= q_last;
  const int qpos = a.pos0 + qi;
  float qv[16][8];
  {
    const size_t qbase = ((size_t)qi * a.n_q_heads + (size_t)g * kGqa + (col & 7)) * 256;
    for (int kk = 0; kk < 16; kk++) {
      const int d0 = 16 * kk + 8 * h;
      if (!QF32) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (qvalid) w = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.q) + qbase + d0);
        const f16x8 hv = __builtin_bit_cast(f16x8, w);
        for (int e = 0; e < 8; e++) qv[kk][e] = (float)hv[e];
      } else {
        f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
        if (qvalid) {
          x0 = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(a.q) + qbase + d0);
          x1 = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(a.q) + qbase + d0 + 4);
        }
        for (int e = 0; e < 4; e++) {
          qv[kk][e] = x0[e];
          qv[kk][4 + e] = x1[e];
        }
      }
    }
  }
  if (FMT == KV_FMT_Q4_0) {
    for (int kk = 0; kk < 16; kk++)
      for (int st = 1; st < 8; st <<= 1)
        for (int e = 0; e < 8; e++)
          if (!(e & st)) {
            const float x = qv[kk][e], y = qv[kk][e + st];
            qv[kk][e] = x + y;
            qv[kk][e + st] = x - y;
          }
    const uint32_t neg = h ? 0x80000000u : 0u;
    for (int kk = 0; kk < 16; kk++)
      for (int e = 0; e < 8; e++) qv[kk][e] = fwht_pair<32>(qv[kk][e], neg);
    for (int st = 1; st < 16; st <<= 1)
      for (int kk = 0; kk < 16; kk++)
        if (!(kk & st))
          for (int e = 0; e < 8; e++) {
            const float x = qv[kk][e], y = qv[kk + st][e];
            qv[kk][e] = x + y;
            qv[kk + st][e] = x - y;
          }
    for (int kk = 0; kk < 16; kk++)
      for (int e = 0; e < 8; e++) qv[kk][e] *= 0.0625f;
  }
  // fp16 operand; fp32 queries add a second MFMA on the rounding remainder
  f16x8 qop[16], qlo[QF32 ? 16 : 1];
  for (int kk = 0; kk < 16; kk++)
    for (int e = 0; e < 8; e++) {
      const _Float16 hv = (_Float16)qv[kk][e];
      qop[kk][e] = hv;
      if (QF32) qlo[kk][e] = (_Float16)(qv[kk][e] - (float)hv);
    }

  float m = -1e30f, lsum = 0.f;
  f32x16 o[8];
  for (int jd = 0; jd < 8; jd++)
    for (int e = 0; e < 16; e++) o[jd][e] = 0.f;

  auto kbuf = [&](int b) { return reinterpret_cast<const _Float16 *>(lds_img + b * kPfImageBytes); };
  // Copy tile t's image into buffer b: 1 KB per wave and instruction straight
  // into LDS (lane l's 16 bytes land at 16 l), no registers; chunk r of a
  // wave is the image's KB 4 r + wave (32 KB: 8 rounds).  A tile past the
  // staged ones (a pair's second tile, masked out whole) copies the last one.
  constexpr int kCopyRounds = kPfImageBytes / 1024 / kPfWaves;
  static_assert(kCopyRounds * kPfWaves * 1024 == kPfImageBytes, "whole rounds");
  const uint8_t *img_head = a.img + (size_t)g * a.n_tiles * kPfImageBytes + wave * 1024 + lane * 16;
  auto copy_chunk = [&](int b, int t, int r) {
    const uint8_t *src = img_head + (size_t)min(t, a.n_tiles - 1) * kPfImageBytes + r * kPfWaves * 1024;
    uint8_t *dst = lds_img + b * kPfImageBytes + wave * 1024 + r * kPfWaves * 1024;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(src),
                                     (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
  };
  auto copy_tile = [&](int b, int t) {
    for (int r = 0; r < kCopyRounds; r++) copy_chunk(b, t, r);
  };
  // the copies issued so far have landed (each wave waits for its own; the
  // barrier that follows makes every wave's visible)
  auto copies_done = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  // S^T = K.Q^T of the tile in buffer b: its 16 K operands, then 16 (fp32
  // queries: 32) MFMAs.  The image's K carries the softmax scale (times
  // log2 e), so these are the base-2 scores.  This lane's scores are row
  // col, cells 8 (e / 4) + 4 h + e % 4 of a tile (element e of the 32 x 32
  // accumulator).
  auto k_operands = [&](int b, f16x8 (&kop)[16]) {
    const _Float16 *kr = kbuf(b) + k_off(col, 8 * h);
    for (int kk = 0; kk < 16; kk++) kop[kk] = *reinterpret_cast<const f16x8 *>(kr + k_off(0, 16 * kk));
  };
  auto qk = [&](const f16x8 (&kop)[16], f32x16 &acc) {
    for (int e = 0; e < 16; e++) acc[e] = 0.f;
    for (int kk = 0; kk < 16; kk++) {
      acc = mfma32(kop[kk], qop[kk], acc);
      if (QF32) acc = mfma32(kop[kk], qlo[kk], acc);
    }
  };
  // tile u's cells past a row's position (and every cell of an invalid row)
  // to -inf -- needed from the first tile some row does not see whole on
  auto mask = [&](int u, float (&sc)[16]) {
    for (int e = 0; e < 16; e++) {
      const int cell = u * kPfTile + 8 * (e >> 2) + 4 * h + (e & 3);
      sc[e] = (qvalid && cell <= qpos) ? sc[e] : -INFINITY;
    }
  };
  auto lane_max = [](const float (&sc)[16]) {
    float mx = sc[0];
    for (int e = 1; e < 16; e++) mx = fmaxf(mx, sc[e]);
    return mx;
  };
  // a row's max: the maxima of the lane pair that holds its scores
  auto pair_max = [](float mx) { return fmaxf(mx, lane_xor<32>(mx)); };

  // One step of the pipeline, for tile t held in buffer b0 (the next tile in
  // b1), with this tile's masked scores in `cur` and their row max in mx_cur:
  // the copy of tile t + 3 into b3 is issued (one chunk per section); the
  // next tile's scores are computed (into `nxt`, mx_nxt) on the MFMAs while
  // this tile's exponentials run on the VALU; then O += P.V, beside it this
  // tile's row sum and the next tile's row max.  The sections are
  // hand-ordered (scheduling fences), each with one MFMA, the LDS read of an
  // operand eight MFMAs ahead and a little VALU work: the compiler otherwise
  // reads each operand just before its MFMA and waits out the LDS latency
  // every time, and gathers the sum and max chains after the last MFMA (an
  // empty asm statement that takes them as inputs keeps each link in its
  // section).  Tiles t .. t + 4 sit in five buffers, tile i in buffer i % 5.
  // Steps run in pairs (t even, t + 1) with one barrier, after the pair, once
  // each wave's copies have landed: the pair reads tiles t .. t + 2, all
  // copied before the previous barrier, and writes tiles t + 3 and t + 4
  // over tiles t - 2 and t - 1, last read before it.
  const int n_tiles = (n_cells + kPfTile - 1) / kPfTile;
  const int n_full = ((a.pos0 + qb0 + 1) / kPfTile) & ~1;  // tiles every row sees whole, even
  const int n_end = n_full + ((n_tiles - n_full + 1) & ~1);
  auto step = [&](int t, int b0, int b1, int b3, const float (&cur)[16], float mx_cur, float (&nxt)[16],
                  float &mx_nxt, bool pair_end) {
    // the reference max moves (for every row, to at least its max) only when
    // some row's max exceeds it by more than 2^kPfLazy
    if (__any(mx_cur > m + kPfLazy)) {
      const float mnew = fmaxf(m, mx_cur);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      lsum *= alpha;
      m = mnew;
      // O rows of element e: 8 (e / 4) + 4 h + e % 4; their factor lives in
      // the lanes whose column is that row
      for (int e = 0; e < 16; e++) {
        const float al = lane_at(alpha, 8 * (e >> 2) + 4 * h + (e & 3));
        for (int jd = 0; jd < 8; jd++) o[jd][e] *= al;
      }
    }
    // K operand i: dims 16 i + 8 h .. of cell col (tile t + 1); V operand
    // i = 8 st + jd: dim 32 jd + col, the lane half's 8 cells of k-step st
    f16x8 kop[16], vop[16];
    const _Float16 *kr = kbuf(b1) + k_off(col, 8 * h);
    const _Float16 *lv = kbuf(b0) + kKElems + v_off_pos(col, 8 * h);
    auto rd_k = [&](int i) { kop[i] = *reinterpret_cast<const f16x8 *>(kr + k_off(0, 16 * i)); };
    auto rd_v = [&](int i) {
      vop[i] = *reinterpret_cast<const f16x8 *>(lv + v_off_pos(32 * (i & 7), 16 * (i >> 3)));
    };
    f32x16 acc;
    for (int e = 0; e < 16; e++) acc[e] = 0.f;
    f16x8 pop[2];
    float pv[16];
    for (int i = 0; i < 8; i++) rd_k(i);
    __builtin_amdgcn_sched_barrier(0);
    // the next tile's scores; this tile's probabilities
    for (int i = 0; i < 16; i++) {
      acc = mfma32(kop[i], qop[i], acc);
      if (QF32) acc = mfma32(kop[i], qlo[i], acc);
      if (i + 8 < 16) rd_k(i + 8);
      else rd_v(i - 8);
      if (i < kCopyRounds) copy_chunk(b3, t + 3, i);  // tile t + 3, one KB per wave
      pv[i] = __builtin_amdgcn_exp2f(cur[i] - m);
      pop[i >> 3][i & 7] = (_Float16)pv[i];
      __builtin_amdgcn_sched_barrier(0);
    }
    // this tile's O += P.V; its row sum; the next tile's row max (unmasked;
    // the scores are read two MFMAs after the last Q.K^T one was issued)
    float ps = 0.f, mx = -INFINITY;
    for (int i = 0; i < 16; i++) {
      o[i & 7] = mfma32(pop[i >> 3], vop[i], o[i & 7]);
      if (i + 8 < 16) rd_v(i + 8);
      ps += pv[i];
      nxt[i] = acc[i];
      if (i >= 2) mx = fmaxf(mx, acc[i - 2]);
      asm volatile("" ::"v"(ps), "v"(mx));
      __builtin_amdgcn_sched_barrier(0);
    }
    mx = fmaxf(mx, fmaxf(acc[14], acc[15]));
    lsum += ps;
    if (t + 1 >= n_full) {
      mask(t + 1, nxt);
      mx = lane_max(nxt);
    }
    mx_nxt = pair_max(mx);
    if (pair_end) {
      copies_done();
      __syncthreads();
    }
  };

  // Prologue: tiles 0 .. 2 copied, tile 0's scores computed.  The loop takes
  // tiles in pairs (the score registers swap roles), past the visible cells
  // if need be (such a tile is masked out whole; its copy repeats the last
  // staged tile).
  copy_tile(0, 0);
  copy_tile(1, 1);
  copy_tile(2, 2);
  copies_done();
  __syncthreads();
  float sa[16], sb[16], mxa, mxb;
  {
    f16x8 kop[16];
    f32x16 acc;
    k_operands(0, kop);
    qk(kop, acc);
    for (int e = 0; e < 16; e++) sa[e] = acc[e];
    if (0 >= n_full) mask(0, sa);
    mxa = pair_max(lane_max(sa));
  }
  auto buf = [](int t) { return t % kPfBufs; };
  for (int t = 0; t < n_end; t += 2) {
    step(t, buf(t), buf(t + 1), buf(t + 3), sa, mxa, sb, mxb, false);
    step(t + 1, buf(t + 1), buf(t + 2), buf(t + 4), sb, mxb, sa, mxa, true);
  }

  // ---------------- epilogue: O / l; the lane holds dim 32 jd + col of rows
  // 8 (e / 4) + 4 h + e % 4
  const float lt = lsum + lane_xor<32>(lsum);  // row col's total
  for (int e = 0; e < 16; e++) {
    const int r = 8 * (e >> 2) + 4 * h + (e & 3);
    const float inv = 1.0f / lane_at(lt, r);
    float y[8];
    for (int jd = 0; jd < 8; jd++) y[jd] = o[jd][e] * inv;
    if (kRotV) {
      // inverse rotation of the row: strides 32, 64, 128 in registers,
      // 1 .. 16 across the 32 lanes of the half
      for (int st = 1; st < 8; st <<= 1)
        for (int jd = 0; jd < 8; jd++)
          if (!(jd & st)) {
            const float x = y[jd], z = y[jd + st];
            y[jd] = x + z;
            y[jd + st] = x - z;
          }
      const uint32_t n1 = (lane & 1) ? 0x80000000u : 0u, n2 = (lane & 2) ? 0x80000000u : 0u;
      const uint32_t n4 = (lane & 4) ? 0x80000000u : 0u, n8 = (lane & 8) ? 0x80000000u : 0u;
      const uint32_t n16 = (lane & 16) ? 0x80000000u : 0u;
      for (int jd = 0; jd < 8; jd++) {
        float v = y[jd];
        v = fwht_pair<1>(v, n1);
        v = fwht_pair<2>(v, n2);
        v = fwht_pair<4>(v, n4);
        v = fwht_pair<8>(v, n8);
        v = fwht_pair<16>(v, n16);
        y[jd] = v * 0.0625f;
      }
    }
    const int ri = wpos0 + (r >> 3);
    if (ri <= q_last) {
      float *op = a.out + ((size_t)ri * a.n_q_heads + (size_t)g * kGqa + (r & 7)) * 256 + col;
      for (int jd = 0; jd < 8; jd++) op[32 * jd] = y[jd];
    }
  }
}

size_t prefill_workspace_bytes(const kv_pool *pool, int64_t n_cells) {
  if (n_cells <= 0) return 0;
  return (size_t)pool->n_kv_heads * (size_t)((n_cells + kPfTile - 1) / kPfTile) * kPfImageBytes;
}

int launch_attn_prefill(const kv_pool *pool, const kv_seq *seq, const void *q, int q_dtype,
                        int n_q_heads, int pos0, int n_new, float scale, float *out, void *ws,
                        hipStream_t s) {
  PrefillArgs a;
  for (int i = 0; i < 4; i++) a.run[i] = (const uint8_t *)pool->run[i];
  a.pt = seq->page_table;
  a.q = q;
  a.out = out;
  a.n_pages = pool->n_pages;
  a.P = pool->page_size;
  a.H = pool->n_kv_heads;
  a.n_q_heads = n_q_heads;
  a.pos0 = pos0;
  a.n_new = n_new;
  a.scale2 = scale * 1.4426950408889634f;
  a.img = (uint8_t *)ws;
  a.n_tiles = (pos0 + n_new + kPfTile - 1) / kPfTile;
  const bool qf32 = q_dtype == KV_DTYPE_F32;
  const int pos_per_wg = kPfWaves * 32 / kGqa;
  const dim3 sgrid(a.n_tiles, a.H), grid((n_new + pos_per_wg - 1) / pos_per_wg, a.H), block(kPfWaves * 64);
  // an armed timing pair brackets both kernels of the call
  hipEvent_t e0, e1;
  take_launch_events(&e0, &e1);
  auto stage = [&](auto kernel) { hipExtLaunchKernelGGL(kernel, sgrid, block, 0, s, e0, nullptr, 0, a); };
  auto attend = [&](auto kernel) { hipExtLaunchKernelGGL(kernel, grid, block, 0, s, nullptr, e1, 0, a); };
  switch (pool->fmt) {
    case KV_FMT_F16: stage(prefill_stage_kernel<KV_FMT_F16>); break;
    case KV_FMT_INT8: stage(prefill_stage_kernel<KV_FMT_INT8>); break;
    case KV_FMT_Q4_0: stage(prefill_stage_kernel<KV_FMT_Q4_0>); break;
    case KV_FMT_K8V4: stage(prefill_stage_kernel<KV_FMT_K8V4>); break;
    default: return KV_ERR_UNSUPPORTED;
  }
  switch (pool->fmt * 2 + (qf32 ? 1 : 0)) {
    case KV_FMT_F16 * 2: attend(attn_prefill_kernel<false, KV_FMT_F16>); break;
    case KV_FMT_F16 * 2 + 1: attend(attn_prefill_kernel<true, KV_FMT_F16>); break;
    case KV_FMT_INT8 * 2: attend(attn_prefill_kernel<false, KV_FMT_INT8>); break;
    case KV_FMT_INT8 * 2 + 1: attend(attn_prefill_kernel<true, KV_FMT_INT8>); break;
    case KV_FMT_Q4_0 * 2: attend(attn_prefill_kernel<false, KV_FMT_Q4_0>); break;
    case KV_FMT_Q4_0 * 2 + 1: attend(attn_prefill_kernel<true, KV_FMT_Q4_0>); break;
    case KV_FMT_K8V4 * 2: attend(attn_prefill_kernel<false, KV_FMT_K8V4>); break;
    case KV_FMT_K8V4 * 2 + 1: attend(attn_prefill_kernel<true, KV_FMT_K8V4>); break;
    default: return KV_ERR_UNSUPPORTED;
  }
  return launch_status();
}

}  // namespace k8v4
