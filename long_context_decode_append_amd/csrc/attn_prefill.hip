// Causal prefill-chunk attention over a paged pool, for gfx950.
//
// Computes, for n_new queries at positions [pos0, pos0 + n_new), the same
// attention as decode ("#120 --kv k8v4: hybrid KV cache -- INT8 K +
// Hadamard-rotated Q4_0 V (816 B/cell)", How: one fused attention serves
// decode, verify and prefill), row i attending cells [0, pos0 + i].  The
// pool may hold any of the three formats of those pages (k8v4; int8 K and V;
// rotated q4_0 K and V, scored against the rotated query).
//
// Here Q.K^T and P.V are dense contractions (128 query rows share every K/V
// tile), so both run on the matrix cores (v_mfma_f32_16x16x32_f16):
//   * workgroup = 8 waves = 16 query positions x 8 GQA heads of one KV head
//     (128 rows), one workgroup per CU; each wave owns one 16-row tile;
//   * per 32-cell tile the workgroup loads the raw pages once and
//     dequantizes into LDS: INT8 K as exact fp16 codes (the two group scales
//     applied to the two half-dots), q4_0 K as (code - 8) * d16, V as
//     (code - 8) * d16 or code * d in fp16, stored transposed [dim][cell]
//     (two cells per 4-byte write, cells ordered so that the P.V B-operand
//     of a lane is one 16-byte read);
//   * two LDS tile buffers: tile i + 1 is dequantized into one while tile i
//     is computed from the other, from registers loaded a tile earlier; the
//     two waves of a SIMD take the halves in opposite order;
//   * S^T = K.Q^T keeps P in registers in the P.V A-operand layout; online
//     softmax in base 2 against a lazily moved reference max; the causal
//     mask only in the tiles that reach a wave's rows;
//   * epilogue: O / l, then (rotated V) the inverse Walsh-Hadamard transform
//     one row at a time through LDS (4 dims per lane).
#include "device.hpp"
#include "launch.hpp"

namespace k8v4 {

constexpr int kPfWaves = 8;
constexpr int kPfPos = kPfWaves * 16 / kGqa;  // query positions per workgroup (x 8 heads)
constexpr int kPfTile = 32;                   // cells per tile
constexpr int kKRow = 256 + 16;               // fp16 elements per K row in LDS (padded; measured best)
constexpr int kVRow = kPfTile + 16;          // fp16 elements per transposed V row (16-byte multiple)
constexpr int kVBlockPad = 32;                // fp16 elements after every 32 rows (one block)
constexpr float kPfLazy = 8.0f;               // log2 headroom of the lazy softmax reference
static_assert(kPfWaves * 64 == 512, "one tile load unit per thread");

// offset of dim d0 + d (d0 a multiple of 32, 0 <= d < 32) in the V tile
__device__ __forceinline__ int v_row(int d0, int d) { return (d0 + d) * kVRow + (d0 >> 5) * kVBlockPad; }
// position of cell c (0..31) within a V row: the P.V B-operand of lane group
// lg takes cells 4lg..4lg+3 and 16+4lg..16+4lg+3, stored side by side so one
// 16-byte read fetches them (cells 2i, 2i+1 stay adjacent)
__device__ __forceinline__ int v_pos(int c) { return 8 * ((c & 15) >> 2) + 4 * (c >> 4) + (c & 3); }

struct PrefillArgs {
  const uint8_t *run[4];  // the pool's runs (format-dependent, as the header lays them out)
  const int32_t *pt;
  const void *q;
  float *out;
  int n_pages, P, H;
  int n_q_heads;
  int p_shift;            // log2(P) when P is a power of two, else -1
  int pos0, n_new;
  float scale2;           // softmax scale * log2(e)
};

// (x & m) | c in one VALU op (the compiler splits it when both are literals)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}

// Raw pages of one tile, in the registers of the thread that dequantizes
// them.  Work unit u in [0, 512), one per thread:
//   INT8 K: 16 codes of cell u / 16, dims 16 (u % 16) ..; scale (u < 64) of
//           cell u / 2, group u % 2
//   q4_0 K: bytes 8 (u % 2) .. + 7 of block (u % 16) / 2 of cell u / 16 and
//           that block's fp16 scale
//   q4_0 V: bytes 4 (u / 128) .. + 3 of block (u / 16) % 8 of cells 2 (u % 16)
//           and 2 (u % 16) + 1, and the two blocks' scales
//   INT8 V: codes of dims 8 (u / 16) .. + 7 of the same two cells, and the two
//           cells' scales of that 128-dim group
//   fp16 K: dims 16 (u % 16) .. + 15 of cell u / 16 (32 bytes, two loads)
//   fp16 V: 32 consecutive bytes of half u / 256 of the tile: chunks 2i and
//           2i + 1 (i = u % 256) of its 8 KB block, each 4 cells x 2 dims
struct PfRaw {
  u32x4 k;          // INT8 K: 16 codes; q4_0 K: .x .y nibble bytes, .z scale
  float kd;         // INT8 K scale (x softmax scale); q4_0 K: the softmax scale
  u32x2 va, vb;     // V of the two cells (q4_0: .x only)
  uint32_t vd;      // q4_0 V: the two fp16 scales (lo: first cell)
  float vsa, vsb;   // INT8 V: the two cells' scales
  u32x4 k2;         // fp16 K: dims 8 .. 15 of the unit
  u32x4 v16[2];     // fp16 V: the unit's two 16-byte chunks
};

// Per tile: the physical (page, head) tile of each 16-cell half (P is a
// multiple of 16 and tiles start at multiples of 32, so a half never
// straddles a page) and the slot of its first cell; wave-uniform.
struct PfHalves {
  int tile[2];
  int slot0[2];
  int bad[2];  // page-table entry out of range: read page 0 instead, give NaN scores
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
  for (int i = 0; i < 2; i++) {
    const int c = c0 + 16 * i;
    h.tile[i] = 0;
    h.slot0[i] = 0;
    h.bad[i] = 0;
    if (c < n_cells) {  // page-table entries past the visible cells are never read
      const int pidx = a.p_shift >= 0 ? (c >> a.p_shift) : c / a.P;
      int page = a.pt[pidx];
      h.bad[i] = page < 0 || page >= a.n_pages;
      page = h.bad[i] ? 0 : page;
      h.tile[i] = page * a.H + g;
      h.slot0[i] = c - pidx * a.P;
    }
  }
  return h;
}

template <int FMT>
__device__ __forceinline__ void pf_load_units(const PrefillArgs &a, const PfHalves &hv, int c0, int n_cells, int u,
                                              PfRaw &r);

// The tile's raw pages for work unit u; the K scale slots (units u < 64,
// cell u / 2) of a half whose page-table entry is out of range hold NaN, so
// every row whose causal window reaches that half returns NaN (rows that
// stop before it mask those cells to -inf), while the loads read page 0
// and never leave the pool.
template <int FMT>
__device__ __forceinline__ void pf_load(const PrefillArgs &a, const PfHalves &hv, int c0, int n_cells, int u,
                                        PfRaw &r) {
  pf_load_units<FMT>(a, hv, c0, n_cells, u, r);
  if (u < 2 * kPfTile && c0 + (u >> 1) < n_cells && (((u >> 5) ? hv.bad[1] : hv.bad[0]) != 0))
    r.kd = __builtin_nanf("");
}

template <int FMT>
__device__ __forceinline__ void pf_load_units(const PrefillArgs &a, const PfHalves &hv, int c0, int n_cells, int u,
                                              PfRaw &r) {
  r.k = u32x4{0u, 0u, 0u, 0u};
  r.kd = a.scale2;
  if (FMT == KV_FMT_F16) {
    // fp16 blocks (8 KB per 16 cells in each of K and V, the layout the
    // decode kernel loads as MFMA operands); values of cells past the
    // visible ones are zeroed (they may hold any bits)
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int cl = u >> 4, hf = cl >> 4, m = u & 15;
    r.k2 = z;
    if (c0 + cl < n_cells) {
      const uint8_t *kb = a.run[0] + hv.cell(hf) * 512 + (m >> 1) * 1024 + (m & 1) * 512 + (cl & 15) * 16;
      r.k = *reinterpret_cast<const u32x4 *>(kb);
      r.k2 = *reinterpret_cast<const u32x4 *>(kb + 256);
    }
    r.kd = 0.f;
    if (u < 2 * kPfTile && c0 + (u >> 1) < n_cells) r.kd = a.scale2;
    const int vh = u >> 8, idx = u & 255;
    const int lq = (idx >> 3) & 3;  // cell quad of the two chunks
    const uint8_t *vb = a.run[2] + hv.cell(vh) * 512 + 32 * idx;
    r.v16[0] = r.v16[1] = z;
    const int cq = c0 + 16 * vh + 4 * lq;
    if (cq < n_cells) {
      r.v16[0] = *reinterpret_cast<const u32x4 *>(vb);
      r.v16[1] = *reinterpret_cast<const u32x4 *>(vb + 16);
      if (cq + 3 >= n_cells) {
        const uint32_t m01 = (cq < n_cells ? 0x0000ffffu : 0u) | (cq + 1 < n_cells ? 0xffff0000u : 0u);
        const uint32_t m23 = (cq + 2 < n_cells ? 0x0000ffffu : 0u) | (cq + 3 < n_cells ? 0xffff0000u : 0u);
        for (int q = 0; q < 2; q++) {
          r.v16[q].x &= m01;
          r.v16[q].y &= m23;
          r.v16[q].z &= m01;
          r.v16[q].w &= m23;
        }
      }
    }
    return;
  }
  if (FMT != KV_FMT_Q4_0) {
    const int cl = u >> 4, hf = cl >> 4;
    // K-code run: 4 KB per 16 cells, [dim quarter][cell % 16][64 codes];
    // a wave's 64 units read four 256-byte stretches
    const int m = u & 15;
    if (c0 + cl < n_cells)
      r.k = *reinterpret_cast<const u32x4 *>(a.run[0] + hv.cell(hf) * 256 + (m >> 2) * 1024 + (cl & 15) * 64 +
                                             16 * (m & 3));
    r.kd = 0.f;
    if (u < 2 * kPfTile) {
      const int cs = u >> 1, hs = cs >> 4;
      if (c0 + cs < n_cells)
        r.kd = a.scale2 * reinterpret_cast<const float *>(a.run[1])[(hv.cell(hs) + (cs & 15)) * 2 + (u & 1)];
    }
  } else {
    const int cl = u >> 4, hf = cl >> 4, b = (u & 15) >> 1, hh = u & 1;
    if (c0 + cl < n_cells) {
      const uint8_t *kt = a.run[0] + (size_t)hv.tile_of(hf) * 144 * a.P;
      const int slot = hv.slot_of(hf) + (cl & 15);
      const u32x2 w = *reinterpret_cast<const u32x2 *>(kt + (size_t)slot * 128 + 16 * b + 8 * hh);
      r.k.x = w.x;
      r.k.y = w.y;
      r.k.z = *reinterpret_cast<const uint16_t *>(kt + q4_scale_off(a.P, slot, b));
    }
  }
  const int cp = u & 15;
  const int hf = cp >> 3;  // cells 2cp, 2cp+1 lie in half cp / 8
  const int slot = hv.slot_of(hf) + 2 * (cp & 7);
  const bool ok_a = c0 + 2 * cp < n_cells, ok_b = c0 + 2 * cp + 1 < n_cells;
  r.va = r.vb = u32x2{0u, 0u};
  r.vd = 0u;
  r.vsa = r.vsb = 0.f;
  if (FMT != KV_FMT_INT8) {
    const int b = (u >> 4) & 7, qq = u >> 7;
    const uint8_t *vt = a.run[2] + (size_t)hv.tile_of(hf) * 144 * a.P;
    // slot is even, so the two cells' block-b scales are one aligned word
    if (ok_a) {
      r.va.x = *reinterpret_cast<const uint32_t *>(vt + (size_t)slot * 128 + 16 * b + 4 * qq);
      r.vd = *reinterpret_cast<const uint32_t *>(vt + q4_scale_off(a.P, slot, b));
    }
    if (ok_b)
      r.vb.x = *reinterpret_cast<const uint32_t *>(vt + (size_t)(slot + 1) * 128 + 16 * b + 4 * qq);
    else
      r.vd &= 0xFFFFu;  // the unwritten slot's scale may be anything
  } else {
    const int dg = u >> 4;  // dims 8 dg .. 8 dg + 7, scale group dg / 16
    const size_t ca = (size_t)hv.tile_of(hf) * a.P + slot;
    const float *vs = reinterpret_cast<const float *>(a.run[3]);
    if (ok_a) {
      r.va = *reinterpret_cast<const u32x2 *>(a.run[2] + ca * 256 + 8 * dg);
      r.vsa = vs[ca * 2 + (dg >> 4)];
    }
    if (ok_b) {
      r.vb = *reinterpret_cast<const u32x2 *>(a.run[2] + (ca + 1) * 256 + 8 * dg);
      r.vsb = vs[(ca + 1) * 2 + (dg >> 4)];
    }
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

template <int FMT>
__device__ __forceinline__ void pf_store(const PfRaw &r, int u, _Float16 *lk, _Float16 *lv, float *lks) {
  if (FMT == KV_FMT_F16) {
    // K as loaded, row-major [cell][dim]; V transposed [dim][cell]: chunk
    // (uu, lq, nn) holds dims 16 nn + 2 uu (+1) of cells 4 lq .. 4 lq + 3
    // of its half, which sit side by side in a V row (v_pos)
    _Float16 *kd = lk + (u >> 4) * kKRow + 16 * (u & 15);
    *reinterpret_cast<u32x4 *>(kd) = r.k;
    *reinterpret_cast<u32x4 *>(kd + 8) = r.k2;
    if (u < 2 * kPfTile) lks[u] = r.kd;
    const int vh = u >> 8, idx = u & 255;
    const int uu = idx >> 5, lq = (idx >> 3) & 3;
    for (int q = 0; q < 2; q++) {
      const int nn = 2 * (idx & 7) + q;
      const int d = 16 * nn + 2 * uu;
      _Float16 *v0 = lv + v_row(32 * (d >> 5), d & 31) + v_pos(16 * vh + 4 * lq);
      _Float16 *v1 = lv + v_row(32 * ((d + 1) >> 5), (d + 1) & 31) + v_pos(16 * vh + 4 * lq);
      *reinterpret_cast<u32x2 *>(v0) = u32x2{r.v16[q].x, r.v16[q].y};
      *reinterpret_cast<u32x2 *>(v1) = u32x2{r.v16[q].z, r.v16[q].w};
    }
    return;
  }
  if (FMT != KV_FMT_Q4_0) {
    // INT8 K -> exact fp16 codes, row-major [cell][dim]
    const f16x2 c1152 = {(_Float16)1152.0f, (_Float16)1152.0f};
    uint32_t kf[8];
    const uint32_t kw[4] = {r.k.x, r.k.y, r.k.z, r.k.w};
    for (int i = 0; i < 4; i++) {
      uint32_t lo, hi;
      i8x4_to_f16_biased(kw[i], lo, hi);
      kf[2 * i] = as_u32(as_f16x2(lo) - c1152);
      kf[2 * i + 1] = as_u32(as_f16x2(hi) - c1152);
    }
    _Float16 *kd = lk + (u >> 4) * kKRow + 16 * (u & 15);
    *reinterpret_cast<u32x4 *>(kd) = u32x4{kf[0], kf[1], kf[2], kf[3]};
    *reinterpret_cast<u32x4 *>(kd + 8) = u32x4{kf[4], kf[5], kf[6], kf[7]};
  } else {
    // q4_0 K -> (code - 8) * d16: elements 8hh .. 8hh + 7 (low nibbles) and
    // 16 + 8hh .. (high nibbles) of block b
    const int b = (u & 15) >> 1, hh = u & 1;
    const uint32_t d16 = r.k.z & 0xFFFFu;
    const f16x2 d = as_f16x2(d16 | (d16 << 16));
    uint32_t lo[4], hi[4];
    q4_word_to_f16(r.k.x, d, lo, hi);
    q4_word_to_f16(r.k.y, d, lo + 2, hi + 2);
    _Float16 *kd = lk + (u >> 4) * kKRow + 32 * b + 8 * hh;
    *reinterpret_cast<u32x4 *>(kd) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    *reinterpret_cast<u32x4 *>(kd + 16) = u32x4{hi[0], hi[1], hi[2], hi[3]};
  }
  if (u < 2 * kPfTile) lks[u] = r.kd;  // K scale x softmax scale x log2(e)
  const int cp = u & 15;
  if (FMT != KV_FMT_INT8) {
    // q4_0 V -> (code - 8) * d16, transposed [dim][cell]; byte i of the block
    // holds element i (low nibble) and element 16 + i (high nibble)
    const f16x2 c1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
    const f16x2 c72 = {(_Float16)72.0f, (_Float16)72.0f};
    const int b = (u >> 4) & 7, qq = u >> 7;
    const f16x2 dd = as_f16x2(r.vd);
    _Float16 *vb = lv + v_row(32 * b, 4 * qq) + v_pos(2 * cp);  // element 4qq of block b
    for (int e = 0; e < 4; e++) {
      // [a.byte, 0, b.byte, 0] for byte e of each cell: elements 4qq + e
      // (low nibbles) and 16 + 4qq + e (high nibbles)
      const uint32_t sel = (0x0cu << 24) | ((4u + e) << 16) | (0x0cu << 8) | (uint32_t)e;
      const uint32_t x = perm(r.vb.x, r.va.x, sel);
      const uint32_t lo = as_u32((as_f16x2(and_or(x, 0x000F000Fu, 0x64006400u)) - c1032) * dd);
      const uint32_t hi = as_u32((as_f16x2(and_or(x, 0x00F000F0u, 0x54005400u)) - c72) * dd);
      *reinterpret_cast<uint32_t *>(vb + e * kVRow) = lo;
      *reinterpret_cast<uint32_t *>(vb + (16 + e) * kVRow) = hi;
    }
  } else {
    // INT8 V -> code * d rounded to fp16, transposed [dim][cell]
    const int dg = u >> 4;
    _Float16 *vb = lv + v_row(32 * (dg >> 2), 8 * (dg & 3)) + v_pos(2 * cp);
    const uint32_t wa[2] = {r.va.x, r.va.y}, wb[2] = {r.vb.x, r.vb.y};
    for (int e = 0; e < 8; e++) {
      const float xa = (float)(int8_t)(wa[e >> 2] >> (8 * (e & 3))) * r.vsa;
      const float xb = (float)(int8_t)(wb[e >> 2] >> (8 * (e & 3))) * r.vsb;
      const f16x2 pr = {(_Float16)xa, (_Float16)xb};
      *reinterpret_cast<uint32_t *>(vb + e * kVRow) = as_u32(pr);
    }
  }
}

template <bool QF32, int FMT>
__global__ __launch_bounds__(kPfWaves * 64, 1) void attn_prefill_kernel(const PrefillArgs a) {
  // two tile buffers (K tile, then V tile), in one array that also holds the
  // per-wave row slices (kPfWaves x 16 rows x 256 fp32) of the q rotation
  // and of the epilogue
  constexpr int kKElems = kPfTile * kKRow, kVElems = 256 * kVRow + 8 * kVBlockPad;
  constexpr int kBufElems = kKElems + kVElems;
  constexpr int kTileElems = 2 * kBufElems;
  constexpr int kEpiElems = kPfWaves * 16 * 256 * 2;  // fp16 units
  __shared__ __attribute__((aligned(16))) _Float16 lds_kv[kTileElems > kEpiElems ? kTileElems : kEpiElems];
  __shared__ __attribute__((aligned(16))) float lds_ks[2 * kPfTile * 2];
  _Float16 *const lds_k = lds_kv;
  _Float16 *const lds_v = lds_kv + kKElems;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, lg = lane >> 4;
  const int g = blockIdx.y;
  const int qb0 = blockIdx.x * kPfPos;                    // first query (chunk-relative)
  const int q_last = min(qb0 + kPfPos, a.n_new) - 1;      // last valid query of the block
  const int n_cells = a.pos0 + q_last + 1;                // cells any row of the block sees
  // first cell at which this wave's rows need the causal mask
  const int mask_from = a.pos0 + qb0 + 2 * wave;          // rows 16 wave ..: positions qb0 + 2 wave ..
  float *const wrow = reinterpret_cast<float *>(lds_kv) + wave * 16 * 256;  // this wave's slice

  // ---- queries: B operand of S^T = K.Q^T; row r = 16 wave + n, position
  // qb0 + r / 8, head 8 g + r % 8; k-step kk holds dims 32 kk + 8 lg .. + 7.
  // The q4_0 format scores against rotated keys: q~ = H q / 16 first,
  // through this wave's LDS slice.
  const int r = 16 * wave + n;
  const int qi = qb0 + (r >> 3);
  const bool rvalid = qi <= q_last;
  const int qpos = a.pos0 + qi;
  float qv[8][8];
  {
    const size_t qbase = ((size_t)qi * a.n_q_heads + (size_t)g * kGqa + (r & 7)) * 256;
    for (int kk = 0; kk < 8; kk++) {
      const int d0 = 32 * kk + 8 * lg;
      if (!QF32) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (rvalid) w = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.q) + qbase + d0);
        const f16x8 h = __builtin_bit_cast(f16x8, w);
        for (int e = 0; e < 8; e++) qv[kk][e] = (float)h[e];
      } else {
        f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
        if (rvalid) {
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
    for (int kk = 0; kk < 8; kk++) {
      float *dst = wrow + n * 256 + 32 * kk + 8 * lg;
      *reinterpret_cast<f32x4 *>(dst) = f32x4{qv[kk][0], qv[kk][1], qv[kk][2], qv[kk][3]};
      *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{qv[kk][4], qv[kk][5], qv[kk][6], qv[kk][7]};
    }
    for (int rr = 0; rr < 16; rr++) {
      f32x4 y4 = *reinterpret_cast<const f32x4 *>(&wrow[rr * 256 + 4 * lane]);
      float y[4] = {y4[0], y4[1], y4[2], y4[3]};
      fwht256_lane4(y, lane);
      *reinterpret_cast<f32x4 *>(&wrow[rr * 256 + 4 * lane]) = f32x4{y[0], y[1], y[2], y[3]};
    }
    for (int kk = 0; kk < 8; kk++) {
      const float *src = wrow + n * 256 + 32 * kk + 8 * lg;
      const f32x4 x0 = *reinterpret_cast<const f32x4 *>(src);
      const f32x4 x1 = *reinterpret_cast<const f32x4 *>(src + 4);
      for (int e = 0; e < 4; e++) {
        qv[kk][e] = x0[e];
        qv[kk][4 + e] = x1[e];
      }
    }
    __syncthreads();  // the slices are free again before the first tile lands there
  }
  f16x8 qop[8];
  f16x8 qlo[QF32 ? 8 : 1];
  for (int kk = 0; kk < 8; kk++) {
    f16x8 hi, lo;
    for (int e = 0; e < 8; e++) {
      const _Float16 h = (_Float16)qv[kk][e];
      hi[e] = h;
      if (QF32) lo[e] = (_Float16)(qv[kk][e] - (float)h);
    }
    qop[kk] = hi;
    if (QF32) qlo[kk] = lo;
  }

  float m = -1e30f, lsum = 0.f;
  f32x4 o[16];
  for (int j = 0; j < 16; j++) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  PfRaw raw;
  auto load_tile = [&](int c) {
    const PfHalves hv = pf_halves(a, g, c, n_cells);
    pf_load<FMT>(a, hv, c, n_cells, tid, raw);
  };
  auto store_tile = [&](int buf) {
    pf_store<FMT>(raw, tid, lds_k + buf * kBufElems, lds_v + buf * kBufElems, lds_ks + buf * 2 * kPfTile);
  };
  auto compute_tile = [&](int c0, const _Float16 *lk, const _Float16 *lv, const float *lks) {
    const bool masked = c0 + kPfTile - 1 >= mask_from;

    // ---------------- S^T = K . Q^T for 2 cell tiles of 16
    float s[8];
    for (int ct = 0; ct < 2; ct++) {
      const _Float16 *kr = lk + (16 * ct + n) * kKRow + 8 * lg;
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      for (int kk = 0; kk < 8; kk++) {
        const f16x8 kop = *reinterpret_cast<const f16x8 *>(kr + 32 * kk);
        acc[kk >> 2] = mfma16x16x32(kop, qop[kk], acc[kk >> 2]);
        if (QF32) acc[kk >> 2] = mfma16x16x32(kop, qlo[kk], acc[kk >> 2]);
      }
      for (int i = 0; i < 4; i++) {
        const float2 dk = *reinterpret_cast<const float2 *>(&lks[(16 * ct + 4 * lg + i) * 2]);
        float sv = dk.x * acc[0][i] + dk.y * acc[1][i];
        if (masked) {
          const int cell = c0 + 16 * ct + 4 * lg + i;
          sv = (rvalid && cell <= qpos) ? sv : -INFINITY;
        }
        s[4 * ct + i] = sv;
      }
    }

    // ---------------- online softmax, P operand; the reference max moves
    // only when a row's max exceeds it by more than 2^kPfLazy
    f16x8 pop;
    {
      float mx = s[0];
      for (int e = 1; e < 8; e++) mx = fmaxf(mx, s[e]);
      mx = max_lg(mx);
      if (__any(mx > m + kPfLazy)) {
        const float mnew = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        lsum *= alpha;
        m = mnew;
        float al[4];
        for (int i = 0; i < 4; i++) al[i] = lane_get(alpha, 4 * lg + i);
        for (int j = 0; j < 16; j++)
          for (int i = 0; i < 4; i++) o[j][i] *= al[i];
      }
      float ps = 0.f;
      for (int e = 0; e < 8; e++) {
        const float p = __builtin_amdgcn_exp2f(s[e] - m);
        ps += p;
        pop[e] = (_Float16)p;
      }
      lsum += ps;
    }

    // ---------------- O += P . V; B for dim tile j, column n: dim 16j + n,
    // k-slots = cells 4lg + 0..3 and 16 + 4lg + 0..3
    for (int j = 0; j < 16; j++) {
      const _Float16 *vr = lv + v_row(32 * (j >> 1), 16 * (j & 1) + n) + 8 * lg;
      const f16x8 B = *reinterpret_cast<const f16x8 *>(vr);
      o[j] = mfma16x16x32(pop, B, o[j]);
    }
  };

  // Tile i + 1 is staged into buffer (i + 1) % 2 while tile i is computed
  // from buffer i % 2; the waves sharing a SIMD (w, w + 4) stage and compute
  // in opposite order, so one's dequantization overlaps the other's MFMAs.
  // Tiles past the visible cells load nothing and store zeros (unread).
  load_tile(0);
  store_tile(0);
  load_tile(kPfTile);
  __syncthreads();
  const bool store_first = (wave & 4) == 0;
  int buf = 0;
  for (int c0 = 0; c0 < n_cells; c0 += kPfTile, buf ^= 1) {
    if (store_first) {
      store_tile(buf ^ 1);
      load_tile(c0 + 2 * kPfTile);
    }
    compute_tile(c0, lds_k + buf * kBufElems, lds_v + buf * kBufElems, lds_ks + buf * 2 * kPfTile);
    if (!store_first) {
      store_tile(buf ^ 1);
      load_tile(c0 + 2 * kPfTile);
    }
    __syncthreads();
  }

  // ---------------- epilogue: normalize, then (rotated V) the inverse
  // Walsh-Hadamard transform row by row through this wave's LDS slice (free
  // after the last barrier), and store
  lsum = sum_lg(lsum);
  float inv[4];
  for (int i = 0; i < 4; i++) inv[i] = 1.0f / lane_get(lsum, 4 * lg + i);
  // value (row 4lg + i, dim 16j + n) lives in o[j][i]
  for (int j = 0; j < 16; j++)
    for (int i = 0; i < 4; i++) wrow[(4 * lg + i) * 256 + 16 * j + n] = o[j][i] * inv[i];
  for (int rr = 0; rr < 16; rr++) {
    const int rw = 16 * wave + rr;
    const int qw = qb0 + (rw >> 3);
    const f32x4 y4 = *reinterpret_cast<const f32x4 *>(&wrow[rr * 256 + 4 * lane]);
    float y[4] = {y4[0], y4[1], y4[2], y4[3]};
    if (FMT == KV_FMT_Q4_0 || FMT == KV_FMT_K8V4) fwht256_lane4(y, lane);
    if (qw <= q_last) {
      float *op = a.out + ((size_t)qw * a.n_q_heads + (size_t)g * kGqa + (rw & 7)) * 256 + 4 * lane;
      *reinterpret_cast<f32x4 *>(op) = f32x4{y[0], y[1], y[2], y[3]};
    }
  }
}

int launch_attn_prefill(const kv_pool *pool, const kv_seq *seq, const void *q, int q_dtype,
                        int n_q_heads, int pos0, int n_new, float scale, float *out,
                        hipStream_t s) {
  PrefillArgs a;
  for (int i = 0; i < 4; i++) a.run[i] = (const uint8_t *)pool->run[i];
  a.pt = seq->page_table;
  a.q = q;
  a.out = out;
  a.n_pages = pool->n_pages;
  a.P = pool->page_size;
  a.H = pool->n_kv_heads;
  a.p_shift = -1;
  for (int sh = 0; sh < 31; sh++)
    if ((1 << sh) == a.P) a.p_shift = sh;
  a.n_q_heads = n_q_heads;
  a.pos0 = pos0;
  a.n_new = n_new;
  a.scale2 = scale * 1.4426950408889634f;
  const dim3 grid((n_new + kPfPos - 1) / kPfPos, a.H), block(kPfWaves * 64);
  const bool qf32 = q_dtype == KV_DTYPE_F32;
  switch (pool->fmt * 2 + (qf32 ? 1 : 0)) {
    case KV_FMT_F16 * 2: launch((attn_prefill_kernel<false, KV_FMT_F16>), grid, block, s, a); break;
    case KV_FMT_F16 * 2 + 1: launch((attn_prefill_kernel<true, KV_FMT_F16>), grid, block, s, a); break;
    case KV_FMT_INT8 * 2: launch((attn_prefill_kernel<false, KV_FMT_INT8>), grid, block, s, a); break;
    case KV_FMT_INT8 * 2 + 1: launch((attn_prefill_kernel<true, KV_FMT_INT8>), grid, block, s, a); break;
    case KV_FMT_Q4_0 * 2: launch((attn_prefill_kernel<false, KV_FMT_Q4_0>), grid, block, s, a); break;
    case KV_FMT_Q4_0 * 2 + 1: launch((attn_prefill_kernel<true, KV_FMT_Q4_0>), grid, block, s, a); break;
    case KV_FMT_K8V4 * 2: launch((attn_prefill_kernel<false, KV_FMT_K8V4>), grid, block, s, a); break;
    case KV_FMT_K8V4 * 2 + 1: launch((attn_prefill_kernel<true, KV_FMT_K8V4>), grid, block, s, a); break;
    default: return KV_ERR_UNSUPPORTED;
  }
  return launch_status();
}

}  // namespace k8v4
