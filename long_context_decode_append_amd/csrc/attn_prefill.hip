// Causal prefill-chunk attention over a k8v4 pool, for gfx950.
//
// Computes, for n_new queries at positions [pos0, pos0 + n_new), the same
// attention as decode ("#120 --kv k8v4: hybrid KV cache -- INT8 K +
// Hadamard-rotated Q4_0 V (816 B/cell)", How: one fused attention serves
// decode, verify and prefill), row i attending cells [0, pos0 + i].
//
// Here Q.K^T and P.V are dense contractions (256 query rows share every K/V
// tile), so both run on the matrix cores (v_mfma_f32_16x16x32_f16):
//   * workgroup = 4 waves = 16 query positions x 8 GQA heads of one KV head
//     (128 rows), two workgroups per CU; each wave owns 32 rows (2 row
//     tiles of 16);
//   * per 32-cell tile the workgroup loads the raw pages once and
//     dequantizes into LDS: K codes as exact fp16 (scales kept per cell and
//     128-dim group, applied to the two half-dots), V as (code - 8) * d16 in
//     fp16, stored transposed [dim][cell] (two cells per 4-byte write) so the
//     P.V B-operand is two 8-byte reads; while one workgroup loads a tile
//     the other one on the CU computes;
//   * S^T = K.Q^T keeps P in registers in the P.V A-operand layout; online
//     softmax in base 2 against a lazily moved reference max; the causal
//     mask only in the tiles that reach a wave's rows;
//   * epilogue: O / l, then the inverse Walsh-Hadamard transform one row at
//     a time through LDS (4 dims per lane).
#include "device.hpp"
#include "launch.hpp"

#ifndef PF_WAVES
#define PF_WAVES 8
#endif
#ifndef PF_ROWT
#define PF_ROWT 1
#endif
#ifndef PF_STAGGER
#define PF_STAGGER 1
#endif
#ifndef PF_SB
#define PF_SB 1
#endif
#ifndef PF_OCC
#define PF_OCC 1
#endif

namespace k8v4 {

constexpr int kPfWaves = PF_WAVES;
constexpr int kRowT = PF_ROWT;       // 16-row tiles per wave
constexpr int kPfPos = kPfWaves * 16 * kRowT / 8;  // query positions per workgroup (x 8 heads)
constexpr int kUnits = 512 / (kPfWaves * 64);      // tile load units per thread
constexpr int kPfTile = 32;          // cells per tile
constexpr int kKRow = 256 + 8;       // fp16 elements per K row in LDS (padded)
constexpr int kVRow = kPfTile + 4;   // fp16 elements per transposed V row (72 bytes)
constexpr int kVBlockPad = 32;      // fp16 elements after every 32 rows (one block)
// offset of dim d0 + d (d0 a multiple of 32, 0 <= d < 32) in the V tile
__device__ __forceinline__ int v_row(int d0, int d) { return (d0 + d) * kVRow + (d0 >> 5) * kVBlockPad; }
constexpr float kPfLazy = 8.0f;      // log2 headroom of the lazy softmax reference

struct PrefillArgs {
  const int8_t *kc;
  const float *ks;
  const uint8_t *vq;
  const int32_t *pt;
  const void *q;
  float *out;
  int n_pages, P, H;
  int n_q_heads;
  int p_shift;          // log2(P) when P is a power of two, else -1
  int pos0, n_new;
  float scale2;
};

// (x & m) | c in one VALU op (the compiler splits it when both are literals)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}

// raw pages of one tile, in the registers of the thread that dequantizes them
struct PfRaw {
  u32x4 k;       // 16 K codes: cell tid / 16, dims 16 (tid % 16) ..
  float kd;      // K scale (threads < 64): cell tid / 2, group tid % 2
  uint32_t va, vb;  // 4 nibble bytes of block b for cells 2cp, 2cp + 1
  uint32_t vd;   // their fp16 scales (lo: cell 2cp, hi: cell 2cp + 1)
};

// Per tile: the physical (page, head) tile of each 16-cell half (P is a
// multiple of 16 and tiles start at multiples of 32, so a half never
// straddles a page) and the slot of its first cell; wave-uniform.
struct PfHalves {
  int tile[2];
  int slot0[2];
  // first cell of half hf in the pool's cell order (a select: hf varies by lane)
  __device__ __forceinline__ size_t cell(int hf) const {
    return hf ? (size_t)tile[1] * P + slot0[1] : (size_t)tile[0] * P + slot0[0];
  }
  __device__ __forceinline__ int tile_of(int hf) const { return hf ? tile[1] : tile[0]; }
  __device__ __forceinline__ int slot_of(int hf) const { return hf ? slot0[1] : slot0[0]; }
  int P;
};

__device__ __forceinline__ PfHalves pf_halves(const PrefillArgs &a, int g, int c0, int n_cells) {
  PfHalves h;
  h.P = a.P;
  for (int i = 0; i < 2; i++) {
    const int c = c0 + 16 * i;
    h.tile[i] = 0;
    h.slot0[i] = 0;
    if (c < n_cells) {  // page-table entries past the visible cells are never read
      const int pidx = a.p_shift >= 0 ? (c >> a.p_shift) : c / a.P;
      int page = a.pt[pidx];
      page = (page < 0 || page >= a.n_pages) ? 0 : page;
      h.tile[i] = page * a.H + g;
      h.slot0[i] = c - pidx * a.P;
    }
  }
  return h;
}

__device__ __forceinline__ void pf_load(const PrefillArgs &a, const PfHalves &hv, int c0, int n_cells, int u,
                                        PfRaw &r) {
  // work unit u in [0, 512): K codes of cell u / 16, dims 16 (u % 16) ..;
  // K scale (u < 64) of cell u / 2, group u % 2; V bytes 4 (u / 128) ..
  // 4 (u / 128) + 3 of block (u / 16) % 8 of the cells 2 (u % 16), 2 (u % 16) + 1
  {
    const int cl = u >> 4, hf = cl >> 4;
    r.k = u32x4{0u, 0u, 0u, 0u};
    if (c0 + cl < n_cells)
      r.k = *reinterpret_cast<const u32x4 *>(a.kc + (hv.cell(hf) + (cl & 15)) * 256 + 16 * (u & 15));
  }
  r.kd = 0.f;
  if (u < 2 * kPfTile) {
    const int cl = u >> 1, hf = cl >> 4;
    if (c0 + cl < n_cells) r.kd = a.scale2 * a.ks[(hv.cell(hf) + (cl & 15)) * 2 + (u & 1)];
  }
  {
    const int cp = u & 15, b = (u >> 4) & 7, qq = u >> 7;
    const int hf = cp >> 3;  // cells 2cp, 2cp+1 lie in half cp / 8
    const uint8_t *vt = a.vq + (size_t)hv.tile_of(hf) * 144 * a.P;
    const int slot = hv.slot_of(hf) + 2 * (cp & 7);
    r.va = 0u;
    r.vb = 0u;
    r.vd = 0u;
    // slot is even, so the two cells' block-b scales are one aligned word
    if (c0 + 2 * cp < n_cells) {
      r.va = *reinterpret_cast<const uint32_t *>(vt + (size_t)slot * 128 + 16 * b + 4 * qq);
      r.vd = *reinterpret_cast<const uint32_t *>(vt + q4_scale_off(a.P, slot, b));
    }
    if (c0 + 2 * cp + 1 < n_cells)
      r.vb = *reinterpret_cast<const uint32_t *>(vt + (size_t)(slot + 1) * 128 + 16 * b + 4 * qq);
    else
      r.vd &= 0xFFFFu;  // the unwritten slot's scale may be anything
  }
}

__device__ __forceinline__ void pf_store(const PfRaw &r, int u, _Float16 *lk, _Float16 *lv, float *lks) {
  const f16x2 c1152 = {(_Float16)1152.0f, (_Float16)1152.0f};
  const f16x2 c1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2 c72 = {(_Float16)72.0f, (_Float16)72.0f};
  {
    // K -> exact fp16 codes, row-major [cell][dim]
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
  }
  if (u < 2 * kPfTile) lks[u] = r.kd;  // already times scale * log2(e)
  {
    // V -> (code - 8) * d16 in fp16, transposed [dim][cell]; byte i of the
    // block holds element i (low nibble) and element 16 + i (high nibble)
    const int cp = u & 15, b = (u >> 4) & 7, qq = u >> 7;
    const f16x2 dd = as_f16x2(r.vd);
    _Float16 *vb = lv + v_row(32 * b, 4 * qq) + 2 * cp;  // element 4qq of block b
    for (int e = 0; e < 4; e++) {
      // [a.byte, 0, b.byte, 0] for byte e of each cell: elements 4qq + e
      // (low nibbles) and 16 + 4qq + e (high nibbles)
      const uint32_t sel = (0x0cu << 24) | ((4u + e) << 16) | (0x0cu << 8) | (uint32_t)e;
      const uint32_t x = perm(r.vb, r.va, sel);
      const uint32_t lo = as_u32((as_f16x2(and_or(x, 0x000F000Fu, 0x64006400u)) - c1032) * dd);
      const uint32_t hi = as_u32((as_f16x2(and_or(x, 0x00F000F0u, 0x54005400u)) - c72) * dd);
      *reinterpret_cast<uint32_t *>(vb + e * kVRow) = lo;
      *reinterpret_cast<uint32_t *>(vb + (16 + e) * kVRow) = hi;
    }
  }
}

template <bool QF32>
__global__ __launch_bounds__(kPfWaves * 64, PF_OCC) void attn_prefill_kernel(const PrefillArgs a) {
  // K tile, then V tile, in one array that also holds the epilogue's
  // per-wave row slices (kPfWaves x 16 rows x 256 fp32)
  constexpr int kKElems = kPfTile * kKRow, kVElems = 256 * kVRow + 8 * kVBlockPad;
  constexpr int kBufElems = kKElems + kVElems;  // one buffer: K tile, then V tile
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
  const int mask_from = a.pos0 + qb0 + 2 * kRowT * wave;  // first position of the wave's rows

  // ---- queries: B operand of S^T = K.Q^T; row r = 32*wave + 16*t + n,
  // position qb0 + r/8, head g*8 + r%8; k-step kk holds dims 32kk + 8lg..+7
  f16x8 qop[kRowT][8];
  f16x8 qlo[QF32 ? kRowT : 1][QF32 ? 8 : 1];
  int qpos[kRowT];
  bool rvalid[kRowT];
  for (int t = 0; t < kRowT; t++) {
    const int r = 16 * kRowT * wave + 16 * t + n;
    const int qi = qb0 + (r >> 3);
    rvalid[t] = qi <= q_last;
    qpos[t] = a.pos0 + qi;
    const size_t qbase = ((size_t)qi * a.n_q_heads + (size_t)g * kGqa + (r & 7)) * 256;
    for (int kk = 0; kk < 8; kk++) {
      const int d0 = 32 * kk + 8 * lg;
      f16x8 hi, lo;
      if (!QF32) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (rvalid[t]) w = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.q) + qbase + d0);
        hi = __builtin_bit_cast(f16x8, w);
      } else {
        f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
        if (rvalid[t]) {
          x0 = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(a.q) + qbase + d0);
          x1 = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(a.q) + qbase + d0 + 4);
        }
        for (int e = 0; e < 8; e++) {
          const float x = e < 4 ? x0[e] : x1[e - 4];
          const _Float16 h = (_Float16)x;
          hi[e] = h;
          lo[e] = (_Float16)(x - (float)h);
        }
      }
      qop[t][kk] = hi;
      if (QF32) qlo[t][kk] = lo;
    }
  }

  float m[kRowT], lsum[kRowT];
  f32x4 o[kRowT][16];
  for (int t = 0; t < kRowT; t++) m[t] = -1e30f, lsum[t] = 0.f;
  for (int t = 0; t < kRowT; t++)
    for (int j = 0; j < 16; j++) o[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Two LDS tile buffers: while tile i is computed from one, tile i + 1 is
  // dequantized into the other from registers loaded during tile i - 1.
  // The waves sharing a SIMD (w, w + 4) do the two halves in opposite
  // order, so one's dequantization overlaps the other's MFMAs.
  PfRaw raw[kUnits];
  auto load_tile = [&](int c) {
    const PfHalves hv = pf_halves(a, g, c, n_cells);
    for (int h = 0; h < kUnits; h++) pf_load(a, hv, c, n_cells, tid + 64 * kPfWaves * h, raw[h]);
  };
  auto store_tile = [&](int buf) {
    for (int h = 0; h < kUnits; h++)
      pf_store(raw[h], tid + 64 * kPfWaves * h, lds_k + buf * kBufElems, lds_v + buf * kBufElems,
               lds_ks + buf * 2 * kPfTile);
  };
  auto compute_tile = [&](int c0, const _Float16 *lk, const _Float16 *lv, const float *lks) {
    const bool masked = c0 + kPfTile - 1 >= mask_from;

    // ---------------- S^T = K . Q^T for 2 cell tiles x 2 row tiles (each K
    // operand read once from LDS and used for both row tiles)
    float s[kRowT][8];
    for (int ct = 0; ct < 2; ct++) {
      const _Float16 *kr = lk + (16 * ct + n) * kKRow + 8 * lg;
      f32x4 acc[kRowT][2];
      for (int t = 0; t < kRowT; t++) acc[t][0] = acc[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int kk = 0; kk < 8; kk++) {
        const f16x8 kop = *reinterpret_cast<const f16x8 *>(kr + 32 * kk);
        for (int t = 0; t < kRowT; t++) {
          acc[t][kk >> 2] = mfma16x16x32(kop, qop[t][kk], acc[t][kk >> 2]);
          if (QF32) acc[t][kk >> 2] = mfma16x16x32(kop, qlo[t][kk], acc[t][kk >> 2]);
        }
        if (PF_SB && (kk & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
      for (int i = 0; i < 4; i++) {
        const float2 dk = *reinterpret_cast<const float2 *>(&lks[(16 * ct + 4 * lg + i) * 2]);
        for (int t = 0; t < kRowT; t++) {
          float sv = dk.x * acc[t][0][i] + dk.y * acc[t][1][i];
          if (masked) {
            const int cell = c0 + 16 * ct + 4 * lg + i;
            sv = (rvalid[t] && cell <= qpos[t]) ? sv : -INFINITY;
          }
          s[t][4 * ct + i] = sv;
        }
      }
    }

    // ---------------- online softmax, P operand; the reference max moves
    // only when a row's max exceeds it by more than 2^kPfLazy
    f16x8 pop[kRowT];
    for (int t = 0; t < kRowT; t++) {
      float mx = s[t][0];
      for (int e = 1; e < 8; e++) mx = fmaxf(mx, s[t][e]);
      mx = fmaxf(mx, lane_xor(mx, 16));
      mx = fmaxf(mx, lane_xor(mx, 32));
      if (__any(mx > m[t] + kPfLazy)) {
        const float mnew = fmaxf(m[t], mx);
        const float alpha = __builtin_amdgcn_exp2f(m[t] - mnew);
        lsum[t] *= alpha;
        m[t] = mnew;
        float al[4];
        for (int i = 0; i < 4; i++) al[i] = lane_get(alpha, 4 * lg + i);
        for (int j = 0; j < 16; j++)
          for (int i = 0; i < 4; i++) o[t][j][i] *= al[i];
      }
      float ps = 0.f;
      for (int e = 0; e < 8; e++) {
        const float p = __builtin_amdgcn_exp2f(s[t][e] - m[t]);
        ps += p;
        pop[t][e] = (_Float16)p;
      }
      lsum[t] += ps;
    }

    // ---------------- O += P . V; B for dim tile j, column n: dim 16j + n,
    // k-slots = cells 4lg + 0..3 and 16 + 4lg + 0..3
    for (int j = 0; j < 16; j++) {
      const _Float16 *vr = lv + v_row(32 * (j >> 1), 16 * (j & 1) + n) + 4 * lg;
      const u32x2 lo = *reinterpret_cast<const u32x2 *>(vr);
      const u32x2 hi = *reinterpret_cast<const u32x2 *>(vr + 16);
      const f16x8 B = __builtin_bit_cast(f16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      for (int t = 0; t < kRowT; t++) o[t][j] = mfma16x16x32(pop[t], B, o[t][j]);
      // keep at most four tiles' operands in flight (register budget)
      if (PF_SB && (j & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
  };
  load_tile(0);
  store_tile(0);
  load_tile(kPfTile);
  __syncthreads();
  const bool store_first = PF_STAGGER ? (wave & 4) == 0 : true;
  int buf = 0;
  for (int c0 = 0; c0 < n_cells; c0 += kPfTile, buf ^= 1) {
    // tiles past the visible cells load nothing and store zeros (unread)
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

  // ---------------- epilogue: normalize, then the inverse Walsh-Hadamard
  // transform row by row through LDS (this wave's 16 x 256 fp32 slice of
  // the tile buffers, free after the last barrier), and store
  float *ws = reinterpret_cast<float *>(lds_kv);  // [kPfWaves][16][256] fp32
  float *wrow = ws + wave * 16 * 256;
  for (int t = 0; t < kRowT; t++) {
    lsum[t] += lane_xor(lsum[t], 16);
    lsum[t] += lane_xor(lsum[t], 32);
    float inv[4];
    for (int i = 0; i < 4; i++) inv[i] = 1.0f / lane_get(lsum[t], 4 * lg + i);
    // value (row 4lg + i, dim 16j + n) lives in o[t][j][i]
    for (int j = 0; j < 16; j++)
      for (int i = 0; i < 4; i++) wrow[(4 * lg + i) * 256 + 16 * j + n] = o[t][j][i] * inv[i];
    for (int rr = 0; rr < 16; rr++) {
      const int r = 16 * kRowT * wave + 16 * t + rr;
      const int qi = qb0 + (r >> 3);
      f32x4 y4 = *reinterpret_cast<const f32x4 *>(&wrow[rr * 256 + 4 * lane]);
      float y[4] = {y4[0], y4[1], y4[2], y4[3]};
      fwht256_lane4(y, lane);
      if (qi <= q_last) {
        float *op = a.out + ((size_t)qi * a.n_q_heads + (size_t)g * kGqa + (r & 7)) * 256 + 4 * lane;
        *reinterpret_cast<f32x4 *>(op) = f32x4{y[0], y[1], y[2], y[3]};
      }
    }
  }
}

int launch_attn_prefill(const kv_pool *pool, const kv_seq *seq, const void *q, int q_dtype,
                        int n_q_heads, int pos0, int n_new, float scale, float *out,
                        hipStream_t s) {
  PrefillArgs a;
  a.kc = (const int8_t *)pool->run[0];
  a.ks = (const float *)pool->run[1];
  a.vq = (const uint8_t *)pool->run[2];
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
  dim3 grid((n_new + kPfPos - 1) / kPfPos, a.H);
  if (q_dtype == KV_DTYPE_F32)
    launch(attn_prefill_kernel<true>, grid, dim3(kPfWaves * 64), s, a);
  else
    launch(attn_prefill_kernel<false>, grid, dim3(kPfWaves * 64), s, a);
  return launch_status();
}

}  // namespace k8v4
