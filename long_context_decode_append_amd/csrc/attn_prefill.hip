// Causal prefill-chunk attention over a k8v4 pool, for gfx950.
//
// Computes, for n_new queries at positions [pos0, pos0 + n_new), the same
// attention as decode ("#120 --kv k8v4: hybrid KV cache -- INT8 K +
// Hadamard-rotated Q4_0 V (816 B/cell)", How: one fused attention serves
// decode, verify and prefill), row i attending cells [0, pos0 + i].
//
// Here Q.K^T and P.V are dense contractions (128 query rows share every K/V
// tile), so both run on the matrix cores (v_mfma_f32_16x16x32_f16):
//   * workgroup = 4 waves = 16 query positions x 8 GQA heads of one KV head
//     (128 rows); each wave owns 32 rows (2 row tiles of 16);
//   * per 32-cell tile the workgroup loads the raw pages once and
//     dequantizes into LDS: K codes as exact fp16 (scales kept per cell and
//     128-dim group, applied to the two half-dots), V as (code - 8) * d16 in
//     fp16, stored transposed [dim][cell] so the P.V B-operand is two 8-byte
//     reads;
//   * S^T = K.Q^T keeps P in registers in the P.V A-operand layout; online
//     softmax in base 2; causal mask only where the tile reaches the rows;
//   * epilogue: O / l, then the inverse Walsh-Hadamard transform across the
//     accumulator layout (dims 16j + n: 4 butterfly stages across lanes,
//     4 across registers).
#include "device.hpp"
#include "launch.hpp"

namespace k8v4 {

constexpr int kPfPos = 16;           // query positions per workgroup
constexpr int kPfTile = 32;          // cells per tile
constexpr int kKRow = 256 + 8;       // fp16 elements per K row in LDS (padded)
constexpr int kVRow = kPfTile + 4;   // fp16 elements per transposed V row (72 bytes)

struct PrefillArgs {
  const int8_t *kc;
  const float *ks;
  const uint8_t *vq;
  const int32_t *pt;
  const void *q;
  float *out;
  int n_pages, P, H;
  int n_q_heads;
  int pos0, n_new;
  float scale2;
};

template <bool QF32>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const PrefillArgs a) {
  __shared__ _Float16 lds_k[kPfTile * kKRow];
  __shared__ _Float16 lds_v[256 * kVRow];
  __shared__ float lds_ks[kPfTile * 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, lg = lane >> 4;
  const int g = blockIdx.y;
  const int qb0 = blockIdx.x * kPfPos;                    // first query (chunk-relative)
  const int q_last = min(qb0 + kPfPos, a.n_new) - 1;      // last valid query of the block
  const int n_cells = a.pos0 + q_last + 1;                // cells any row of the block sees

  // ---- queries: B operand of S^T = K.Q^T; row r = 32*wave + 16*t + n,
  // position qb0 + r/8, head g*8 + r%8; k-step kk holds dims 32kk + 8lg..+7
  f16x8 qop[2][8];
  f16x8 qlo[QF32 ? 2 : 1][QF32 ? 8 : 1];
  int qpos[2];
  bool rvalid[2];
  for (int t = 0; t < 2; t++) {
    const int r = 32 * wave + 16 * t + n;
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

  float m[2] = {-1e30f, -1e30f}, lsum[2] = {0.f, 0.f};
  f32x4 o[2][16];
  for (int t = 0; t < 2; t++)
    for (int j = 0; j < 16; j++) o[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t q4_tile = (size_t)144 * a.P;
  const f16x2 c1152 = {(_Float16)1152.0f, (_Float16)1152.0f};
  const f16x2 c1032 = {(_Float16)1032.0f, (_Float16)1032.0f};

  for (int c0 = 0; c0 < n_cells; c0 += kPfTile) {
    // ---------------- cooperative load + dequant into LDS
    {
      // K codes: thread -> cell tid/8, 32 bytes at 32*(tid%8)
      const int cl = tid >> 3, part = tid & 7;
      const int cell = c0 + cl;
      u32x4 w0 = {0u, 0u, 0u, 0u}, w1 = {0u, 0u, 0u, 0u};
      float d0 = 0.f, d1 = 0.f;
      uint32_t vd = 0;
      u32x4 vw = {0u, 0u, 0u, 0u};
      if (cell < n_cells) {
        int page = a.pt[cell / a.P];
        page = (page < 0 || page >= a.n_pages) ? 0 : page;
        const int slot = cell % a.P;
        const size_t tile = (size_t)page * a.H + g;
        const int8_t *kp = a.kc + (tile * a.P + slot) * 256 + 32 * part;
        w0 = *reinterpret_cast<const u32x4 *>(kp);
        w1 = *reinterpret_cast<const u32x4 *>(kp + 16);
        if (part < 2) {
          const float *ksp = a.ks + (tile * a.P + slot) * 2;
          d0 = ksp[part];
        }
        // V: block `part` of this cell: 16 nibble bytes + fp16 scale
        const uint8_t *vt = a.vq + tile * q4_tile;
        vw = *reinterpret_cast<const u32x4 *>(vt + (size_t)slot * 128 + 16 * part);
        vd = *reinterpret_cast<const uint16_t *>(vt + q4_scale_off(a.P, slot, part));
      }
      (void)d1;
      // K -> exact fp16 codes
      uint32_t kf[16];
      const uint32_t kw[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      for (int i = 0; i < 8; i++) {
        uint32_t lo, hi;
        i8x4_to_f16_biased(kw[i], lo, hi);
        kf[2 * i] = as_u32(as_f16x2(lo) - c1152);
        kf[2 * i + 1] = as_u32(as_f16x2(hi) - c1152);
      }
      _Float16 *kd = lds_k + cl * kKRow + 32 * part;
      for (int i = 0; i < 4; i++)
        *reinterpret_cast<u32x4 *>(kd + 8 * i) = u32x4{kf[4 * i], kf[4 * i + 1], kf[4 * i + 2], kf[4 * i + 3]};
      if (part < 2) lds_ks[cl * 2 + part] = d0;
      // V -> (code - 8) * d16 as fp16, transposed to [dim][cell]
      const f16x2 dd = as_f16x2(vd | (vd << 16));
      const uint32_t vwa[4] = {vw.x, vw.y, vw.z, vw.w};
      for (int i = 0; i < 4; i++) {
        // byte 4i + e: element 4i + e (low nibble) and 16 + 4i + e (high)
        const uint32_t x = vwa[i];
        for (int e = 0; e < 4; e++) {
          const uint32_t by = (x >> (8 * e)) & 0xffu;
          const uint32_t pr = (by & 15u) | ((by >> 4) << 16) | 0x64006400u;
          const f16x2 val = (as_f16x2(pr) - c1032) * dd;
          const int el = 4 * i + e;
          lds_v[(32 * part + el) * kVRow + cl] = val.x;
          lds_v[(32 * part + 16 + el) * kVRow + cl] = val.y;
        }
      }
    }
    __syncthreads();

    // ---------------- S^T = K . Q^T for 2 cell tiles x 2 row tiles
    float s[2][8];
    for (int ct = 0; ct < 2; ct++) {
      f16x8 kop[8];
      const _Float16 *kr = lds_k + (16 * ct + n) * kKRow + 8 * lg;
      for (int kk = 0; kk < 8; kk++) kop[kk] = *reinterpret_cast<const f16x8 *>(kr + 32 * kk);
      float dk[4][2];
      for (int i = 0; i < 4; i++) {
        dk[i][0] = lds_ks[(16 * ct + 4 * lg + i) * 2];
        dk[i][1] = lds_ks[(16 * ct + 4 * lg + i) * 2 + 1];
      }
      for (int t = 0; t < 2; t++) {
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < 4; kk++) {
          acc0 = mfma16x16x32(kop[kk], qop[t][kk], acc0);
          if (QF32) acc0 = mfma16x16x32(kop[kk], qlo[t][kk], acc0);
        }
        for (int kk = 4; kk < 8; kk++) {
          acc1 = mfma16x16x32(kop[kk], qop[t][kk], acc1);
          if (QF32) acc1 = mfma16x16x32(kop[kk], qlo[t][kk], acc1);
        }
        for (int i = 0; i < 4; i++) {
          const int cell = c0 + 16 * ct + 4 * lg + i;
          float sv = a.scale2 * (dk[i][0] * acc0[i] + dk[i][1] * acc1[i]);
          sv = (rvalid[t] && cell <= qpos[t]) ? sv : -INFINITY;
          s[t][4 * ct + i] = sv;
        }
      }
    }

    // ---------------- online softmax, P operand
    f16x8 pop[2];
    for (int t = 0; t < 2; t++) {
      float mx = s[t][0];
      for (int e = 1; e < 8; e++) mx = fmaxf(mx, s[t][e]);
      mx = fmaxf(mx, lane_xor(mx, 16));
      mx = fmaxf(mx, lane_xor(mx, 32));
      const float mnew = fmaxf(m[t], mx);
      const float alpha = exp2f(m[t] - mnew);
      float ps = 0.f;
      for (int e = 0; e < 8; e++) {
        const float p = exp2f(s[t][e] - mnew);
        ps += p;
        pop[t][e] = (_Float16)p;
      }
      lsum[t] = lsum[t] * alpha + ps;
      m[t] = mnew;
      float al[4];
      for (int i = 0; i < 4; i++) al[i] = lane_get(alpha, 4 * lg + i);
      for (int j = 0; j < 16; j++)
        for (int i = 0; i < 4; i++) o[t][j][i] *= al[i];
    }

    // ---------------- O += P . V; B for dim tile j, column n: dim 16j + n,
    // k-slots = cells 4lg + 0..3 and 16 + 4lg + 0..3
    for (int j = 0; j < 16; j++) {
      const _Float16 *vr = lds_v + (16 * j + n) * kVRow + 4 * lg;
      const u32x2 lo = *reinterpret_cast<const u32x2 *>(vr);
      const u32x2 hi = *reinterpret_cast<const u32x2 *>(vr + 16);
      const f16x8 B = __builtin_bit_cast(f16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
      for (int t = 0; t < 2; t++) o[t][j] = mfma16x16x32(pop[t], B, o[t][j]);
    }
    __syncthreads();
  }

  // ---------------- epilogue: normalize, inverse Walsh-Hadamard, store
  for (int t = 0; t < 2; t++) {
    lsum[t] += lane_xor(lsum[t], 16);
    lsum[t] += lane_xor(lsum[t], 32);
    float inv[4];
    for (int i = 0; i < 4; i++) inv[i] = 1.0f / lane_get(lsum[t], 4 * lg + i);
    // value (row 4lg + i, dim 16j + n) lives in o[t][j][i]
    float y[16][4];
    for (int j = 0; j < 16; j++)
      for (int i = 0; i < 4; i++) y[j][i] = o[t][j][i] * inv[i];
    // dim bits 0..3 = lane bits 0..3 (n): butterflies across lanes
    for (int mbit = 1; mbit < 16; mbit <<= 1) {
      const bool upper = (n & mbit) != 0;
      for (int j = 0; j < 16; j++)
        for (int i = 0; i < 4; i++) {
          const float p = lane_xor(y[j][i], mbit);
          y[j][i] = upper ? (p - y[j][i]) : (y[j][i] + p);
        }
    }
    // dim bits 4..7 = tile index j: butterflies across registers
    for (int jb = 1; jb < 16; jb <<= 1)
      for (int j = 0; j < 16; j++) {
        if (j & jb) continue;
        for (int i = 0; i < 4; i++) {
          const float x0 = y[j][i], x1 = y[j + jb][i];
          y[j][i] = x0 + x1;
          y[j + jb][i] = x0 - x1;
        }
      }
    for (int i = 0; i < 4; i++) {
      const int r = 32 * wave + 16 * t + 4 * lg + i;
      const int qi = qb0 + (r >> 3);
      if (qi > q_last) continue;
      float *op = a.out + ((size_t)qi * a.n_q_heads + (size_t)g * kGqa + (r & 7)) * 256;
      for (int j = 0; j < 16; j++) op[16 * j + n] = y[j][i] * 0.0625f;
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
  a.n_q_heads = n_q_heads;
  a.pos0 = pos0;
  a.n_new = n_new;
  a.scale2 = scale * 1.4426950408889634f;
  dim3 grid((n_new + kPfPos - 1) / kPfPos, a.H);
  if (q_dtype == KV_DTYPE_F32)
    launch(attn_prefill_kernel<true>, grid, dim3(256), s, a);
  else
    launch(attn_prefill_kernel<false>, grid, dim3(256), s, a);
  return launch_status();
}

}  // namespace k8v4
