// Split-K decode / verify attention over a k8v4 pool, for gfx950.
//
// What it computes follows "#120 --kv k8v4: hybrid KV cache -- INT8 K +
// Hadamard-rotated Q4_0 V (816 B/cell)", How and Tests: the fused attention
// gathers the pages through the page table, scores q against the unrotated
// INT8 K (K = code * d per 128-dim group), runs a softmax over the visible
// cells, accumulates the rotated Q4_0 V ((code - 8) * d16) and rotates the
// result back with H/16; the batched (verify) form gives each query row its
// own number of visible cells.
//
// Mapping onto MI355X:
//   * grid (splits, KV heads, row passes); a workgroup = 4 waves owns one
//     contiguous logical cell range ("split"), its waves take 32-cell steps
//     round robin.  The split plan depends only on the context length, so
//     identity and permuted page tables give bitwise-equal outputs.
//   * per step a wave loads K codes / K scales / V nibbles / V scales
//     straight into registers in the operand layouts of
//     v_mfma_f32_16x16x32_f16 (16-byte K loads, 8-byte V loads), converts
//     the codes to fp16 in registers (K exactly, biased by +1152 with the
//     bias removed from the score; V as (code - 8) * d16) and runs
//       S^T[cells x rows] = K[cells x dims] . Q^T        (8 MFMA / 16 cells)
//       O[rows x dims]   += P[rows x cells] . V[cells x dims]  (16 MFMA / 32 cells)
//     The GQA group (8 query heads of a KV head) and the verify rows form
//     the 16-wide row tiles, so the QK output already sits in the layout the
//     PV A-operand needs and P never leaves registers.
//   * online softmax in base 2 with fp32 running max / sum per row.
//   * the 4 wave states merge through LDS in fixed order, then the
//     workgroup writes one partial (m, l, O) per row; arrival counters pick
//     the last workgroup of each group of 16 splits to merge the group, and
//     the last group merger per (KV head, row pass) merges the groups in
//     fixed order, normalizes and applies the inverse Walsh-Hadamard
//     transform.  No float atomics: results are deterministic.
#include "device.hpp"
#include "launch.hpp"

namespace k8v4 {


struct SplitArgs {
  const int8_t *kc;
  const float *ks;
  const uint8_t *vq;
  const int32_t *pt;
  const void *q;
  float *out;
  uint32_t *counters;   // [passes][H][kCounterStride]
  float2 *part_ml;      // [H][splits][rows]
  float *part_o;        // [H][splits][rows][256]
  float2 *grp_ml;       // [H][groups][rows]
  float *grp_o;         // [H][groups][rows][256]
  int n_pages, P, H;
  int n_q_heads, n_rows, rows_per_pass;
  int limits[kMaxQ];
  int max_limit;
  float scale2;         // softmax scale * log2(e)
  int steps_per_split, n_splits, n_groups;
};

// dim of output tile j held by column n of the PV MFMA: column n reads bytes
// [8n, 8n+8) of a cell's 128 nibble bytes (block n/2), tile j takes byte
// j % 8, low nibble for j < 8 and high nibble for j >= 8.
__device__ __forceinline__ int o_dim(int n, int j) {
  return 32 * (n >> 1) + 8 * (n & 1) + (j & 7) + 16 * (j >> 3);
}

__device__ __forceinline__ f16x8 pack8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 u = {a, b, c, d};
  return __builtin_bit_cast(f16x8, u);
}

// merge the (m, l, O) rows [row0, row0+rows) of `count` partials into one
__device__ __forceinline__ void merge_rows(const float2 *src_ml, const float *src_o, int count,
                                           int stride_rows, int row0, int rows, float2 *dst_ml,
                                           float *dst_o, int lane, int wave) {
  for (int r = wave; r < rows; r += kWaves) {
    const int row = row0 + r;
    float M = -1e30f;
    for (int s = 0; s < count; s++) M = fmaxf(M, src_ml[(size_t)s * stride_rows + row].x);
    float L = 0.0f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < count; s++) {
      const float2 ml = src_ml[(size_t)s * stride_rows + row];
      const float f = exp2f(ml.x - M);
      L += ml.y * f;
      const f32x4 o = *reinterpret_cast<const f32x4 *>(src_o + ((size_t)s * stride_rows + row) * 256 + 4 * lane);
      acc += f * o;
    }
    if (lane == 0) dst_ml[row] = make_float2(M, L);
    *reinterpret_cast<f32x4 *>(dst_o + (size_t)row * 256 + 4 * lane) = acc;
  }
}

template <int NQT, bool QF32>
__global__ __launch_bounds__(256) void attn_splitk_kernel(const SplitArgs a) {
  __shared__ float lds_o[NQT * 16 * 256];
  __shared__ float lds_m[NQT * 16];
  __shared__ float lds_l[NQT * 16];
  __shared__ int lds_flag;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, lg = lane >> 4;
  const int split = blockIdx.x, g = blockIdx.y, pass = blockIdx.z;
  const int row_base = pass * a.rows_per_pass;
  const int rows_here = min(a.rows_per_pass, a.n_rows - row_base);

  // ---------------------------------------------------------------- queries
  // B operand of the QK MFMA for row tile t and k-step kk: lane (n, lg)
  // holds q[row t*16+n][dims 64*(kk/2) + 16*lg + 8*(kk%2) + 0..7].
  f16x8 qop[NQT][8];
  f16x8 qlo[QF32 ? NQT : 1][QF32 ? 8 : 1];
  float cbias[NQT][2];
  int lim[NQT];
  for (int t = 0; t < NQT; t++) {
    const int r = t * 16 + n;
    const int row = row_base + r;
    const bool rv = r < rows_here;
    lim[t] = rv ? a.limits[row >> 3] : 0;
    const int qi = row >> 3, hl = row & 7;
    const size_t qbase = ((size_t)qi * a.n_q_heads + (size_t)g * kGqa + hl) * 256;
    float s0 = 0.f, s1 = 0.f;
    for (int kk = 0; kk < 8; kk++) {
      const int d0 = 64 * (kk >> 1) + 16 * lg + 8 * (kk & 1);
      f16x8 hi, lo;
      if (!QF32) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (rv) w = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.q) + qbase + d0);
        hi = __builtin_bit_cast(f16x8, w);
        float ss = 0.f;
        for (int e = 0; e < 8; e++) ss += (float)hi[e];
        if (kk < 4) s0 += ss; else s1 += ss;
      } else {
        f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
        if (rv) {
          x0 = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(a.q) + qbase + d0);
          x1 = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(a.q) + qbase + d0 + 4);
        }
        float ss = 0.f;
        for (int e = 0; e < 8; e++) {
          const float x = e < 4 ? x0[e] : x1[e - 4];
          const _Float16 h = (_Float16)x;
          const _Float16 l = (_Float16)(x - (float)h);
          hi[e] = h;
          lo[e] = l;
          ss += (float)h + (float)l;
        }
        if (kk < 4) s0 += ss; else s1 += ss;
      }
      qop[t][kk] = hi;
      if (QF32) qlo[t][kk] = lo;
    }
    s0 += lane_xor(s0, 16);
    s0 += lane_xor(s0, 32);
    s1 += lane_xor(s1, 16);
    s1 += lane_xor(s1, 32);
    cbias[t][0] = 1152.0f * s0;
    cbias[t][1] = 1152.0f * s1;
  }

  // ---------------------------------------------------------------- main loop
  float m[NQT], lsum[NQT];
  f32x4 o[NQT][16];
  for (int t = 0; t < NQT; t++) {
    m[t] = -1e30f;
    lsum[t] = 0.f;
    for (int j = 0; j < 16; j++) o[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int c_begin = split * a.steps_per_split * kStep;
  const int c_end = min(a.max_limit, c_begin + a.steps_per_split * kStep);
  int lim_eff[NQT];
  for (int t = 0; t < NQT; t++) lim_eff[t] = min(lim[t], c_end);
  const size_t q4_tile = (size_t)144 * a.P;

  for (int c0 = c_begin + wave * kStep; c0 < c_end; c0 += kWaves * kStep) {
    u32x4 kraw[2][4];
    f32x4 ksr[2][2];
    u32x2 vraw[2][4];
    u32x2 vdr[2];
    bool badp[2];
    for (int h2 = 0; h2 < 2; h2++) {
      const int cb = c0 + 16 * h2;
      const int cl = cb < c_end ? cb : c0;  // a half past the end reads (masked) cells of c0's page
      int page = a.pt[cl / a.P];
      badp[h2] = page < 0 || page >= a.n_pages;
      page = badp[h2] ? 0 : page;
      const int slot0 = cl % a.P;
      const size_t tile = (size_t)page * a.H + g;
      const int8_t *kp = a.kc + (tile * a.P + slot0 + n) * 256 + 16 * lg;
      for (int j = 0; j < 4; j++) kraw[h2][j] = *reinterpret_cast<const u32x4 *>(kp + 64 * j);
      const float *ksp = a.ks + (tile * a.P + slot0 + 4 * lg) * 2;
      ksr[h2][0] = *reinterpret_cast<const f32x4 *>(ksp);
      ksr[h2][1] = *reinterpret_cast<const f32x4 *>(ksp + 4);
      const uint8_t *vt = a.vq + tile * q4_tile;
      for (int i = 0; i < 4; i++)
        vraw[h2][i] = *reinterpret_cast<const u32x2 *>(vt + (size_t)(slot0 + 4 * lg + i) * 128 + 8 * n);
      vdr[h2] = *reinterpret_cast<const u32x2 *>(vt + (size_t)128 * a.P + ((size_t)(n >> 1) * a.P + slot0 + 4 * lg) * 2);
    }

    // ---- scores S^T = K . Q^T  (A = K codes + 1152 as fp16, B = q)
    float s[NQT][8];
    for (int h2 = 0; h2 < 2; h2++) {
      f16x8 kf[8];
      for (int j = 0; j < 4; j++) {
        uint32_t l0, h0, l1, h1, l2, h2w, l3, h3;
        i8x4_to_f16_biased(kraw[h2][j].x, l0, h0);
        i8x4_to_f16_biased(kraw[h2][j].y, l1, h1);
        i8x4_to_f16_biased(kraw[h2][j].z, l2, h2w);
        i8x4_to_f16_biased(kraw[h2][j].w, l3, h3);
        kf[2 * j] = pack8(l0, h0, l1, h1);
        kf[2 * j + 1] = pack8(l2, h2w, l3, h3);
      }
      for (int t = 0; t < NQT; t++) {
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < 4; kk++) {
          acc0 = mfma16x16x32(kf[kk], qop[t][kk], acc0);
          if (QF32) acc0 = mfma16x16x32(kf[kk], qlo[t][kk], acc0);
        }
        for (int kk = 4; kk < 8; kk++) {
          acc1 = mfma16x16x32(kf[kk], qop[t][kk], acc1);
          if (QF32) acc1 = mfma16x16x32(kf[kk], qlo[t][kk], acc1);
        }
        for (int i = 0; i < 4; i++) {
          const f32x4 kq = ksr[h2][i >> 1];
          const float d0 = kq[2 * (i & 1)], d1 = kq[2 * (i & 1) + 1];
          float sv = a.scale2 * (d0 * (acc0[i] - cbias[t][0]) + d1 * (acc1[i] - cbias[t][1]));
          const int cell = c0 + 16 * h2 + 4 * lg + i;
          sv = cell < lim_eff[t] ? sv : -INFINITY;
          sv = badp[h2] ? __builtin_nanf("") : sv;
          s[t][4 * h2 + i] = sv;
        }
      }
    }

    // ---- online softmax (base 2) and the P operand
    f16x8 pop[NQT];
    for (int t = 0; t < NQT; t++) {
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
      // O rows in the accumulator layout are 4*lg + i: fetch their factor
      float al[4];
      for (int i = 0; i < 4; i++) al[i] = lane_get(alpha, 4 * lg + i);
      for (int j = 0; j < 16; j++)
        for (int i = 0; i < 4; i++) o[t][j][i] *= al[i];
    }

    // ---- O += P . V  (B = (code - 8) * d16 in fp16, 4 tiles per byte pair)
    uint32_t dsc[4];
    for (int k = 0; k < 4; k++) {
      const int h2 = k >> 1;
      uint32_t w = (k & 1) ? vdr[h2].y : vdr[h2].x;
      const int ca = c0 + 16 * h2 + 4 * lg + 2 * (k & 1);
      if (ca >= c_end) w &= 0xffff0000u;      // zero the scale of cells past the split
      if (ca + 1 >= c_end) w &= 0x0000ffffu;
      dsc[k] = w;
    }
    for (int grp = 0; grp < 4; grp++) {
      const int dw = grp >> 1;
      const uint32_t sel = (grp & 1) ? 0x07060302u : 0x05040100u;
      uint32_t b0[4], b1[4], b2[4], b3[4];
      for (int k = 0; k < 4; k++) {
        const int h2 = k >> 1, ia = 2 * (k & 1);
        const uint32_t wa = dw ? vraw[h2][ia].y : vraw[h2][ia].x;
        const uint32_t wb = dw ? vraw[h2][ia + 1].y : vraw[h2][ia + 1].x;
        const uint32_t x = perm(wb, wa, sel);  // [a.byte, a.byte+1, b.byte, b.byte+1]
        const f16x2 dd = as_f16x2(dsc[k]);
        const f16x2 c1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
        b0[k] = as_u32((as_f16x2((x & 0x000F000Fu) | 0x64006400u) - c1032) * dd);
        b1[k] = as_u32((as_f16x2(((x >> 4) & 0x000F000Fu) | 0x64006400u) - c1032) * dd);
        b2[k] = as_u32((as_f16x2(((x >> 8) & 0x000F000Fu) | 0x64006400u) - c1032) * dd);
        b3[k] = as_u32((as_f16x2(((x >> 12) & 0x000F000Fu) | 0x64006400u) - c1032) * dd);
      }
      const int jb = 2 * grp;
      const f16x8 B0 = pack8(b0[0], b0[1], b0[2], b0[3]);  // tile jb     (byte lo nibble)
      const f16x8 B1 = pack8(b1[0], b1[1], b1[2], b1[3]);  // tile jb + 8 (byte hi nibble)
      const f16x8 B2 = pack8(b2[0], b2[1], b2[2], b2[3]);  // tile jb + 1
      const f16x8 B3 = pack8(b3[0], b3[1], b3[2], b3[3]);  // tile jb + 9
      for (int t = 0; t < NQT; t++) {
        o[t][jb] = mfma16x16x32(pop[t], B0, o[t][jb]);
        o[t][jb + 8] = mfma16x16x32(pop[t], B1, o[t][jb + 8]);
        o[t][jb + 1] = mfma16x16x32(pop[t], B2, o[t][jb + 1]);
        o[t][jb + 9] = mfma16x16x32(pop[t], B3, o[t][jb + 9]);
      }
    }
  }

  // ---------------------------------------------------------------- workgroup merge
  for (int t = 0; t < NQT; t++) {
    lsum[t] += lane_xor(lsum[t], 16);
    lsum[t] += lane_xor(lsum[t], 32);
  }
  for (int w = 0; w < kWaves; w++) {
    if (wave == w) {
      for (int t = 0; t < NQT; t++) {
        float fo[4], fw[4];
        float mold = 0.f, lold = 0.f, mn = m[t];
        if (w > 0) {
          mold = lds_m[t * 16 + n];
          lold = lds_l[t * 16 + n];
          mn = fmaxf(mold, m[t]);
        }
        const float a_old = w > 0 ? exp2f(mold - mn) : 0.f;
        const float a_new = exp2f(m[t] - mn);
        for (int i = 0; i < 4; i++) {
          fo[i] = lane_get(a_old, 4 * lg + i);
          fw[i] = lane_get(a_new, 4 * lg + i);
        }
        if (lg == 0) {
          lds_m[t * 16 + n] = mn;
          lds_l[t * 16 + n] = lold * a_old + lsum[t] * a_new;
        }
        for (int j = 0; j < 16; j++) {
          const int dim = o_dim(n, j);
          for (int i = 0; i < 4; i++) {
            float *p = &lds_o[(t * 16 + 4 * lg + i) * 256 + dim];
            *p = (w > 0 ? *p * fo[i] : 0.f) + o[t][j][i] * fw[i];
          }
        }
      }
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- partial out
  const int H = a.H;
  const size_t rows_total = (size_t)a.n_rows;
  {
    const size_t sp = (size_t)g * a.n_splits + split;
    for (int idx = threadIdx.x; idx < rows_here * 64; idx += 256) {
      const int r = idx >> 6, c = (idx & 63) * 4;
      const f32x4 v = *reinterpret_cast<const f32x4 *>(&lds_o[r * 256 + c]);
      *reinterpret_cast<f32x4 *>(a.part_o + (sp * rows_total + row_base + r) * 256 + c) = v;
    }
    for (int r = threadIdx.x; r < rows_here; r += 256)
      a.part_ml[sp * rows_total + row_base + r] = make_float2(lds_m[r], lds_l[r]);
  }

  // ---------------------------------------------------------------- first-level combine
  uint32_t *cnt = a.counters + ((size_t)pass * H + g) * kCounterStride;
  const int grp = split / kGroup;
  const int gsize = min(kGroup, a.n_splits - grp * kGroup);
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(&cnt[grp], 1u);
    lds_flag = (prev == (uint32_t)(gsize - 1));
  }
  __syncthreads();
  if (!lds_flag) return;
  __threadfence();
  {
    const size_t s0 = (size_t)g * a.n_splits + (size_t)grp * kGroup;
    const size_t gi = (size_t)g * a.n_groups + grp;
    merge_rows(a.part_ml + s0 * rows_total, a.part_o + s0 * rows_total * 256, gsize, (int)rows_total,
               row_base, rows_here, a.grp_ml + gi * rows_total, a.grp_o + gi * rows_total * 256,
               lane, wave);
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicExch(&cnt[grp], 0u);
    const uint32_t prev = atomicAdd(&cnt[kCounterStride - 1], 1u);
    lds_flag = (prev == (uint32_t)(a.n_groups - 1));
  }
  __syncthreads();
  if (!lds_flag) return;
  __threadfence();

  // ---------------------------------------------------------------- final combine
  for (int r = wave; r < rows_here; r += kWaves) {
    const int row = row_base + r;
    const float2 *gml = a.grp_ml + (size_t)g * a.n_groups * rows_total;
    const float *go = a.grp_o + (size_t)g * a.n_groups * rows_total * 256;
    float M = -1e30f;
    for (int q = 0; q < a.n_groups; q++) M = fmaxf(M, gml[(size_t)q * rows_total + row].x);
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < a.n_groups; q++) {
      const float2 ml = gml[(size_t)q * rows_total + row];
      const float f = exp2f(ml.x - M);
      L += ml.y * f;
      acc += f * *reinterpret_cast<const f32x4 *>(go + ((size_t)q * rows_total + row) * 256 + 4 * lane);
    }
    float y[4];
    const float inv = 1.0f / L;
    for (int i = 0; i < 4; i++) y[i] = acc[i] * inv;
    fwht256_lane4(y, lane);
    const int qi = row >> 3, hl = row & 7;
    float *op = a.out + ((size_t)qi * a.n_q_heads + (size_t)g * kGqa + hl) * 256 + 4 * lane;
    *reinterpret_cast<f32x4 *>(op) = f32x4{y[0], y[1], y[2], y[3]};
  }
  if (threadIdx.x == 0) atomicExch(&cnt[kCounterStride - 1], 0u);
}

// ---------------------------------------------------------------- host side

template <int NQT, bool QF32>
static const void *kernel_ptr() {
  return reinterpret_cast<const void *>(&attn_splitk_kernel<NQT, QF32>);
}

int attn_target_splits(int n_kv_heads, int n_rows) {
  static int cached_dev = -1, cached_cus = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 64;
  if (dev != cached_dev) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 64;
    cached_cus = prop.multiProcessorCount;
    cached_dev = dev;
  }
  (void)n_rows;
  int per_head = cached_cus / (n_kv_heads > 0 ? n_kv_heads : 1);
  return per_head < 1 ? 1 : per_head;
}

int launch_attn_splitk(const AttnCall &c) {
  const kv_pool *pool = c.pool;
  const int H = pool->n_kv_heads;
  const int n_rows = c.n_q * kGqa;
  const bool qf32 = c.q_dtype == KV_DTYPE_F32;
  const int tiles = (n_rows + 15) / 16;
  const int nqt = qf32 ? 1 : (tiles < 3 ? tiles : 3);
  const int rows_per_pass = nqt * 16;
  const int passes = (n_rows + rows_per_pass - 1) / rows_per_pass;
  const SplitPlan plan = plan_splits(c.max_limit, attn_target_splits(H, n_rows));
  const WsLayout ws = ws_layout(H, n_rows, plan.n_splits, plan.n_groups);
  if (ws.total > c.ws_bytes) return KV_ERR_WORKSPACE;
  if (passes > kMaxPasses) return KV_ERR_UNSUPPORTED;

  SplitArgs a;
  char *base = (char *)c.ws;
  a.kc = (const int8_t *)pool->run[0];
  a.ks = (const float *)pool->run[1];
  a.vq = (const uint8_t *)pool->run[2];
  a.pt = c.seq->page_table;
  a.q = c.q;
  a.out = c.out;
  a.counters = (uint32_t *)(base + ws.counters);
  a.part_ml = (float2 *)(base + ws.part_ml);
  a.part_o = (float *)(base + ws.part_o);
  a.grp_ml = (float2 *)(base + ws.grp_ml);
  a.grp_o = (float *)(base + ws.grp_o);
  a.n_pages = pool->n_pages;
  a.P = pool->page_size;
  a.H = H;
  a.n_q_heads = c.n_q_heads;
  a.n_rows = n_rows;
  a.rows_per_pass = rows_per_pass;
  for (int i = 0; i < kMaxQ; i++) a.limits[i] = i < c.n_q ? c.limits[i] : 0;
  a.max_limit = c.max_limit;
  a.scale2 = c.scale * 1.4426950408889634f;
  a.steps_per_split = plan.steps_per_split;
  a.n_splits = plan.n_splits;
  a.n_groups = plan.n_groups;

  dim3 grid(plan.n_splits, H, passes);
  if (qf32) {
    hipLaunchKernelGGL((attn_splitk_kernel<1, true>), grid, dim3(256), 0, c.stream, a);
  } else if (nqt == 1) {
    hipLaunchKernelGGL((attn_splitk_kernel<1, false>), grid, dim3(256), 0, c.stream, a);
  } else if (nqt == 2) {
    hipLaunchKernelGGL((attn_splitk_kernel<2, false>), grid, dim3(256), 0, c.stream, a);
  } else {
    hipLaunchKernelGGL((attn_splitk_kernel<3, false>), grid, dim3(256), 0, c.stream, a);
  }
  return launch_status();
}

}  // namespace k8v4
