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
//     contiguous logical cell range ("split") and one tile of 16 query rows
//     (decode: the 8 heads of the KV head; verify: 2 queries per pass), its
//     waves take 32-cell steps round robin, the loads of a wave's next step
//     in flight while it computes the current one.  The split plan depends only on the context length, so
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
//     transform.  No float atomics: results are deterministic.  Partials
//     move between workgroups through device-scope (L2-bypassing) 8-byte
//     accesses, so no cache write-back fences are needed.
#include "device.hpp"
#include "launch.hpp"

namespace k8v4 {

constexpr float kLazy = 8.0f;  // log2 headroom of the lazy softmax reference


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

// Raw operands of one 32-cell step of one wave, as loaded from the pool.
struct StepRaw {
  u32x4 k[2][4];   // K codes: half h2, 16-byte chunk j (cell n, bytes 64j + 16lg ..)
  f32x4 ks[2][2];  // K scales of cells 4lg..4lg+3 of half h2, groups 0/1 interleaved
  u32x2 v[2][4];   // V nibbles: cell 4lg+i of half h2, bytes [8n, 8n+8) of its 128
  u32x2 vd[2];     // V scales d16[block n/2][cells 4lg..4lg+3] of half h2
};

// Logical position whose page serves half h2 of the step at c: a half that
// starts past the split end reuses the step's first half (its cells are
// masked and its V scales zeroed).
__device__ __forceinline__ int half_pos(int c, int h2, int c_end) {
  const int cb = c + 16 * h2;
  return cb < c_end ? cb : c;
}

// Page-table entries of the two halves of the step at c (wave-uniform:
// scalar loads).  Steps past the end are clamped to a valid entry.
__device__ __forceinline__ int2 step_pages(const SplitArgs &a, int c, int c_end) {
  const int cl = min(c, c_end - 1);
  const int p0 = a.pt[cl / a.P];
  const int p1 = a.pt[half_pos(cl, 1, c_end) / a.P];
  return make_int2(p0, p1);
}

__device__ __forceinline__ bool page_bad(const SplitArgs &a, int p) { return p < 0 || p >= a.n_pages; }

__device__ __forceinline__ void issue_step(StepRaw &d, const SplitArgs &a, int g, int c, int c_end,
                                           int2 pg, int n, int lg) {
  const size_t q4_tile = (size_t)144 * a.P;
  for (int h2 = 0; h2 < 2; h2++) {
    int page = h2 ? pg.y : pg.x;
    page = page_bad(a, page) ? 0 : page;
    const int slot0 = half_pos(c, h2, c_end) % a.P;
    const size_t tile = (size_t)page * a.H + g;
    const int8_t *kp = a.kc + (tile * a.P + slot0 + n) * 256 + 16 * lg;
    for (int j = 0; j < 4; j++) d.k[h2][j] = *reinterpret_cast<const u32x4 *>(kp + 64 * j);
    const float *ksp = a.ks + (tile * a.P + slot0 + 4 * lg) * 2;
    d.ks[h2][0] = *reinterpret_cast<const f32x4 *>(ksp);
    d.ks[h2][1] = *reinterpret_cast<const f32x4 *>(ksp + 4);
    const uint8_t *vt = a.vq + tile * q4_tile;
    for (int i = 0; i < 4; i++)
      d.v[h2][i] = *reinterpret_cast<const u32x2 *>(vt + (size_t)(slot0 + 4 * lg + i) * 128 + 8 * n);
    d.vd[h2] = *reinterpret_cast<const u32x2 *>(vt + (size_t)128 * a.P +
                                                 ((size_t)(n >> 1) * a.P + slot0 + 4 * lg) * 2);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Partials cross workgroups (and XCDs, whose L2s are not coherent with each
// other) through device-scope relaxed 8-byte atomic stores and loads: the
// device scope bit makes them write through / miss the per-XCD L2, so no
// L2 write-back or invalidate fence is needed.  A writer waits for its
// stores to complete before the arrival counter is bumped; the last arrival
// reads them after the counter returns.
__device__ __forceinline__ void st_dev2(void *p, float x, float y) {
  const uint64_t u = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
  __hip_atomic_store((uint64_t *)p, u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_dev2(const void *p) {
  const uint64_t u = __hip_atomic_load((uint64_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
}
__device__ __forceinline__ void st_dev4(float *p, f32x4 v) {
  st_dev2(p, v.x, v.y);
  st_dev2(p + 2, v.z, v.w);
}
__device__ __forceinline__ f32x4 ld_dev4(const float *p) {
  const float2 a = ld_dev2(p), b = ld_dev2(p + 2);
  return f32x4{a.x, a.y, b.x, b.y};
}
// wait until every memory access this wave issued has completed
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ float readlane(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Wave-level merge of `count` (<= 64) partial (m, l, O) rows for one row:
// lane s reads partial s's (m, l); the O rows are loaded 8 at a time before
// being combined in ascending partial order (deterministic).
__device__ __forceinline__ void merge_row(const float2 *ml_base, const float *o_base, int count,
                                          size_t stride_rows, int row, int lane, float &M_out,
                                          float &L_out, f32x4 &acc_out) {
  float2 ml = make_float2(-1e30f, 0.f);
  if (lane < count) ml = ld_dev2(ml_base + (size_t)lane * stride_rows + row);
  float M = ml.x;
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, lane_xor(M, m));
  const float w = lane < count ? fast_exp2(ml.x - M) : 0.f;
  float L = w * ml.y;
  for (int m = 32; m >= 1; m >>= 1) L += lane_xor(L, m);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < count; s0 += 8) {
    f32x4 o[8];
    for (int i = 0; i < 8; i++)
      if (s0 + i < count)
        o[i] = ld_dev4(o_base + ((size_t)(s0 + i) * stride_rows + row) * 256 + 4 * lane);
    for (int i = 0; i < 8; i++)
      if (s0 + i < count) acc += readlane(w, s0 + i) * o[i];
  }
  M_out = M;
  L_out = L;
  acc_out = acc;
}

template <int NQT, bool QF32>
__global__ __launch_bounds__(256) void attn_splitk_kernel(const SplitArgs a) {
  __shared__ float lds_o[NQT * 16 * 256];
  __shared__ float lds_m[NQT * 16];
  __shared__ float lds_l[NQT * 16];
  __shared__ int lds_flag;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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

  // one 32-cell step: scores, online softmax, P.V
  auto compute = [&](const StepRaw &d, int c0, int2 pg) {
    const bool badp[2] = {page_bad(a, pg.x), page_bad(a, pg.y)};
    float s[NQT][8];
    for (int h2 = 0; h2 < 2; h2++) {
      f16x8 kf[8];
      for (int j = 0; j < 4; j++) {
        uint32_t l0, h0, l1, h1, l2, h2w, l3, h3;
        i8x4_to_f16_biased(d.k[h2][j].x, l0, h0);
        i8x4_to_f16_biased(d.k[h2][j].y, l1, h1);
        i8x4_to_f16_biased(d.k[h2][j].z, l2, h2w);
        i8x4_to_f16_biased(d.k[h2][j].w, l3, h3);
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
          const f32x4 kq = d.ks[h2][i >> 1];
          const float d0 = kq[2 * (i & 1)], d1 = kq[2 * (i & 1) + 1];
          float sv = a.scale2 * (d0 * (acc0[i] - cbias[t][0]) + d1 * (acc1[i] - cbias[t][1]));
          const int cell = c0 + 16 * h2 + 4 * lg + i;
          sv = cell < lim_eff[t] ? sv : -INFINITY;
          sv = badp[h2] ? __builtin_nanf("") : sv;
          s[t][4 * h2 + i] = sv;
        }
      }
    }

    // online softmax against a reference max m[t] that only moves when a
    // row's max exceeds it by more than 2^kLazy: p <= 2^kLazy stays exact
    // enough in fp16 and the 64 accumulators are rarely touched
    f16x8 pop[NQT];
    for (int t = 0; t < NQT; t++) {
      float mx = s[t][0];
      for (int e = 1; e < 8; e++) mx = fmaxf(mx, s[t][e]);
      mx = fmaxf(mx, lane_xor(mx, 16));
      mx = fmaxf(mx, lane_xor(mx, 32));
      if (__any(mx > m[t] + kLazy)) {
        const float mnew = fmaxf(m[t], mx);
        const float alpha = fast_exp2(m[t] - mnew);
        lsum[t] *= alpha;
        m[t] = mnew;
        // O rows in the accumulator layout are 4*lg + i: fetch their factor
        float al[4];
        for (int i = 0; i < 4; i++) al[i] = lane_get(alpha, 4 * lg + i);
        for (int j = 0; j < 16; j++)
          for (int i = 0; i < 4; i++) o[t][j][i] *= al[i];
      }
      float ps = 0.f;
      for (int e = 0; e < 8; e++) {
        const float p = fast_exp2(s[t][e] - m[t]);
        ps += p;
        pop[t][e] = (_Float16)p;
      }
      lsum[t] += ps;
    }

    uint32_t dsc[4];
    for (int k = 0; k < 4; k++) {
      const int h2 = k >> 1;
      uint32_t w = (k & 1) ? d.vd[h2].y : d.vd[h2].x;
      const int ca = c0 + 16 * h2 + 4 * lg + 2 * (k & 1);
      if (ca >= c_end) w &= 0xffff0000u;      // zero the scale of cells past the split
      if (ca + 1 >= c_end) w &= 0x0000ffffu;
      dsc[k] = w;
    }
    const f16x2 c1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
    for (int grp = 0; grp < 4; grp++) {
      const int dw = grp >> 1;
      const uint32_t sel = (grp & 1) ? 0x07060302u : 0x05040100u;
      uint32_t b0[4], b1[4], b2[4], b3[4];
      for (int k = 0; k < 4; k++) {
        const int h2 = k >> 1, ia = 2 * (k & 1);
        const uint32_t wa = dw ? d.v[h2][ia].y : d.v[h2][ia].x;
        const uint32_t wb = dw ? d.v[h2][ia + 1].y : d.v[h2][ia + 1].x;
        const uint32_t x = perm(wb, wa, sel);  // [a.byte, a.byte+1, b.byte, b.byte+1]
        const f16x2 dd = as_f16x2(dsc[k]);
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
  };

  // two register buffers: the loads of the next step are in flight while
  // the current one is computed; page-table entries are read two steps
  // ahead.  The prefetch is issued unconditionally (a step past the end
  // re-reads the wave's last valid step) so every wait for the current
  // step's data leaves the next step's loads outstanding.
  {
    const int stride = kWaves * kStep;
    const int c_first = c_begin + wave * kStep;
    if (c_first < c_end) {
      // last step start of this wave (wave-uniform)
      const int c_last = c_first + ((c_end - 1 - c_first) / stride) * stride;
      StepRaw A, B;
      int c = c_first;
      int2 pgA = step_pages(a, c, c_end);
      issue_step(A, a, g, c, c_end, pgA, n, lg);
      int2 pgB = step_pages(a, min(c + stride, c_last), c_end);
      while (true) {
        const int cn = c + stride;
        issue_step(B, a, g, min(cn, c_last), c_end, pgB, n, lg);
        const int2 pgA_next = step_pages(a, min(cn + stride, c_last), c_end);
        compute(A, c, pgA);
        c = cn;
        if (c > c_last) break;
        const int cn2 = c + stride;
        issue_step(A, a, g, min(cn2, c_last), c_end, pgA_next, n, lg);
        const int2 pgB_next = step_pages(a, min(cn2 + stride, c_last), c_end);
        compute(B, c, pgB);
        c = cn2;
        if (c > c_last) break;
        pgA = pgA_next;
        pgB = pgB_next;
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
        const float a_old = w > 0 ? fast_exp2(mold - mn) : 0.f;
        const float a_new = fast_exp2(m[t] - mn);
        for (int i = 0; i < 4; i++) {
          fo[i] = lane_get(a_old, 4 * lg + i);
          fw[i] = lane_get(a_new, 4 * lg + i);
        }
        if (lg == 0) {
          lds_m[t * 16 + n] = mn;
          lds_l[t * 16 + n] = lold * a_old + lsum[t] * a_new;
        }
        if (t * 16 + 4 * lg < rows_here) {
          for (int j = 0; j < 16; j++) {
            const int dim = o_dim(n, j);
            for (int i = 0; i < 4; i++) {
              float *p = &lds_o[(t * 16 + 4 * lg + i) * 256 + dim];
              *p = (w > 0 ? *p * fo[i] : 0.f) + o[t][j][i] * fw[i];
            }
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
      st_dev4(a.part_o + (sp * rows_total + row_base + r) * 256 + c, v);
    }
    for (int r = threadIdx.x; r < rows_here; r += 256)
      st_dev2(a.part_ml + sp * rows_total + row_base + r, lds_m[r], lds_l[r]);
  }

  // ---------------------------------------------------------------- first-level combine
  // every wave's partial stores complete before the arrival is counted
  uint32_t *cnt = a.counters + ((size_t)pass * H + g) * kCounterStride;
  const int grp = split / kGroup;
  const int gsize = min(kGroup, a.n_splits - grp * kGroup);
  wait_all_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(&cnt[grp], 1u);
    lds_flag = (prev == (uint32_t)(gsize - 1));
  }
  __syncthreads();
  if (!lds_flag) return;
  {
    const size_t s0 = (size_t)g * a.n_splits + (size_t)grp * kGroup;
    const size_t gi = (size_t)g * a.n_groups + grp;
    for (int r = wave; r < rows_here; r += kWaves) {
      const int row = row_base + r;
      float M, L;
      f32x4 acc;
      merge_row(a.part_ml + s0 * rows_total, a.part_o + s0 * rows_total * 256, gsize, rows_total,
                row, lane, M, L, acc);
      if (lane == 0) st_dev2(a.grp_ml + gi * rows_total + row, M, L);
      st_dev4(a.grp_o + (gi * rows_total + row) * 256 + 4 * lane, acc);
    }
  }
  wait_all_memory();
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicExch(&cnt[grp], 0u);
    const uint32_t prev = atomicAdd(&cnt[kCounterStride - 1], 1u);
    lds_flag = (prev == (uint32_t)(a.n_groups - 1));
  }
  __syncthreads();
  if (!lds_flag) return;

  // ---------------------------------------------------------------- final combine
  for (int r = wave; r < rows_here; r += kWaves) {
    const int row = row_base + r;
    const size_t g0 = (size_t)g * a.n_groups;
    float M, L;
    f32x4 acc;
    merge_row(a.grp_ml + g0 * rows_total, a.grp_o + g0 * rows_total * 256, a.n_groups, rows_total,
              row, lane, M, L, acc);
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
  // one 16-row tile per workgroup; more rows run as passes (blockIdx.z) over
  // the same splits, which share the split's KV reads through L2 / MALL
  const int rows_per_pass = 16;
  const int passes = (n_rows + rows_per_pass - 1) / rows_per_pass;
  if (passes > kMaxPasses) return KV_ERR_UNSUPPORTED;
  int target = attn_target_splits(H, n_rows) / passes;
  if (target < 1) target = 1;
  const SplitPlan plan = plan_splits(c.max_limit, target);
  const WsLayout ws = ws_layout(H, n_rows, plan.n_splits, plan.n_groups);
  if (ws.total > c.ws_bytes) return KV_ERR_WORKSPACE;

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
  if (qf32)
    launch((attn_splitk_kernel<1, true>), grid, dim3(256), c.stream, a);
  else
    launch((attn_splitk_kernel<1, false>), grid, dim3(256), c.stream, a);
  return launch_status();
}

}  // namespace k8v4
