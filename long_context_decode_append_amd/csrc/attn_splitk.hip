// Split-K decode / verify attention over a paged pool, for gfx950.
//
// What it computes follows "#120 --kv k8v4: hybrid KV cache -- INT8 K +
// Hadamard-rotated Q4_0 V (816 B/cell)", How and Tests: the fused attention
// gathers the pages through the page table, scores q against the unrotated
// INT8 K (K = code * d per 128-dim group), runs a softmax over the visible
// cells, accumulates the rotated Q4_0 V ((code - 8) * d16) and rotates the
// result back with H/16; the batched (verify) form gives each query row its
// own number of visible cells.  The comparison formats of the same pages run
// through the same kernel (template FMT): int8 (K and V INT8, no rotation)
// and q4_0 (rotated K and V, scored against the rotated query); the fp16
// format (no quantization, no rotation) is the no-dequantization reference:
// its blocks hold the MFMA operands as they are loaded.
//
// Mapping onto MI355X:
//   * grid (splits [+ 1 for a fused append], KV heads, row passes); a
//     workgroup = 4 waves owns one contiguous logical cell range ("split")
//     and one tile of 16 query rows (decode: the 8 heads of the KV head;
//     verify: 2 queries per pass; a batch: one sequence per pass), its waves
//     take 32-cell steps round robin, the loads of a wave's next step in
//     flight while it computes the current one.  The split plan depends only
//     on the context length, so identity and permuted page tables give
//     bitwise-equal outputs.
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
//   * the 4 wave states merge through LDS, and the workgroup writes one
//     partial (m, l, O) per row; a second, small kernel merges the partials
//     of each row in fixed split order, normalizes and applies the inverse
//     Walsh-Hadamard transform.  The kernel boundary makes the partials
//     visible across XCDs (an in-kernel arrival-counter combine cost several
//     device-scope round trips).  No float atomics: results are
//     deterministic.
//   * a fused append (decode of a k8v4 pool) adds one workgroup per KV head
//     that quantizes the new token into its cell and writes it as one more
//     partial, beside the streaming splits.
#include <atomic>
#include <numeric>

#include "device.hpp"
#include "launch.hpp"
#include "quant.hpp"

namespace k8v4 {

constexpr float kLazy = 8.0f;  // log2 headroom of the lazy softmax reference


struct SplitArgs {
  const int8_t *kc;
  const float *ks;
  const uint8_t *vq;
  const float *vs;      // V scales (int8 format only)
  const int32_t *pt;
  const void *q;
  float *out;
  float2 *part_ml;      // [H][splits][rows]: (m, l) of each split partial
  float *part_o;        // [H][splits][rows][256]: unnormalized O (unrotated basis)
  int n_pages, P, H;
  int p_shift;          // log2(P) when P is a power of two, else -1
  int k_bytes, ks_bytes, v_bytes, vs_bytes;  // run sizes (each < 2^31)
  int k_bytes_m, ks_bytes_m, v_bytes_m, vs_bytes_m;  // the same for a streamed cache's mirror
  int n_q_heads, n_rows, rows_per_pass;
  int limits[kMaxQ];
  int max_limit;
  float scale2;         // softmax scale * log2(e)
  int steps_per_split, n_splits;
  int n_parts;          // partials per (KV head, row): n_splits, + 1 with a fused append
  // fused append (k8v4 decode only): the token k_new / v_new ([H][256],
  // kv_dtype) goes into cell append_pos (-1: no append); workgroup x =
  // n_splits of each KV head quantizes it and writes it as one more partial,
  // while the splits stream cells [0, append_pos) (max_limit = append_pos)
  const void *k_new;
  const void *v_new;
  int kv_dtype;
  int append_pos;
  // batch of sequences (decode of n_q independent sequences, 8 rows each):
  // pass b reads table pts[b] over cells [0, limits[b])
  int batch;
  const int32_t *pts[kMaxQ];
  int v_rot;            // V stored rotated (k8v4, q4_0): the combine finishes the inverse rotation
  // streamed cache: pt is the window map (logical page -> window slot, -1 when
  // not resident) and the pool above the window; a page not resident is read
  // from the mirror (mapped pinned host memory), at mirror_table[page]
  const int32_t *mirror_table;
  const int8_t *m_kc;
  const float *m_ks;
  const uint8_t *m_vq;
  const float *m_vs;
  int m_n_pages;
};

// dim of output tile j held by column n of the PV MFMA.  q4_0 V: column n
// reads bytes [8n, 8n+8) of a cell's 128 nibble bytes (block n/2), tile j
// takes byte j % 8, low nibble for j < 8 and high nibble for j >= 8.  INT8
// V: column n reads bytes [16n, 16n+16), tile j takes byte j.
template <bool kQ4V>
__device__ __forceinline__ int o_dim(int n, int j) {
  return kQ4V ? 32 * (n >> 1) + 8 * (n & 1) + (j & 7) + 16 * (j >> 3) : 16 * n + j;
}

// LDS position of dim d in a merged 256-float row: bits 6 and 7 of d are
// folded into bits 2 and 4, so the merge's stores (16 lanes of one row
// 8 dims apart in bit 3 and 32 apart in bits 5..7) hit distinct banks; pairs
// (d, d + 1), d even, and aligned quads stay together
__device__ __forceinline__ int row_swz(int d) {
  return d ^ (((d >> 6) & 1) << 2) ^ (((d >> 7) & 1) << 4);
}

__device__ __forceinline__ f16x8 pack8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 u = {a, b, c, d};
  return __builtin_bit_cast(f16x8, u);
}

// (x & m) | c in one VALU op (the compiler splits it when both are literals)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}
// the same with a per-lane mask
__device__ __forceinline__ uint32_t and_or_v(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(c));
  return r;
}

constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit elements (gfx9 family)

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float readlane(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Byte offsets of one 16-cell half of a step, per format (all wave-uniform).
// A half that starts past the split end reuses the step's first half (its
// cells are masked and its V scales zeroed).
struct Half {
  int bad;        // page-table entry out of range: rows that read it return NaN
  int none;       // a step past the wave's last: its loads read through empty
                  // buffer descriptors (zeros, no memory access)
  int host;       // streamed cache: the page is read from the mirror
  int k_soff;     // K data of the half's first cell (int8 codes, or q4_0 nibbles)
  int ks_soff;    // K scales (fp32 pairs, or the q4_0 scale group)
  int v_soff;     // V data (q4_0 nibbles, or int8 codes)
  int vd_soff;    // V scales (the q4_0 scale group, or fp32 pairs)
};

// page-table entry i through the constant address space: a scalar load
// (the table is never written while a kernel reads it)
__device__ __forceinline__ int pt_entry(const int32_t *pt, int i) {
  return ((const __attribute__((address_space(4))) int32_t *)pt)[i];
}

__device__ __forceinline__ int page_of(const SplitArgs &a, int pos) {
  return a.p_shift >= 0 ? (pos >> a.p_shift) : pos / a.P;
}

template <int FMT>
__device__ __forceinline__ Half make_half(const SplitArgs &a, int g, int pos, int page, int host) {
  Half h;
  h.none = 0;
  h.host = host;
  h.bad = page < 0 || page >= (host ? a.m_n_pages : a.n_pages);
  const int pg = h.bad ? 0 : page;
  const int slot0 = pos - page_of(a, pos) * a.P;  // a multiple of 16
  const int tile = pg * a.H + g;
  const int cell = tile * a.P + slot0;
  const int q4_tile = tile * 144 * a.P;
  if (FMT == KV_FMT_F16) {
    // 8 KB per 16 cells in each of K and V (cell % 16 == 0 here)
    h.k_soff = cell * 512;
    h.v_soff = cell * 512;
    h.ks_soff = h.vd_soff = 0;
    return h;
  }
  if (FMT == KV_FMT_Q4_0) {
    h.k_soff = q4_tile + slot0 * 128;
    h.ks_soff = q4_tile + 128 * a.P + slot0 * 16;  // scale group slot0 / 16
  } else {
    h.k_soff = cell * 256;  // = the start of the cell's 4 KB K-code block (cell % 16 == 0)
    h.ks_soff = cell * 8;
  }
  if (FMT == KV_FMT_INT8) {
    h.v_soff = cell * 256;
    h.vd_soff = cell * 8;
  } else {
    h.v_soff = q4_tile + slot0 * 128;
    h.vd_soff = q4_tile + 128 * a.P + slot0 * 16;
  }
  return h;
}

// Where logical page idx lives: the table entry, or for a streamed cache
// the window slot when resident and else the mirror page (both entries are
// read, as scalar loads, so no branch waits for the first)
template <bool STREAM>
__device__ __forceinline__ void locate(const SplitArgs &a, const int32_t *pt, int idx, int &page, int &host) {
  const int w = pt_entry(pt, idx);
  if (STREAM) {
    const int m = pt_entry(a.mirror_table, idx);
    host = w < 0;
    page = host ? m : w;
  } else {
    host = 0;
    page = w;
  }
}

// the two halves of the step at c (c < c_end); page entries read here are
// scalar loads
template <int FMT, bool STREAM>
__device__ __forceinline__ void step_halves(const SplitArgs &a, const int32_t *pt, int g, int c, int c_end, Half &h0,
                                            Half &h1) {
  const int p1pos = (c + 16 < c_end) ? c + 16 : c;
  int pg0, pg1, hs0, hs1;
  locate<STREAM>(a, pt, page_of(a, c), pg0, hs0);
  locate<STREAM>(a, pt, page_of(a, p1pos), pg1, hs1);
  h0 = make_half<FMT>(a, g, c, pg0, hs0);
  h1 = make_half<FMT>(a, g, p1pos, pg1, hs1);
}

// The halves of the first two steps of a wave (at c0 and c1): the four
// page-table entries are read together, so the kernel start waits for one
// scalar round trip instead of two.
template <int FMT, bool STREAM>
__device__ __forceinline__ void first_halves(const SplitArgs &a, const int32_t *pt, int g, int c0, int c1, int c_end,
                                             Half &h0, Half &h1,
                                             Half &n0, Half &n1) {
  const int pos[4] = {c0, (c0 + 16 < c_end) ? c0 + 16 : c0, c1, (c1 + 16 < c_end) ? c1 + 16 : c1};
  int pidx[4], pg[4], hs[4];
  if (a.p_shift >= 0) {
    for (int i = 0; i < 4; i++) pidx[i] = pos[i] >> a.p_shift;
  } else {
    for (int i = 0; i < 4; i++) pidx[i] = pos[i] / a.P;
  }
  for (int i = 0; i < 4; i++) locate<STREAM>(a, pt, pidx[i], pg[i], hs[i]);
  h0 = make_half<FMT>(a, g, pos[0], pg[0], hs[0]);
  h1 = make_half<FMT>(a, g, pos[1], pg[1], hs[1]);
  n0 = make_half<FMT>(a, g, pos[2], pg[2], hs[2]);
  n1 = make_half<FMT>(a, g, pos[3], pg[3], hs[3]);
}

// k-slot order inside an 8-dim q4_0 K operand: the nibble unpack yields the
// elements of a 4-byte word as (0, 2) then (1, 3)
__device__ __forceinline__ int q4_kslot(int t) { return (t & 4) | ((t & 1) << 1) | ((t >> 1) & 1); }

// Fused append of a decode (one wave, 4 dims per lane): quantize the new
// token of KV head g with the append kernel's rules, store it into cell
// append_pos, and write it as one more split partial of the 8 rows: m = its
// score (q . K) * scale * log2(e) with K = code * d, l = 1, O = its V as
// streamed cells see it ((code - 8) * d rounded to fp16), rotated back.  A cell whose
// page-table entry is out of range is not written and gives the rows NaN.
template <bool QF32>
__device__ __forceinline__ void append_token_partial(const SplitArgs &a, int g, int lane) {
  const int pos = a.append_pos;
  const int page = pt_entry(a.pt, page_of(a, pos));
  const bool bad = page < 0 || page >= a.n_pages;
  const int slot = pos - page_of(a, pos) * a.P;
  const size_t tile = (size_t)(bad ? 0 : page) * a.H + g;
  float x[4], y[4];
  load4(a.k_new, a.kv_dtype, (size_t)g * 256 + 4 * lane, x);
  load4(a.v_new, a.kv_dtype, (size_t)g * 256 + 4 * lane, y);
  float qx[kGqa][4];  // the 8 query heads of this KV head (a decode has one query)
  for (int r = 0; r < kGqa; r++) load4(a.q, QF32 ? 1 : 0, ((size_t)g * kGqa + r) * 256 + 4 * lane, qx[r]);
  float dk;
  const uint32_t kcodes = quant_k(x, dk);
  fwht256_lane4(y, lane);
  uint16_t d16;
  const uint32_t vcodes = quant_q4(y, lane, d16);
  if (!bad) {
    store_int8<true>(const_cast<uint8_t *>(reinterpret_cast<const uint8_t *>(a.kc)),
               const_cast<uint8_t *>(reinterpret_cast<const uint8_t *>(a.ks)), tile * a.P + slot, lane, kcodes, dk);
    store_q4(const_cast<uint8_t *>(a.vq), tile, a.P, slot, lane, vcodes, d16);
  }
  const _Float16 dh = __builtin_bit_cast(_Float16, d16);
  float kd[4], vr[4];
  for (int i = 0; i < 4; i++) {
    kd[i] = (float)(int8_t)(kcodes >> (8 * i)) * dk;
    vr[i] = (float)((_Float16)(float)((int)((vcodes >> (8 * i)) & 0xffu) - 8) * dh);
  }
  fwht_hi(vr, lane);  // partials carry the strides-64/128 factor of the inverse rotation
  const f32x4 vo = {vr[0], vr[1], vr[2], vr[3]};
  float dot[kGqa];
  for (int r = 0; r < kGqa; r++) dot[r] = qx[r][0] * kd[0] + qx[r][1] * kd[1] + qx[r][2] * kd[2] + qx[r][3] * kd[3];
  for (int r = 0; r < kGqa; r++) dot[r] = wave_sum(dot[r]);
  const size_t rows_total = (size_t)a.n_rows;
  const size_t sp = (size_t)g * a.n_parts + a.n_splits;
  for (int r = 0; r < kGqa; r++) {
    *reinterpret_cast<f32x4 *>(a.part_o + (sp * rows_total + r) * 256 + 4 * lane) = vo;
    if (lane == 0) a.part_ml[sp * rows_total + r] = make_float2(bad ? __builtin_nanf("") : dot[r] * a.scale2, 1.0f);
  }
}

// NT: the KV loads are non-temporal (a single pass reads each cell once, so
// they should not displace other data from L2 / MALL; the row passes of a
// verify share their reads through L2 and load normally)
// T: 16-row tiles per wave.  Verify runs T > 1: each step's K/V is loaded
// and dequantized once and used for all T tiles (the queries' MFMA operands
// are held in AGPRs and the extra tiles' accumulators take the registers a
// second wave would use, so one wave per SIMD).
// fp16 (T = 1 only): a step's raw K and V take 128 VGPRs, one workgroup per
// CU (the split plan's target anyway).
// W: waves per workgroup (4, one per SIMD; the int8 format's one-tile
// decode of long contexts takes 8, see the launch).
template <bool QF32, int FMT, bool NT, int T, bool STREAM, int W = kWaves>
__global__ __launch_bounds__(W * 64, (W == kWaves && T == 1 && FMT != KV_FMT_F16) ? 2 : 1) void attn_splitk_kernel(
    const SplitArgs a) {
  constexpr int kAux = NT ? 2 : 0;  // buffer-load cache policy bits: 2 = nt
  __shared__ __attribute__((aligned(16))) float lds_o[W * 16 * 64 * 4];  // wave states, accumulator layout
  __shared__ __attribute__((aligned(16))) float lds_m[W * 16];
  __shared__ __attribute__((aligned(16))) float lds_l[W * 16];
  constexpr bool kF16 = FMT == KV_FMT_F16;                 // K and V as fp16
  constexpr bool kInt8K = FMT == KV_FMT_INT8 || FMT == KV_FMT_K8V4;   // K as INT8 codes
  constexpr bool kQ4V = FMT == KV_FMT_Q4_0 || FMT == KV_FMT_K8V4;     // V as rotated q4_0
  constexpr int kKLoads = kF16 ? 8 : 4;                    // K loads per 16-cell half

  // one field from each 64-byte line of the argument block, so all four
  // lines are fetched in one scalar round trip rather than one after another
  asm volatile("" ::"s"(a.kc), "s"(a.n_pages), "s"(a.limits[4]), "s"(a.steps_per_split));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, lg = lane >> 4;
  const int split = blockIdx.x, g = blockIdx.y, pass = blockIdx.z;
  if (FMT == KV_FMT_K8V4 && split == a.n_splits) {
    // the fused append's own workgroup (exists only with one), on a CU of
    // its own beside the streaming splits
    if (wave == 0) append_token_partial<QF32>(a, g, lane);
    return;
  }
  const int row_base = pass * a.rows_per_pass;
  const int rows_here = min(a.rows_per_pass, a.n_rows - row_base);

  const int c_begin = split * a.steps_per_split * kStep;
  // a batch of sequences: pass b is sequence b, with its own table and
  // length (verify: every pass reads the one table up to the longest row)
  const int32_t *const ptab = a.batch ? a.pts[pass] : a.pt;
  const int c_end = min(a.batch ? a.limits[pass] : a.max_limit, c_begin + a.steps_per_split * kStep);
  const int stride = W * kStep;
  const int c_first = c_begin + wave * kStep;
  const bool has_work = c_first < c_end;
  // last step start of this wave (wave-uniform)
  const int c_last = has_work ? c_first + ((c_end - 1 - c_first) / stride) * stride : c_first;

  // buffer descriptors over whole runs; the hardware range check returns
  // zeros for any offset past a run
  const __amdgpu_buffer_rsrc_t rk_ = __builtin_amdgcn_make_buffer_rsrc((void *)a.kc, (short)0, a.k_bytes, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rks_ = __builtin_amdgcn_make_buffer_rsrc((void *)a.ks, (short)0, a.ks_bytes, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rv_ = __builtin_amdgcn_make_buffer_rsrc((void *)a.vq, (short)0, a.v_bytes, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rvs_ = __builtin_amdgcn_make_buffer_rsrc((void *)a.vs, (short)0, a.vs_bytes, kRsrcFlags);
  // the same runs with no records: a load through one returns zeros without
  // touching memory (the unconditional prefetch past a wave's last step)
  const __amdgpu_buffer_rsrc_t rk0 = __builtin_amdgcn_make_buffer_rsrc((void *)a.kc, (short)0, 0, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rks0 = __builtin_amdgcn_make_buffer_rsrc((void *)a.ks, (short)0, 0, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rv0 = __builtin_amdgcn_make_buffer_rsrc((void *)a.vq, (short)0, 0, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rvs0 = __builtin_amdgcn_make_buffer_rsrc((void *)a.vs, (short)0, 0, kRsrcFlags);
  // lane-constant parts of the operand-layout loads
  //   INT8 K:  + 1024 j: 16 bytes (dims 64 j + 16 lg ..) of cell n (the K-code
  //            run's 16-cell blocks are [dim quarter][cell][64 codes], so
  //            each of these loads reads 1 KB of consecutive bytes)
  //   q4_0 K:  + 32 j: the 16 nibble bytes of block 2 j + lg / 2 of cell n
  //            (low nibbles for even lg, high for odd), its scale at + 64 j
  //   q4_0 V:  + 128 i: bytes [8n, 8n+8) of cell 4lg+i; scales of block n/2
  //   INT8 V:  + 256 i: bytes [16n, 16n+16) of cell 4lg+i; scales of 4 cells
  //   fp16 K:  + 1024 j: dims 32 j + 8 lg .. + 7 of cell n (one A operand)
  //   fp16 V:  + 1024 u: dims 16 n + 2 u and 16 n + 2 u + 1 of cells 4 lg ..
  //            4 lg + 3 (the B operands of output tiles 2 u and 2 u + 1)
  const int k_voff = kF16 ? 256 * lg + 16 * n : kInt8K ? n * 64 + 16 * lg : n * 128 + 16 * (lg >> 1);
  const int ks_voff = kInt8K ? 32 * lg : 32 * (lg >> 1) + 2 * n;
  const int v_voff = kF16 ? 256 * lg + 16 * n : kQ4V ? 4 * lg * 128 + 8 * n : 4 * lg * 256 + 16 * n;
  const int vd_voff = kQ4V ? (n >> 1) * 32 + 8 * lg : 32 * lg;
  const int kstep_j = (kInt8K || kF16) ? 1024 : 32;
  // q4_0 K: even lg takes the low nibbles (fp16 1024 + n under exponent 25),
  // odd lg the high ones left in bits 4..7 (64 + n under exponent 21)
  const uint32_t q4_mask = (lg & 1) ? 0x00F000F0u : 0x000F000Fu;
  const uint32_t q4_expo = (lg & 1) ? 0x54005400u : 0x64006400u;
  const int v8_grp = n >> 3;                     // INT8 V: scale group of this lane's dims

  // The descriptor a half's loads use: its run's, the mirror's for a page
  // of a streamed cache read from the host, or an empty one past the wave's
  // last step.  The streamed variant builds it at each use from the base
  // pointer and byte count (a few scalar instructions): its twelve live
  // descriptors would exceed the scalar registers, and the compiler then
  // keeps them in vector registers and scratch memory and wraps every load
  // in a loop over the lanes.
  auto desc = [&](const Half &h, const void *base, int bytes, const void *mbase, int mbytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)(h.host ? mbase : base), (short)0,
                                             h.none ? 0 : (h.host ? mbytes : bytes), kRsrcFlags);
  };
  auto d_k = [&](const Half &h) {
    if constexpr (STREAM) return desc(h, a.kc, a.k_bytes, a.m_kc, a.k_bytes_m);
    else return h.none ? rk0 : rk_;
  };
  auto d_ks = [&](const Half &h) {
    if constexpr (STREAM) return desc(h, a.ks, a.ks_bytes, a.m_ks, a.ks_bytes_m);
    else return h.none ? rks0 : rks_;
  };
  auto d_v = [&](const Half &h) {
    if constexpr (STREAM) return desc(h, a.vq, a.v_bytes, a.m_vq, a.v_bytes_m);
    else return h.none ? rv0 : rv_;
  };
  auto d_vs = [&](const Half &h) {
    if constexpr (STREAM) return desc(h, a.vs, a.vs_bytes, a.m_vs, a.vs_bytes_m);
    else return h.none ? rvs0 : rvs_;
  };

  u32x4 kr[2][kKLoads];
  f32x4 ksr[2][2];      // INT8 K scales
  uint32_t kdr[2][4];   // q4_0 K scales (fp16 bits)
  u32x2 vr[2][4];       // q4_0 V
  u32x2 vdr[2];
  u32x4 vr8[2][4];      // INT8 V
  u32x4 vr16[2][kF16 ? 8 : 1];  // fp16 V
  f32x4 vsr[2][2];
  Half cur0, cur1, nxt0, nxt1;
  auto load_k = [&](int h2, const Half &h) {
    const __amdgpu_buffer_rsrc_t rk = d_k(h);
    for (int j = 0; j < kKLoads; j++)
      kr[h2][j] = __builtin_amdgcn_raw_buffer_load_b128(rk, k_voff + kstep_j * j, h.k_soff, kAux);
  };
  auto load_ks = [&](int h2, const Half &h) {
    const __amdgpu_buffer_rsrc_t rks = d_ks(h);
    const __amdgpu_buffer_rsrc_t rk = d_k(h);
    if (kF16) {
      // no scales
    } else if (kInt8K) {
      ksr[h2][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rks, ks_voff, h.ks_soff, kAux));
      ksr[h2][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rks, ks_voff + 16, h.ks_soff, kAux));
    } else {
      for (int j = 0; j < 4; j++) kdr[h2][j] = __builtin_amdgcn_raw_buffer_load_b16(rk, ks_voff + 64 * j, h.ks_soff, kAux);
    }
  };
  auto load_v = [&](int h2, const Half &h) {
    const __amdgpu_buffer_rsrc_t rv = d_v(h);
    if (kF16) {
      for (int u = 0; u < 8; u++) vr16[h2][u] = __builtin_amdgcn_raw_buffer_load_b128(rv, v_voff + 1024 * u, h.v_soff, kAux);
    } else if (kQ4V) {
      for (int i = 0; i < 4; i++) vr[h2][i] = __builtin_amdgcn_raw_buffer_load_b64(rv, v_voff + 128 * i, h.v_soff, kAux);
    } else {
      for (int i = 0; i < 4; i++) vr8[h2][i] = __builtin_amdgcn_raw_buffer_load_b128(rv, v_voff + 256 * i, h.v_soff, kAux);
    }
  };
  auto load_vd = [&](int h2, const Half &h) {
    const __amdgpu_buffer_rsrc_t rvs = d_vs(h);
    const __amdgpu_buffer_rsrc_t rv = d_v(h);
    if (kF16) {
      // no scales
    } else if (kQ4V) {
      vdr[h2] = __builtin_amdgcn_raw_buffer_load_b64(rv, vd_voff, h.vd_soff, kAux);
    } else {
      vsr[h2][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rvs, vd_voff, h.vd_soff, kAux));
      vsr[h2][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rvs, vd_voff + 16, h.vd_soff, kAux));
    }
  };
  // the query loads go first: they depend only on the kernel arguments, so
  // their latency overlaps the page-table round trip of the first K/V loads
  bool row_ok[T];
  int lim_eff[T];
  u32x4 qraw[T][QF32 ? 16 : 8];
  for (int t = 0; t < T; t++) {
    const int row = row_base + 16 * t + n;
    row_ok[t] = 16 * t + n < rows_here;
    int lim_row = a.limits[0];  // selects over the argument array keep it in scalar loads
    for (int i = 1; i < kMaxQ; i++) lim_row = ((row >> 3) == i) ? a.limits[i] : lim_row;
    lim_eff[t] = min(row_ok[t] ? lim_row : 0, c_end);
    // padding rows read row_base's query (always present) and are zeroed
    // after the loads, which keeps the loads free of branches (so waiting
    // for them does not also wait for the K/V loads issued later)
    const int rr = row_ok[t] ? row : row_base;
    const int qi = rr >> 3, hl = rr & 7;
    const size_t qbase = ((size_t)qi * a.n_q_heads + (size_t)g * kGqa + hl) * 256;
    for (int kk = 0; kk < 8; kk++) {
      const int d0 = kF16 ? 32 * kk + 8 * lg : 64 * (kk >> 1) + 16 * lg + 8 * (kk & 1);
      if (!QF32) {
        qraw[t][kk] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(a.q) + qbase + d0);
      } else {
        qraw[t][2 * kk] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const float *>(a.q) + qbase + d0);
        qraw[t][2 * kk + 1] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const float *>(a.q) + qbase + d0 + 4);
      }
    }
  }
  {
    // unconditional (a wave without work loads cell 0's step and never uses
    // it), so no control-flow join makes the compiler over-wait below
    const int cf = has_work ? c_first : 0, ce = has_work ? c_end : 16;
    first_halves<FMT, STREAM>(a, ptab, g, cf, has_work ? min(c_first + stride, c_last) : 0, ce, cur0, cur1, nxt0, nxt1);
    // loads of steps that do not exist fetch nothing
    cur0.none = cur1.none = !has_work;
    nxt0.none = nxt1.none = !has_work || c_first + stride > c_last;
    const Half *hs[2] = {&cur0, &cur1};
    for (int h2 = 0; h2 < 2; h2++) {
      load_k(h2, *hs[h2]);
      load_ks(h2, *hs[h2]);
      load_v(h2, *hs[h2]);
      load_vd(h2, *hs[h2]);
    }
    // keep these loads ahead of the query conversion (which waits for q)
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---------------------------------------------------------------- queries
  // B operand of the QK MFMA for k-step kk: lane (n, lg) holds row n, dims
  // 64 (kk/2) + 16 lg + 8 (kk%2) + 0..7 (q4_0 K: in q4_kslot order; fp16 K:
  // dims 32 kk + 8 lg + 0..7).  The
  // q4_0 format scores against rotated keys, so q is rotated first,
  // q~ = H q / 16 (through this wave's part of lds_o).
  f16x8 qop[T][8];
  f16x8 qlo[QF32 ? T : 1][QF32 ? 8 : 1];
  float cbias[T][2];
  for (int t = 0; t < T; t++) {
    cbias[t][0] = cbias[t][1] = 0.f;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    float qv[8][8];
    for (int kk = 0; kk < 8; kk++) {
      if (!QF32) {
        const f16x8 h = __builtin_bit_cast(f16x8, row_ok[t] ? qraw[t][kk] : zero4);
        for (int e = 0; e < 8; e++) qv[kk][e] = (float)h[e];
      } else {
        const f32x4 x0 = __builtin_bit_cast(f32x4, row_ok[t] ? qraw[t][2 * kk] : zero4);
        const f32x4 x1 = __builtin_bit_cast(f32x4, row_ok[t] ? qraw[t][2 * kk + 1] : zero4);
        for (int e = 0; e < 4; e++) {
          qv[kk][e] = x0[e];
          qv[kk][4 + e] = x1[e];
        }
      }
    }
    if (FMT == KV_FMT_Q4_0) {
      // Every wave of the workgroup holds the same rows: wave 0 writes them
      // to a shared buffer (rows 260 floats apart, so the 16 rows' writes
      // fall on different banks), each wave rotates the valid rows r with
      // r % 4 == wave in place, and every wave reads the tile back.
      constexpr int kQs = 256 + 4;
      float *qs = lds_o;  // [16 rows][kQs]; lds_o is free until the merge
      if (t > 0) __syncthreads();  // the previous tile's readers are done
      if (wave == 0)
        for (int kk = 0; kk < 8; kk++) {
          const int d0 = 64 * (kk >> 1) + 16 * lg + 8 * (kk & 1);
          *reinterpret_cast<f32x4 *>(&qs[n * kQs + d0]) = f32x4{qv[kk][0], qv[kk][1], qv[kk][2], qv[kk][3]};
          *reinterpret_cast<f32x4 *>(&qs[n * kQs + d0 + 4]) = f32x4{qv[kk][4], qv[kk][5], qv[kk][6], qv[kk][7]};
        }
      __syncthreads();
      const int rows_t = min(16, rows_here - 16 * t);  // valid rows of the tile (wave-uniform)
      for (int r = wave; r < rows_t; r += W) {
        f32x4 y4 = *reinterpret_cast<const f32x4 *>(&qs[r * kQs + 4 * lane]);
        float y[4] = {y4[0], y4[1], y4[2], y4[3]};
        fwht256_lane4(y, lane);
        *reinterpret_cast<f32x4 *>(&qs[r * kQs + 4 * lane]) = f32x4{y[0], y[1], y[2], y[3]};
      }
      __syncthreads();
      for (int kk = 0; kk < 8; kk++) {
        const int d0 = 64 * (kk >> 1) + 16 * lg + 8 * (kk & 1);
        const f32x4 x0 = *reinterpret_cast<const f32x4 *>(&qs[n * kQs + d0]);
        const f32x4 x1 = *reinterpret_cast<const f32x4 *>(&qs[n * kQs + d0 + 4]);
        for (int u = 0; u < 8; u++) {
          const int e = q4_kslot(u);
          qv[kk][u] = e < 4 ? x0[e] : x1[e - 4];
        }
      }
    }
    float s0 = 0.f, s1 = 0.f;
    for (int kk = 0; kk < 8; kk++) {
      f16x8 hi, lo;
      float ss = 0.f;
      for (int e = 0; e < 8; e++) {
        const float x = qv[kk][e];
        const _Float16 h = (_Float16)x;
        hi[e] = h;
        if (QF32) {
          const _Float16 l = (_Float16)(x - (float)h);
          lo[e] = l;
          ss += (float)h + (float)l;
        } else {
          ss += (float)h;
        }
      }
      if (kk < 4) s0 += ss; else s1 += ss;
      qop[t][kk] = hi;
      // several row tiles: the queries' operands live in AGPRs, where the
      // Q.K^T MFMAs read them directly (left to the register allocator
      // they are spilled there and copied back before every use)
      if (T > 1) asm volatile("" : "+a"(qop[t][kk]));
      if (QF32) qlo[t][kk] = lo;
    }
    if (kInt8K) {
      s0 = sum_lg(s0);
      s1 = sum_lg(s1);
      cbias[t][0] = 1152.0f * s0;
      cbias[t][1] = 1152.0f * s1;
    }
  }
  if (FMT == KV_FMT_Q4_0) __syncthreads();  // every wave has read the rotated rows (lds_o is reused)
  // smallest visible-cell limit over the valid rows of this tile (wave-
  // uniform): steps that end below it need no masking at all
  int lim_min;
  {
    int lm = 0x7fffffff;
    for (int t = 0; t < T; t++) lm = row_ok[t] ? min(lm, lim_eff[t]) : lm;
    lm = min(lm, lane_xor<1>(lm));
    lm = min(lm, lane_xor<2>(lm));
    lm = min(lm, lane_xor<4>(lm));
    lm = min(lm, lane_xor<8>(lm));
    lim_min = __builtin_amdgcn_readfirstlane(lm);
  }

  // ---------------------------------------------------------------- main loop
  // One register buffer per operand; each part is refilled with the next
  // step's data as soon as the current step has consumed it (K after its
  // conversion, K scales after the scores, V after the B operands are
  // built), so those loads fly during the rest of the step.  Page-table
  // entries are read two steps ahead.  The refill is unconditional (past the
  // end it re-reads the wave's last step) so every wait for current data
  // leaves the next step's loads outstanding.
  float m[T], lsum[T];
  f32x4 o[T][16];
  for (int t = 0; t < T; t++) {
    m[t] = -1e30f;
    lsum[t] = 0.f;
    for (int j = 0; j < 16; j++) o[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const f16x2 c1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const f16x2 c72 = {(_Float16)72.0f, (_Float16)72.0f};
  const f16x2 q4_bias = (lg & 1) ? c72 : c1032;  // q4_0 K: the nibble's offset + 8
  const f16x2 c1152 = {(_Float16)1152.0f, (_Float16)1152.0f};

  if (has_work) {
    int c = c_first;
    while (true) {
      // pages of the step after next
      Half nn0, nn1;
      step_halves<FMT, STREAM>(a, ptab, g, min(c + 2 * stride, c_last), c_end, nn0, nn1);
      nn0.none = nn1.none = c + 2 * stride > c_last;
      const int badp[2] = {cur0.bad, cur1.bad};
      // whole step inside every valid row's limit and on valid pages: no
      // masking (rows past rows_here then hold harmless values that are never
      // written out)
      const bool full_step = c + kStep <= lim_min && !(cur0.bad | cur1.bad);
      // the next step's half h2: the streamed variant takes it through a
      // select (with an array of pointers its halves went through scratch
      // memory), the others through the array, which schedules the resident
      // kernels better
      const Half *nx[2] = {&nxt0, &nxt1};
      auto hx = [&](int h2) -> const Half & {
        if constexpr (STREAM) return h2 ? nxt1 : nxt0;
        else return *nx[h2];
      };

      // ---- scores S^T = K . Q^T
      float s[T][8];
      for (int h2 = 0; h2 < 2; h2++) {
        f32x4 acc0[T], acc1[T];
        for (int t = 0; t < T; t++) acc0[t] = acc1[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < kKLoads; j++) {
          f16x8 ka, kb;
          if (kF16) {
            // fp16 K: the load is the A operand of k-step j
            ka = __builtin_bit_cast(f16x8, kr[h2][j]);
            for (int t = 0; t < T; t++) {
              acc0[t] = mfma16x16x32(ka, qop[t][j], acc0[t]);
              if (QF32) acc0[t] = mfma16x16x32(ka, qlo[t][j], acc0[t]);
            }
            kr[h2][j] = __builtin_amdgcn_raw_buffer_load_b128(d_k(hx(h2)), k_voff + kstep_j * j, hx(h2).k_soff, kAux);
            continue;
          }
          if (kInt8K) {
            // INT8 codes -> fp16 code + 1152 (exact); the bias leaves the
            // score through cbias
            uint32_t l0, h0, l1, h1, l2, h2w, l3, h3;
            i8x4_to_f16_biased(kr[h2][j].x, l0, h0);
            i8x4_to_f16_biased(kr[h2][j].y, l1, h1);
            i8x4_to_f16_biased(kr[h2][j].z, l2, h2w);
            i8x4_to_f16_biased(kr[h2][j].w, l3, h3);
            ka = pack8(l0, h0, l1, h1);
            kb = pack8(l2, h2w, l3, h3);
          } else {
            // q4_0 nibbles -> fp16 (code - 8) * d16 of this cell's block
            const uint32_t d = kdr[h2][j] & 0xffffu;
            const f16x2 dd = as_f16x2(d | (d << 16));
            uint32_t w[8];
            for (int q = 0; q < 4; q++) {
              const uint32_t x = kr[h2][j][q];
              const uint32_t y = x >> 8;
              w[2 * q] = as_u32((as_f16x2(and_or_v(x, q4_mask, q4_expo)) - q4_bias) * dd);
              w[2 * q + 1] = as_u32((as_f16x2(and_or_v(y, q4_mask, q4_expo)) - q4_bias) * dd);
            }
            ka = pack8(w[0], w[1], w[2], w[3]);
            kb = pack8(w[4], w[5], w[6], w[7]);
          }
          for (int t = 0; t < T; t++) {
            if (!kInt8K || j < 2) {
              acc0[t] = mfma16x16x32(ka, qop[t][2 * j], acc0[t]);
              acc0[t] = mfma16x16x32(kb, qop[t][2 * j + 1], acc0[t]);
              if (QF32) {
                acc0[t] = mfma16x16x32(ka, qlo[t][2 * j], acc0[t]);
                acc0[t] = mfma16x16x32(kb, qlo[t][2 * j + 1], acc0[t]);
              }
            } else {
              acc1[t] = mfma16x16x32(ka, qop[t][2 * j], acc1[t]);
              acc1[t] = mfma16x16x32(kb, qop[t][2 * j + 1], acc1[t]);
              if (QF32) {
                acc1[t] = mfma16x16x32(ka, qlo[t][2 * j], acc1[t]);
                acc1[t] = mfma16x16x32(kb, qlo[t][2 * j + 1], acc1[t]);
              }
            }
          }
          // K chunk j of this half consumed: refill with the next step's
          kr[h2][j] = __builtin_amdgcn_raw_buffer_load_b128(d_k(hx(h2)), k_voff + kstep_j * j, hx(h2).k_soff, kAux);
        }
        // several row tiles: the softmax scale folds into the cells' two K
        // group scales once, for all of them
        float dk0[4], dk1[4];
        for (int i = 0; i < 4; i++) {
          const f32x4 kq = ksr[h2][i >> 1];
          dk0[i] = kInt8K ? a.scale2 * kq[2 * (i & 1)] : a.scale2;
          dk1[i] = kInt8K ? a.scale2 * kq[2 * (i & 1) + 1] : 0.f;
        }
        for (int t = 0; t < T; t++)
          for (int i = 0; i < 4; i++) {
            if (kInt8K && T > 1) {
              s[t][4 * h2 + i] = dk0[i] * (acc0[t][i] - cbias[t][0]) + dk1[i] * (acc1[t][i] - cbias[t][1]);
            } else if (kInt8K) {
              const f32x4 kq = ksr[h2][i >> 1];
              const float d0 = kq[2 * (i & 1)], d1 = kq[2 * (i & 1) + 1];
              s[t][4 * h2 + i] = a.scale2 * (d0 * (acc0[t][i] - cbias[t][0]) + d1 * (acc1[t][i] - cbias[t][1]));
            } else {
              s[t][4 * h2 + i] = a.scale2 * acc0[t][i];
            }
          }
        if (!full_step) {
          for (int t = 0; t < T; t++)
            for (int i = 0; i < 4; i++) {
              const int cell = c + 16 * h2 + 4 * lg + i;
              const float sv = cell < lim_eff[t] ? s[t][4 * h2 + i] : -INFINITY;
              s[t][4 * h2 + i] = badp[h2] ? __builtin_nanf("") : sv;
            }
        }
        load_ks(h2, hx(h2));
      }

      // ---- online softmax against a reference max m that only moves when
      // a row's max exceeds it by more than 2^kLazy: p <= 2^kLazy stays exact
      // enough in fp16 and the accumulators are rarely rescaled
      f16x8 pop[T];
      for (int t = 0; t < T; t++) {
        float mx = s[t][0];
        for (int e = 1; e < 8; e++) mx = fmaxf(mx, s[t][e]);
        mx = max_lg(mx);
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

      // ---- O += P . V; the V scales of the cell pairs (k-slots 2k, 2k+1)
      // as fp16 pairs, zeroed for cells past the split
      uint32_t dsc[4] = {0u, 0u, 0u, 0u};
      // INT8 V: the fp32 scales of the cell pairs, and whether any nonzero
      // one lies below fp16's normal range (then this step forms code * d in
      // fp32 and rounds once, since an fp16 scale would lose its bits)
      float dsf[kQ4V || kF16 ? 1 : 4][2];
      bool v8_tiny = false;
      for (int k = 0; k < (kF16 ? 0 : 4); k++) {
        const int h2 = k >> 1;
        uint32_t w;
        float da = 0.f, db = 0.f;
        if (kQ4V) {
          w = (k & 1) ? vdr[h2].y : vdr[h2].x;
        } else {
          const f32x4 vs = vsr[h2][k & 1];
          da = v8_grp ? vs[1] : vs[0];
          db = v8_grp ? vs[3] : vs[2];
          w = as_u32(f16x2{(_Float16)da, (_Float16)db});
        }
        if (c + kStep > c_end) {
          const int ca = c + 16 * h2 + 4 * lg + 2 * (k & 1);
          if (ca >= c_end) {  // zero the scale of cells past the split
            w &= 0xffff0000u;
            da = 0.f;
          }
          if (ca + 1 >= c_end) {
            w &= 0x0000ffffu;
            db = 0.f;
          }
        }
        dsc[k] = w;
        if (!kQ4V) {
          dsf[k][0] = da;
          dsf[k][1] = db;
          v8_tiny |= (da != 0.f && fabsf(da) < 6.103515625e-05f) || (db != 0.f && fabsf(db) < 6.103515625e-05f);
        }
      }
      for (int h2 = 0; h2 < 2; h2++) load_vd(h2, hx(h2));
      if (kF16) {
        // fp16 V: one load holds the B operands of tiles 2u and 2u + 1.  The
        // values of cells past the split end are zeroed first: they may hold
        // any bits, and their P of 0 does not cancel a NaN.
        if (c + kStep > c_end) {
          for (int h2 = 0; h2 < 2; h2++) {
            const int cb = c + 16 * h2 + 4 * lg;
            const uint32_t m01 = (cb < c_end ? 0x0000ffffu : 0u) | (cb + 1 < c_end ? 0xffff0000u : 0u);
            const uint32_t m23 = (cb + 2 < c_end ? 0x0000ffffu : 0u) | (cb + 3 < c_end ? 0xffff0000u : 0u);
            for (int u = 0; u < 8; u++) {
              vr16[h2][u].x &= m01;
              vr16[h2][u].y &= m23;
              vr16[h2][u].z &= m01;
              vr16[h2][u].w &= m23;
            }
          }
        }
        for (int u = 0; u < 8; u++) {
          const u32x4 v0 = vr16[0][u], v1 = vr16[1][u];
          const f16x8 blo = pack8(v0.x, v0.y, v1.x, v1.y);  // tile 2u:     dim 16 n + 2 u
          const f16x8 bhi = pack8(v0.z, v0.w, v1.z, v1.w);  // tile 2u + 1: dim 16 n + 2 u + 1
          // chunk u of this step consumed: refill with the next step's
          for (int h2 = 0; h2 < 2; h2++)
            vr16[h2][u] = __builtin_amdgcn_raw_buffer_load_b128(d_v(hx(h2)), v_voff + 1024 * u, hx(h2).v_soff, kAux);
          for (int t = 0; t < T; t++) o[t][2 * u] = mfma16x16x32(pop[t], blo, o[t][2 * u]);
          for (int t = 0; t < T; t++) o[t][2 * u + 1] = mfma16x16x32(pop[t], bhi, o[t][2 * u + 1]);
        }
      } else if (kQ4V) {
        // B = (code - 8) * d16 in fp16, 4 tiles per byte pair
        for (int grp = 0; grp < 4; grp++) {
          const int dw = grp >> 1;
          const uint32_t sel = (grp & 1) ? 0x07060302u : 0x05040100u;
          uint32_t b0[4], b1[4], b2[4], b3[4];
          for (int k = 0; k < 4; k++) {
            const int h2 = k >> 1, ia = 2 * (k & 1);
            const uint32_t wa = dw ? vr[h2][ia].y : vr[h2][ia].x;
            const uint32_t wb = dw ? vr[h2][ia + 1].y : vr[h2][ia + 1].x;
            const uint32_t x = perm(wb, wa, sel);  // [a.byte, a.byte+1, b.byte, b.byte+1]
            const uint32_t y = x >> 8;
            const f16x2 dd = as_f16x2(dsc[k]);
            // a low nibble under exponent 25 reads 1024 + n, a high nibble
            // left in bits 4..7 under exponent 21 reads 64 + n
            b0[k] = as_u32((as_f16x2(and_or(x, 0x000F000Fu, 0x64006400u)) - c1032) * dd);
            b1[k] = as_u32((as_f16x2(and_or(x, 0x00F000F0u, 0x54005400u)) - c72) * dd);
            b2[k] = as_u32((as_f16x2(and_or(y, 0x000F000Fu, 0x64006400u)) - c1032) * dd);
            b3[k] = as_u32((as_f16x2(and_or(y, 0x00F000F0u, 0x54005400u)) - c72) * dd);
          }
          if (grp == 3) {
            // every V byte of this step consumed: refill with the next step's
            for (int h2 = 0; h2 < 2; h2++) load_v(h2, hx(h2));
          }
          const int jb = 2 * grp;
          for (int t = 0; t < T; t++) o[t][jb] = mfma16x16x32(pop[t], pack8(b0[0], b0[1], b0[2], b0[3]), o[t][jb]);          // tile jb     (byte lo nibble)
          for (int t = 0; t < T; t++) o[t][jb + 8] = mfma16x16x32(pop[t], pack8(b1[0], b1[1], b1[2], b1[3]), o[t][jb + 8]);  // tile jb + 8 (byte hi nibble)
          for (int t = 0; t < T; t++) o[t][jb + 1] = mfma16x16x32(pop[t], pack8(b2[0], b2[1], b2[2], b2[3]), o[t][jb + 1]);  // tile jb + 1
          for (int t = 0; t < T; t++) o[t][jb + 9] = mfma16x16x32(pop[t], pack8(b3[0], b3[1], b3[2], b3[3]), o[t][jb + 9]);  // tile jb + 9
        }
      } else {
        // INT8 V: tile j holds dim 16 n + j; B = code * d in fp16, the code
        // made exact as fp16 1152 + code by one xor under the 0x64 exponent
        const bool tiny = __any(v8_tiny);  // wave-uniform
        for (int j = 0; j < 16; j++) {
          const uint32_t sel = (0x0cu << 24) | ((4u + (j & 3)) << 16) | (0x0cu << 8) | (uint32_t)(j & 3);
          uint32_t b[4];
          for (int k = 0; k < 4; k++) {
            const int h2 = k >> 1, ia = 2 * (k & 1);
            const uint32_t x = perm(vr8[h2][ia + 1][j >> 2], vr8[h2][ia][j >> 2], sel);  // [a_j, 0, b_j, 0]
            const f16x2 code = as_f16x2(x ^ 0x64806480u) - c1152;  // exact
            if (!tiny) {
              b[k] = as_u32(code * as_f16x2(dsc[k]));
            } else {
              b[k] = as_u32(f16x2{(_Float16)((float)code[0] * dsf[k][0]), (_Float16)((float)code[1] * dsf[k][1])});
            }
          }
          if (j == 15) {
            for (int h2 = 0; h2 < 2; h2++) load_v(h2, hx(h2));
          }
          for (int t = 0; t < T; t++) o[t][j] = mfma16x16x32(pop[t], pack8(b[0], b[1], b[2], b[3]), o[t][j]);
        }
      }

      c += stride;
      if (c > c_last) break;
      cur0 = nxt0;
      cur1 = nxt1;
      nxt0 = nn0;
      nxt1 = nn1;
    }
  }

  // ---------------------------------------------------------------- workgroup merge
  // per row tile, every wave parks its own state in LDS as plain 256-float
  // rows, then after one barrier each wave takes whole rows: it merges the 4
  // wave states of a row in wave order (4 dims per lane), applies the
  // strides-64/128 factor of the inverse V rotation (H / 16 is linear, so the
  // combine sums partials in this basis and applies the rest once, to each
  // output slice) and stores the row as one coalesced 1 KB write
  const size_t rows_total = (size_t)a.n_rows;
  const size_t sp = (size_t)g * a.n_parts + split;
  for (int t = 0; t < T; t++) {
    const int rows_t = min(rows_here - 16 * t, 16);  // rows of this tile (workgroup-uniform)
    if (rows_t <= 0) break;
    if (t > 0) __syncthreads();  // the previous tile's readers are done
    const float lt = sum_lg(lsum[t]);
    if (lg == 0) {
      lds_m[wave * 16 + n] = m[t];
      lds_l[wave * 16 + n] = lt;
    }
    // lanes hold rows 4 lg + i; padding rows (decode fills 8 of 16) park
    // nothing.  Tiles 4 q .. 4 q + 3 hold 4 consecutive dims of a row (a
    // 4-aligned group, kept contiguous by the swizzle): one 16-byte write.
    for (int i = 0; i < 4; i++) {
      const int r = 4 * lg + i;
      if (r < rows_t)
        for (int qd = 0; qd < 4; qd++)
          *reinterpret_cast<f32x4 *>(&lds_o[(wave * 16 + r) * 256 + row_swz(o_dim<kQ4V>(n, 4 * qd))]) =
              f32x4{o[t][4 * qd][i], o[t][4 * qd + 1][i], o[t][4 * qd + 2][i], o[t][4 * qd + 3][i]};
    }
    __syncthreads();
    // two rows at a time, so their dependency chains (LDS reads, the FWHT's
    // cross-lane stages) overlap
    for (int r0 = wave; r0 < rows_t; r0 += 2 * W) {
      const int nr = r0 + W < rows_t ? 2 : 1;
      float y[2][4], M[2], Ls[2];
      for (int k = 0; k < 2; k++) {
        const int r = k < nr ? r0 + W * k : r0;
        float mw[W], lw[W];
        for (int w = 0; w < W; w++) {
          mw[w] = lds_m[w * 16 + r];
          lw[w] = lds_l[w * 16 + r];
        }
        M[k] = mw[0];
        for (int w = 1; w < W; w++) M[k] = fmaxf(M[k], mw[w]);
        Ls[k] = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < W; w++) {
          const float f = fast_exp2(mw[w] - M[k]);
          Ls[k] += lw[w] * f;
          acc += f * *reinterpret_cast<const f32x4 *>(&lds_o[(w * 16 + r) * 256 + row_swz(4 * lane)]);
        }
        for (int e = 0; e < 4; e++) y[k][e] = acc[e];
      }
      if (kQ4V) fwht_hi_x2(y[0], y[1], lane);  // strides 64, 128; the combine does the rest
      for (int k = 0; k < nr; k++) {
        const size_t prow = sp * rows_total + row_base + 16 * t + r0 + W * k;
        *reinterpret_cast<f32x4 *>(a.part_o + prow * 256 + 4 * lane) = f32x4{y[k][0], y[k][1], y[k][2], y[k][3]};
        if (lane == 0) a.part_ml[prow] = make_float2(M[k], Ls[k]);
      }
    }
  }
}

// Combine of the split partials of one query row of one KV head, after the
// split kernel (the kernel boundary makes every partial visible).  The
// partials carry only the strides-64/128 butterflies of the inverse V
// rotation, whose remaining butterflies (strides 1 .. 32) stay inside
// 64-dim slices, so the rows split into independent slices, one workgroup
// each: 16 split lanes of 16 threads (4 dims
// each) load a strided share of the slice rows and their m up front; every
// wave forms the common max and the weighted sum of l from all (m, l) by
// itself (so only the final sum of the 4 waves needs a barrier), the split
// lanes sum in ascending split order, the lanes and waves add in fixed order
// and O / l is stored.  Deterministic for a given split plan.
constexpr int kCombineWaves = 4;
constexpr int kCombineParts = 4;                                    // 64-dim slices
constexpr int kCombineLanes = kCombineWaves * 64 / 16;              // split lanes
constexpr int kCombineBatch = kMaxSplitsPerHead / kCombineLanes;    // loads per thread
static_assert(kMaxSplitsPerHead % 64 == 0, "whole (m, l) loads per lane");

__global__ __launch_bounds__(kCombineWaves * 64) void attn_combine_kernel(const SplitArgs a) {
  __shared__ f32x4 lds_acc[kCombineWaves][16];
  const int row = blockIdx.x, g = blockIdx.y, part = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int dl = tid & 15, sl = tid >> 4;  // 4-dim lane, split lane
  const int S = a.n_parts;
  const size_t rows_total = (size_t)a.n_rows;
  const size_t base = (size_t)g * S;
  const float *po = a.part_o + (base * rows_total + row) * 256 + 64 * part + 4 * dl;
  const size_t sstride = rows_total * 256;
  const float2 *pml = a.part_ml + base * rows_total + row;

  // this thread's slice rows and their m, issued first
  f32x4 ov[kCombineBatch];
  float mk[kCombineBatch];
  for (int k = 0; k < kCombineBatch; k++) {
    const int sidx = sl + kCombineLanes * k;
    if (sidx < S) {
      ov[k] = *reinterpret_cast<const f32x4 *>(po + (size_t)sidx * sstride);
      mk[k] = pml[(size_t)sidx * rows_total].x;
    }
  }
  // every wave reads all (m, l) of the row and forms the common max M and
  // L = sum l_s 2^(m_s - M) itself, so no workgroup barrier is needed
  constexpr int kMl = kMaxSplitsPerHead / 64;
  float2 mlw[kMl];
  for (int i = 0; i < kMl; i++) {
    const int s = lane + 64 * i;
    mlw[i] = s < S ? pml[(size_t)s * rows_total] : make_float2(-1e30f, 0.f);
  }
  float mx = mlw[0].x;
  for (int i = 1; i < kMl; i++) mx = fmaxf(mx, mlw[i].x);
  const float M = wave_max(mx);
  float lw = 0.f;
  for (int i = 0; i < kMl; i++) lw += (lane + 64 * i < S) ? mlw[i].y * fast_exp2(mlw[i].x - M) : 0.f;
  const float L = wave_sum(lw);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < kCombineBatch; k++) {
    const int sidx = sl + kCombineLanes * k;
    if (sidx < S) acc += fast_exp2(mk[k] - M) * ov[k];
  }
  // the 4 split lanes of a wave, then the waves
  for (int i = 0; i < 4; i++) acc[i] = sum_lg(acc[i]);
  if (lane < 16) lds_acc[wave][lane] = acc;
  __syncthreads();
  if (tid >= 16) return;
  f32x4 tot = lds_acc[0][tid];
  for (int w = 1; w < kCombineWaves; w++) tot += lds_acc[w][tid];
  const float inv = 1.0f / L;
  const int qi = row >> 3, hl = row & 7;
  float y[4] = {tot[0] * inv, tot[1] * inv, tot[2] * inv, tot[3] * inv};
  // rotated V: the partials carry the strides-64/128 factor of the inverse
  // rotation; the strides 1 .. 32 (inside this 64-dim slice) and 1/16 finish it
  if (a.v_rot) fwht_lo16(y, lane);
  float *op = a.out + ((size_t)qi * a.n_q_heads + (size_t)g * kGqa + hl) * 256 + 64 * part + 4 * tid;
  *reinterpret_cast<f32x4 *>(op) = f32x4{y[0], y[1], y[2], y[3]};
}

// Lookups of a streamed attention call: one per logical page [0, n_read),
// a miss per page whose window map entry is negative (not resident).  One
// workgroup; two device-scope additions to the caller's counters.
__global__ __launch_bounds__(256) void stream_lookup_kernel(const int32_t *window_map, int n_read, int32_t *stats) {
  __shared__ int lds_miss[4];
  int miss = 0;
  for (int i = threadIdx.x; i < n_read; i += 256) miss += window_map[i] < 0 ? 1 : 0;
  for (int o = 32; o > 0; o >>= 1) miss += __shfl_xor(miss, o, 64);
  if ((threadIdx.x & 63) == 0) lds_miss[threadIdx.x >> 6] = miss;
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(&stats[0], n_read);
    atomicAdd(&stats[1], lds_miss[0] + lds_miss[1] + lds_miss[2] + lds_miss[3]);
  }
}

// ---------------------------------------------------------------- host side

// Compute units of the current device, cached per device (relaxed atomics:
// concurrent first calls may both query, and store the same value).  The split plan
// targets one 4-wave workgroup per CU and KV head share: measured on
// MI355X, one workgroup per CU (1 wave per SIMD, 128 splits per KV head)
// beats two (256 splits) for decode at 118,750 and 240,000 cells.
static int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];  // 0 = not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess || prop.multiProcessorCount <= 0) return 256;
  if (dev >= 0 && dev < kMaxDevices) cached[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
  return prop.multiProcessorCount;
}

int attn_target_splits(int n_kv_heads, int n_rows) {
  (void)n_rows;
  const int per_head = device_cus() / (n_kv_heads > 0 ? n_kv_heads : 1);
  return per_head < 1 ? 1 : per_head;
}

int launch_attn_splitk(const AttnCall &c) {
  const kv_pool *pool = c.pool;
  const int H = pool->n_kv_heads;
  const int n_rows = c.n_q * kGqa;
  const bool qf32 = c.q_dtype == KV_DTYPE_F32;
  // a workgroup takes T 16-row tiles (up to 3, half-precision queries: the
  // extra accumulators leave no room for fp32 query halves); more rows run
  // as passes (blockIdx.z) over the same splits, which share the split's KV
  // reads through L2 / MALL; a batch runs one sequence (8 rows) per pass
  const int tiles = (n_rows + 15) / 16;
  const int tile_passes = (tiles + 2) / 3;
  const int T = (c.batch || qf32 || pool->fmt == KV_FMT_F16) ? 1 : (tiles + tile_passes - 1) / tile_passes;
  const int rows_per_pass = c.batch ? kGqa : 16 * T;
  const int passes = (n_rows + rows_per_pass - 1) / rows_per_pass;
  if (passes > (c.batch ? kMaxQ : kMaxPasses)) return KV_ERR_UNSUPPORTED;
  if (c.max_limit > (1 << 30)) return KV_ERR_UNSUPPORTED;
  int target = attn_target_splits(H, n_rows) / passes;
  // passes of one split read the same cells: with splits x KV heads a
  // multiple of 8, their workgroups (block ids S * H apart) land on the same
  // XCD (workgroups go round-robin over the 8) and share its L2
  if (passes > 1) {
    const int m = 8 / std::gcd(H, 8);
    if (target >= m) target -= target % m;
  }
  if (target < 1) target = 1;
  // a fused append adds one partial per KV head (its own workgroup); onto an
  // empty cache it streams no cells (one empty split)
  const bool fused = c.append_pos >= 0;
  if (fused && target > kMaxSplitsPerHead - 1) target = kMaxSplitsPerHead - 1;
  const SplitPlan plan = plan_splits(c.max_limit > 0 ? c.max_limit : 1, target);
  const int n_parts = plan.n_splits + (fused ? 1 : 0);
  const WsLayout ws = ws_layout(H, n_rows, n_parts);
  if (ws.total > c.ws_bytes) return KV_ERR_WORKSPACE;

  SplitArgs a;
  char *base = (char *)c.ws;
  a.kc = (const int8_t *)pool->run[0];
  a.ks = (const float *)pool->run[1];
  a.vq = (const uint8_t *)pool->run[2];
  a.vs = (const float *)pool->run[3];
  a.pt = c.batch ? c.pts[0] : c.seq->page_table;
  a.batch = c.batch ? 1 : 0;
  for (int i = 0; i < kMaxQ; i++) a.pts[i] = c.batch ? c.pts[i] : nullptr;
  a.q = c.q;
  a.out = c.out;
  a.part_ml = (float2 *)(base + ws.part_ml);
  a.part_o = (float *)(base + ws.part_o);
  a.n_pages = pool->n_pages;
  a.P = pool->page_size;
  a.H = H;
  a.p_shift = -1;
  for (int sh = 0; sh < 31; sh++)
    if ((1 << sh) == a.P) a.p_shift = sh;
  {
    const size_t kb = run_bytes(pool->fmt, 0, pool->n_pages, a.P, H, kHeadDim);
    const size_t sb = run_bytes(pool->fmt, 1, pool->n_pages, a.P, H, kHeadDim);
    const size_t vb = run_bytes(pool->fmt, 2, pool->n_pages, a.P, H, kHeadDim);
    const size_t vsb = run_bytes(pool->fmt, 3, pool->n_pages, a.P, H, kHeadDim);
    if (kb > 0x7fffffffu || sb > 0x7fffffffu || vb > 0x7fffffffu || vsb > 0x7fffffffu) return KV_ERR_UNSUPPORTED;
    a.k_bytes = (int)kb;
    a.ks_bytes = (int)sb;
    a.v_bytes = (int)vb;
    a.vs_bytes = (int)vsb;
  }
  const bool stream = c.stream_s != nullptr;
  a.mirror_table = nullptr;
  a.m_kc = nullptr;
  a.m_ks = nullptr;
  a.m_vq = nullptr;
  a.m_vs = nullptr;
  a.m_n_pages = 0;
  a.k_bytes_m = a.ks_bytes_m = a.v_bytes_m = a.vs_bytes_m = 0;
  if (stream) {
    const kv_pool *m = &c.stream_s->mirror;
    const size_t kb = run_bytes(m->fmt, 0, m->n_pages, a.P, H, kHeadDim);
    const size_t sb = run_bytes(m->fmt, 1, m->n_pages, a.P, H, kHeadDim);
    const size_t vb = run_bytes(m->fmt, 2, m->n_pages, a.P, H, kHeadDim);
    const size_t vsb = run_bytes(m->fmt, 3, m->n_pages, a.P, H, kHeadDim);
    if (kb > 0x7fffffffu || sb > 0x7fffffffu || vb > 0x7fffffffu || vsb > 0x7fffffffu) return KV_ERR_UNSUPPORTED;
    a.k_bytes_m = (int)kb;
    a.ks_bytes_m = (int)sb;
    a.v_bytes_m = (int)vb;
    a.vs_bytes_m = (int)vsb;
    a.mirror_table = c.stream_s->mirror_table;
    a.m_kc = (const int8_t *)m->run[0];
    a.m_ks = (const float *)m->run[1];
    a.m_vq = (const uint8_t *)m->run[2];
    a.m_vs = (const float *)m->run[3];
    a.m_n_pages = m->n_pages;
  }
  a.n_q_heads = c.n_q_heads;
  a.n_rows = n_rows;
  a.rows_per_pass = rows_per_pass;
  for (int i = 0; i < kMaxQ; i++) a.limits[i] = i < c.n_q ? c.limits[i] : 0;
  a.max_limit = c.max_limit;
  a.scale2 = c.scale * 1.4426950408889634f;
  a.steps_per_split = plan.steps_per_split;
  a.n_splits = plan.n_splits;
  a.n_parts = n_parts;
  a.k_new = c.k_new;
  a.v_new = c.v_new;
  a.kv_dtype = c.kv_dtype;
  a.append_pos = c.append_pos;
  a.v_rot = (pool->fmt == KV_FMT_K8V4 || pool->fmt == KV_FMT_Q4_0) ? 1 : 0;

  dim3 grid(n_parts, H, passes);
  // non-temporal KV loads when no two passes share their reads and one call
  // streams more than 16 MiB: a call reads each cell once, and a long
  // context's pages would only push other data out of L2 and the Infinity
  // Cache (measured with the K-code blocks: 6.7 % faster per layer at
  // 118,750 cells, 3 % at 240,000).  Small contexts keep plain loads, so a
  // model whose whole cache fits the 256 MB Infinity Cache can reuse it
  // from step to step; verify's row passes share their reads through L2.
  size_t stream_cells = 0;
  for (int i = 0; i < (c.batch ? c.n_q : 1); i++) stream_cells += (size_t)(c.batch ? c.limits[i] : c.max_limit);
  const bool nt = (passes == 1 || c.batch) &&
                  stream_cells * kv_cell_bytes(pool->fmt, H, kHeadDim) > ((size_t)16 << 20);
  if (stream) {
    // device-side lookups: one per logical page the call reads, a miss per
    // page not resident; counted before the attention reads them
    const int n_read = (int)(((int64_t)c.max_limit + a.P - 1) / a.P);
    launch(stream_lookup_kernel, dim3(1), dim3(256), c.stream, (const int32_t *)a.pt, n_read, c.stream_s->stats);
    if (int e = launch_status()) return e;
  }
  const bool nt_k = nt && !stream;
  // The int8 format with one 16-row tile runs eight waves per workgroup
  // (two per SIMD) once a split has at least 12 steps: its 1,056-byte cells
  // leave a wave per SIMD short of loads in flight (measured: 6-16 % faster
  // from 49,152 cells on, equal at 32,768; slower for the other formats).
  // A streamed call chooses the same way, so its result stays bitwise the
  // resident one.
  if (pool->fmt == KV_FMT_INT8 && T == 1 && !qf32 && plan.steps_per_split >= 12) {
    if (stream)
      launch((attn_splitk_kernel<false, KV_FMT_INT8, false, 1, true, 8>), grid, dim3(512), c.stream, a);
    else if (nt_k)
      launch((attn_splitk_kernel<false, KV_FMT_INT8, true, 1, false, 8>), grid, dim3(512), c.stream, a);
    else
      launch((attn_splitk_kernel<false, KV_FMT_INT8, false, 1, false, 8>), grid, dim3(512), c.stream, a);
  } else
  switch ((((pool->fmt * 2 + (stream ? 1 : 0)) * 4 + (qf32 ? 2 : 0) + (nt_k ? 1 : 0)) << 2) + T) {
#define K8V4_SPLIT_CASE(F, S, Q, N, T_) \
  case (((F * 2 + (S ? 1 : 0)) * 4 + (Q ? 2 : 0) + (N ? 1 : 0)) << 2) + T_: \
    launch((attn_splitk_kernel<Q, F, N, T_, S>), grid, dim3(256), c.stream, a); \
    break;
#define K8V4_SPLIT_FMT(F)                      \
  K8V4_SPLIT_CASE(F, false, false, false, 1)   \
  K8V4_SPLIT_CASE(F, false, false, true, 1)    \
  K8V4_SPLIT_CASE(F, false, true, false, 1)    \
  K8V4_SPLIT_CASE(F, false, true, true, 1)     \
  K8V4_SPLIT_CASE(F, false, false, false, 2)   \
  K8V4_SPLIT_CASE(F, false, false, true, 2)    \
  K8V4_SPLIT_CASE(F, false, false, false, 3)   \
  K8V4_SPLIT_CASE(F, false, false, true, 3)    \
  K8V4_SPLIT_CASE(F, true, false, false, 1)    \
  K8V4_SPLIT_CASE(F, true, true, false, 1)     \
  K8V4_SPLIT_CASE(F, true, false, false, 2)    \
  K8V4_SPLIT_CASE(F, true, false, false, 3)
    K8V4_SPLIT_CASE(KV_FMT_F16, false, false, false, 1)
    K8V4_SPLIT_CASE(KV_FMT_F16, false, false, true, 1)
    K8V4_SPLIT_CASE(KV_FMT_F16, false, true, false, 1)
    K8V4_SPLIT_CASE(KV_FMT_F16, false, true, true, 1)
    K8V4_SPLIT_CASE(KV_FMT_F16, true, false, false, 1)
    K8V4_SPLIT_CASE(KV_FMT_F16, true, true, false, 1)
    K8V4_SPLIT_FMT(KV_FMT_INT8)
    K8V4_SPLIT_FMT(KV_FMT_Q4_0)
    K8V4_SPLIT_FMT(KV_FMT_K8V4)
#undef K8V4_SPLIT_FMT
#undef K8V4_SPLIT_CASE
    default: return KV_ERR_UNSUPPORTED;
  }
  if (int e = launch_status()) return e;
  launch(attn_combine_kernel, dim3(n_rows, H, kCombineParts), dim3(kCombineWaves * 64), c.stream, a);
  return launch_status();
}

}  // namespace k8v4
