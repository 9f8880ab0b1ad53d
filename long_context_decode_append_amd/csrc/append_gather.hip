// k8v4 append (quantize + place) and gather kernels for gfx950.
//
// Append follows "#120 --kv k8v4: hybrid KV cache -- INT8 K + Hadamard-
// rotated Q4_0 V (816 B/cell)", sections What/How/Tests: K is stored as
// INT8 codes with round-half-even and a scale per 128-dim group, unrotated;
// V is rotated by the 256-point Walsh-Hadamard transform (scaled by 1/16)
// and stored as Q4_0 blocks of 32 with an fp16 scale.  Cells are placed
// through the page table.  One wave (64 lanes x 4 dims) handles one
// (token, KV head) pair: K and V are quantized in the same pass, so there
// is no duplicate write of a folded half.
//
// The two comparison formats of the same pages use the same rules on other
// halves: int8 (K and V both INT8, unrotated, 1,056 B/cell) and q4_0 (K and
// V both rotated Q4_0, 576 B/cell) ("#120", Measured: the k8v4 / int8 /
// q4_0 rows; "#711", How: the format numbers).
//
// Every quantizer step is one IEEE fp32 operation rounded as written: this
// file is built with -ffp-contract=off and the functions also disable
// contraction locally, so x * r + 8.5 is never fused.
#include "device.hpp"
#include "launch.hpp"
#include "quant.hpp"

namespace k8v4 {

struct AppendArgs {
  uint8_t *run[4];
  const int32_t *pt;
  const void *k;
  const void *v;
  int dtype;       // 0 fp16, 1 fp32
  int pos0, n_tokens, n_pages, P, H;
  // a second copy of the same cells (a streamed cache writes its mirror and
  // its window): table pt2 into pool run2 (pt2 null: none); a cell whose
  // entry is out of [0, n_pages2) is not resident there
  uint8_t *run2[4];
  const int32_t *pt2;
  int n_pages2;
};

// one wave per (token, KV head); FMT selects the rule of each half.  The
// token is quantized once and stored into every destination that holds its
// cell (all runs of each).
template <int FMT>
__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (token, head)
  if (item >= (int64_t)a.n_tokens * a.H) return;                       // whole wave exits
  const int t = (int)(item / a.H), g = (int)(item % a.H);
  const int p = a.pos0 + t;
  const int lp = p / a.P, slot = p % a.P;
  const int page = a.pt[lp];
  const bool ok = page >= 0 && page < a.n_pages;                       // never write outside a pool
  const int page2 = a.pt2 ? a.pt2[lp] : -1;
  const bool ok2 = page2 >= 0 && page2 < a.n_pages2;
  if (!ok && !ok2) return;
  const size_t src = ((size_t)t * a.H + g) * 256 + 4 * lane;
  const size_t tile = (size_t)page * a.H + g, tile2 = (size_t)page2 * a.H + g;
  const size_t cell = tile * a.P + slot, cell2 = tile2 * a.P + slot;

  float x[4];
  load4(a.k, a.dtype, src, x);
  if (FMT == KV_FMT_F16) {
    // no quantization: fp16 (round to nearest even) in the operand blocks
    if (ok) store_f16_k(a.run[0], cell, lane, x);
    if (ok2) store_f16_k(a.run2[0], cell2, lane, x);
    load4(a.v, a.dtype, src, x);
    if (ok) store_f16_v(a.run[2], cell, lane, x);
    if (ok2) store_f16_v(a.run2[2], cell2, lane, x);
    return;
  }
  if (FMT == KV_FMT_Q4_0) {
    fwht256_lane4(x, lane);
    uint16_t d16;
    const uint32_t codes = quant_q4(x, lane, d16);
    if (ok) store_q4(a.run[0], tile, a.P, slot, lane, codes, d16);
    if (ok2) store_q4(a.run2[0], tile2, a.P, slot, lane, codes, d16);
  } else {
    float d;
    const uint32_t codes = quant_k(x, d);
    if (ok) store_int8<true>(a.run[0], a.run[1], cell, lane, codes, d);
    if (ok2) store_int8<true>(a.run2[0], a.run2[1], cell2, lane, codes, d);
  }

  load4(a.v, a.dtype, src, x);
  if (FMT == KV_FMT_INT8) {
    float d;
    const uint32_t codes = quant_k(x, d);
    if (ok) store_int8<false>(a.run[2], a.run[3], cell, lane, codes, d);
    if (ok2) store_int8<false>(a.run2[2], a.run2[3], cell2, lane, codes, d);
  } else {
    fwht256_lane4(x, lane);
    uint16_t d16;
    const uint32_t codes = quant_q4(x, lane, d16);
    if (ok) store_q4(a.run[2], tile, a.P, slot, lane, codes, d16);
    if (ok2) store_q4(a.run2[2], tile2, a.P, slot, lane, codes, d16);
  }
}

struct GatherArgs {
  const uint8_t *run[4];
  const int32_t *pt;
  uint8_t *out[4];
  int pos0, n, n_pages, P, H;
};

template <bool KLAYOUT>
__device__ __forceinline__ void gather_int8(const uint8_t *codes_run, const uint8_t *scales_run, bool bad,
                                            size_t cell, size_t o, int lane, uint8_t *oc, uint8_t *os) {
  const size_t src = KLAYOUT ? k_code_off(cell, lane) : cell * 256 + 4 * lane;
  uint32_t w = bad ? 0xffffffffu : *reinterpret_cast<const uint32_t *>(codes_run + src);
  *reinterpret_cast<uint32_t *>(oc + o * 256 + 4 * lane) = w;
  if (lane < 2)
    reinterpret_cast<float *>(os)[o * 2 + lane] =
        bad ? __builtin_nanf("") : reinterpret_cast<const float *>(scales_run)[cell * 2 + lane];
}

__device__ __forceinline__ void gather_q4(const uint8_t *run, bool bad, size_t tile, int P, int slot, size_t o,
                                          int lane, uint8_t *ob) {
  const uint8_t *vt = run + tile * 144 * P;
  for (int e = lane; e < 144; e += 64) {
    const int b = e / 18, off = e % 18;
    uint8_t byte;
    if (off < 2) byte = vt[q4_scale_off(P, slot, b) + off];
    else byte = vt[(size_t)slot * 128 + b * 16 + (off - 2)];
    ob[o * 144 + e] = bad ? 0xff : byte;
  }
}

// fp16 halves: K and V of head-cell `cell` back to [256] fp16 rows
__device__ __forceinline__ void gather_f16(const uint8_t *krun, const uint8_t *vrun, bool bad, size_t cell, size_t o,
                                           int lane, uint8_t *ok, uint8_t *ov) {
  u32x2 kw = {0xffffffffu, 0xffffffffu}, vw = {0xffffffffu, 0xffffffffu};
  if (!bad) {
    kw = *reinterpret_cast<const u32x2 *>(krun + f16_k_off(cell, lane));
    uint16_t h[4];
    for (int e = 0; e < 4; e++) h[e] = *reinterpret_cast<const uint16_t *>(vrun + f16_v_off(cell, 4 * lane + e));
    vw = u32x2{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
  }
  *reinterpret_cast<u32x2 *>(ok + o * 512 + 8 * lane) = kw;
  *reinterpret_cast<u32x2 *>(ov + o * 512 + 8 * lane) = vw;
}

// one wave per (cell, KV head); outputs per format as kv_gather_runs documents
template <int FMT>
__global__ __launch_bounds__(256) void gather_kernel(const GatherArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (int64_t)a.n * a.H) return;
  const int t = (int)(item / a.H), g = (int)(item % a.H);
  const int p = a.pos0 + t;
  int page = a.pt[p / a.P];
  const bool bad = page < 0 || page >= a.n_pages;
  const int slot = p % a.P;
  const size_t tile = (size_t)(bad ? 0 : page) * a.H + g;
  const size_t cell = tile * a.P + slot;
  const size_t o = (size_t)t * a.H + g;
  // an out-of-range table entry yields 0xff bytes / NaN scales, never a read outside the pool
  if (FMT == KV_FMT_F16) {
    gather_f16(a.run[0], a.run[2], bad, cell, o, lane, a.out[0], a.out[2]);
    return;
  }
  if (FMT == KV_FMT_Q4_0) gather_q4(a.run[0], bad, tile, a.P, slot, o, lane, a.out[0]);
  else gather_int8<true>(a.run[0], a.run[1], bad, cell, o, lane, a.out[0], a.out[1]);
  if (FMT == KV_FMT_INT8) gather_int8<false>(a.run[2], a.run[3], bad, cell, o, lane, a.out[2], a.out[3]);
  else gather_q4(a.run[2], bad, tile, a.P, slot, o, lane, a.out[2]);
}

__global__ void fill_zero_kernel(uint32_t *p, size_t n_words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

int launch_append(const kv_pool *pool, const kv_seq *seq, const void *k, const void *v, int dtype, int pos0,
                  int n, hipStream_t s, const kv_pool *pool2, const int32_t *pt2) {
  AppendArgs a;
  for (int r = 0; r < 4; r++) {
    a.run[r] = (uint8_t *)pool->run[r];
    a.run2[r] = pool2 ? (uint8_t *)pool2->run[r] : nullptr;
  }
  a.pt = seq->page_table;
  a.pt2 = pool2 ? pt2 : nullptr;
  a.n_pages2 = pool2 ? pool2->n_pages : 0;
  a.k = k;
  a.v = v;
  a.dtype = dtype;
  a.pos0 = pos0;
  a.n_tokens = n;
  a.n_pages = pool->n_pages;
  a.P = pool->page_size;
  a.H = pool->n_kv_heads;
  const int64_t items = (int64_t)n * a.H;
  const unsigned blocks = (unsigned)((items + 3) / 4);
  switch (pool->fmt) {
    case KV_FMT_F16: launch(append_kernel<KV_FMT_F16>, dim3(blocks), dim3(256), s, a); break;
    case KV_FMT_INT8: launch(append_kernel<KV_FMT_INT8>, dim3(blocks), dim3(256), s, a); break;
    case KV_FMT_Q4_0: launch(append_kernel<KV_FMT_Q4_0>, dim3(blocks), dim3(256), s, a); break;
    default: launch(append_kernel<KV_FMT_K8V4>, dim3(blocks), dim3(256), s, a); break;
  }
  return launch_status();
}

int launch_gather(const kv_pool *pool, const kv_seq *seq, int pos0, int n, void *const out[4], hipStream_t s) {
  GatherArgs a;
  for (int r = 0; r < 4; r++) {
    a.run[r] = (const uint8_t *)pool->run[r];
    a.out[r] = (uint8_t *)out[r];
  }
  a.pt = seq->page_table;
  a.pos0 = pos0;
  a.n = n;
  a.n_pages = pool->n_pages;
  a.P = pool->page_size;
  a.H = pool->n_kv_heads;
  const int64_t items = (int64_t)n * a.H;
  const unsigned blocks = (unsigned)((items + 3) / 4);
  switch (pool->fmt) {
    case KV_FMT_F16: launch(gather_kernel<KV_FMT_F16>, dim3(blocks), dim3(256), s, a); break;
    case KV_FMT_INT8: launch(gather_kernel<KV_FMT_INT8>, dim3(blocks), dim3(256), s, a); break;
    case KV_FMT_Q4_0: launch(gather_kernel<KV_FMT_Q4_0>, dim3(blocks), dim3(256), s, a); break;
    default: launch(gather_kernel<KV_FMT_K8V4>, dim3(blocks), dim3(256), s, a); break;
  }
  return launch_status();
}

// Yardstick for attainable HBM read bandwidth: every workgroup streams its
// own contiguous share of the buffer, its 256 lanes reading four
// consecutive 4 KB blocks per round with non-temporal 16-byte loads.  (On
// MI355X this pattern reads 6.8-7.1 TB/s over GBs; a grid-stride pattern, where
// all workgroups sweep one narrow window together, stays near 5.8 TB/s.)
// One word per workgroup is written only if the xor of everything read
// equals a value that a fill with a repeated byte cannot produce, so the
// loads are not optimized away.
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4 *buf, size_t n16, u32x4 *sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = b0 + threadIdx.x;
  for (; i + 3 * 256 < b1; i += 4 * 256) {
    u32x4 v[4];
    for (int u = 0; u < 4; u++) v[u] = __builtin_nontemporal_load(&buf[i + 256 * u]);
    for (int u = 0; u < 4; u++) acc ^= v[u];
  }
  for (; i < b1; i += 256) acc ^= __builtin_nontemporal_load(&buf[i]);
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[blockIdx.x & 255] = acc;
}

int launch_probe_read(const void *buf, size_t bytes, void *sink, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return KV_OK;
  launch(probe_read_kernel, dim3(512), dim3(256), s, (const u32x4 *)buf, n16, (u32x4 *)sink);
  return launch_status();
}

int launch_fill_zero(void *p, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return KV_OK;
  unsigned blocks = (unsigned)((words + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  launch(fill_zero_kernel, dim3(blocks), dim3(256), s, (uint32_t *)p, words);
  return launch_status();
}

}  // namespace k8v4
