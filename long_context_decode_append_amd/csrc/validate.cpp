// Host-side argument checks and launch planning (see validate.hpp).
#include "validate.hpp"

namespace k8v4 {

static bool fmt_known(int fmt) {
  return fmt == KV_FMT_F16 || fmt == KV_FMT_INT8 || fmt == KV_FMT_Q4_0 || fmt == KV_FMT_K8V4;
}

size_t cell_bytes(int fmt, int n_kv_heads, int head_dim) {
  if (!fmt_known(fmt) || n_kv_heads <= 0 || head_dim != kHeadDim) return 0;
  const size_t int8_half = head_dim + 4 * (head_dim / 128);  // codes + fp32 scale per 128
  const size_t q4_half = (head_dim / 32) * 18;               // 18-byte blocks of 32
  size_t per_head = 0;
  switch (fmt) {
    case KV_FMT_F16: per_head = 2 * 2 * (size_t)head_dim; break;
    case KV_FMT_INT8: per_head = 2 * int8_half; break;
    case KV_FMT_Q4_0: per_head = 2 * q4_half; break;
    default: per_head = int8_half + q4_half; break;
  }
  return per_head * (size_t)n_kv_heads;
}

size_t run_bytes(int fmt, int run, int n_pages, int page_size, int n_kv_heads, int head_dim) {
  if (!fmt_known(fmt) || n_pages <= 0 || page_size <= 0 || n_kv_heads <= 0 || head_dim != kHeadDim)
    return 0;
  const size_t cells = (size_t)n_pages * page_size * n_kv_heads;  // head-cells
  const size_t codes = cells * head_dim, scales = cells * 4 * (head_dim / 128);
  const size_t q4 = cells * (head_dim / 32) * 18;
  switch (fmt) {
    case KV_FMT_K8V4: return run == 0 ? codes : run == 1 ? scales : run == 2 ? q4 : 0;
    case KV_FMT_INT8: return run == 0 || run == 2 ? codes : scales;
    case KV_FMT_F16: return run == 0 || run == 2 ? 2 * codes : 0;
    default: return run == 0 || run == 2 ? q4 : 0;
  }
}

int check_aligned16(const void *p) {
  return ((uintptr_t)p & 15u) ? KV_ERR_ALIGN : KV_OK;
}

int check_pool(const kv_pool *pool, int need_fmt) {
  if (!pool) return KV_ERR_NULL;
  if (!fmt_known(pool->fmt)) return KV_ERR_UNSUPPORTED;
  if (need_fmt && pool->fmt != need_fmt) return KV_ERR_UNSUPPORTED;
  if (pool->head_dim != kHeadDim) return KV_ERR_UNSUPPORTED;
  if (pool->page_size <= 0 || pool->page_size % 16) return KV_ERR_UNSUPPORTED;
  if (pool->n_kv_heads <= 0 || pool->n_pages <= 0) return KV_ERR_SHAPE;
  for (int r = 0; r < 4; r++) {
    if (run_bytes(pool->fmt, r, pool->n_pages, pool->page_size, pool->n_kv_heads, pool->head_dim) == 0)
      continue;
    if (!pool->run[r]) return KV_ERR_NULL;
    if (int e = check_aligned16(pool->run[r])) return e;
  }
  // every byte offset the kernels form must fit in 63 bits and every
  // element index of a run in 32 bits of head-cells
  const int64_t head_cells = (int64_t)pool->n_pages * pool->page_size * pool->n_kv_heads;
  if (head_cells > (int64_t)1 << 31) return KV_ERR_RANGE;
  return KV_OK;
}

int check_seq(const kv_seq *seq, const kv_pool *pool) {
  if (!seq) return KV_ERR_NULL;
  if (!seq->page_table) return KV_ERR_NULL;
  if (seq->n_table < 0) return KV_ERR_SHAPE;
  if ((int64_t)seq->n_table * pool->page_size > ((int64_t)1 << 31) - 1) return KV_ERR_RANGE;
  return KV_OK;
}

int check_dtype(int dtype) {
  return dtype == KV_DTYPE_F16 || dtype == KV_DTYPE_F32 ? KV_OK : KV_ERR_DTYPE;
}

int check_range(const kv_pool *pool, const kv_seq *seq, int64_t pos0, int64_t n) {
  if (pos0 < 0 || n < 0) return KV_ERR_RANGE;
  if (pos0 + n > (int64_t)seq->n_table * pool->page_size) return KV_ERR_RANGE;
  return KV_OK;
}

SplitPlan plan_splits(int64_t n_ctx, int target_splits_per_head) {
  SplitPlan p;
  const int64_t steps = (n_ctx + kStep - 1) / kStep;
  int64_t s = target_splits_per_head;
  if (s > kMaxSplitsPerHead) s = kMaxSplitsPerHead;
  const int64_t by_work = (steps + kWaves - 1) / kWaves;  // at least one step per wave
  if (s > by_work) s = by_work;
  if (s < 1) s = 1;
  // whole rounds of the workgroup's waves, so they finish together
  int64_t per = (steps + s - 1) / s;
  per = (per + kWaves - 1) / kWaves * kWaves;
  p.steps_per_split = (int)per;
  p.n_splits = (int)((steps + p.steps_per_split - 1) / p.steps_per_split);
  return p;
}

static size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(int n_kv_heads, int n_rows, int n_splits) {
  WsLayout w;
  size_t off = 0;
  w.part_ml = off;
  off = up256(off + 8 * (size_t)n_kv_heads * n_splits * n_rows);
  w.part_o = off;
  off = up256(off + 4 * (size_t)kHeadDim * n_kv_heads * n_splits * n_rows);
  w.total = off;
  return w;
}

size_t ws_bytes_bound(int n_kv_heads, int n_rows, int64_t max_ctx) {
  // plan_splits never returns more splits than min(kMaxSplitsPerHead,
  // ceil(steps / kWaves)), which grows with the context: a bound for every
  // context up to max_ctx and every device
  const int64_t steps = (max_ctx + kStep - 1) / kStep;
  int64_t s = (steps + kWaves - 1) / kWaves;
  if (s < 1) s = 1;
  s += 1;  // the partial of a fused append (attn_decode_append)
  if (s > kMaxSplitsPerHead) s = kMaxSplitsPerHead;
  return ws_layout(n_kv_heads, n_rows, (int)s).total;
}

}  // namespace k8v4
