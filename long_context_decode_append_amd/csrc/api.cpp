// extern "C" entry points of libk8v4.so (declared in include/k8v4.h):
// validate on the host, then enqueue the kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <mutex>
#include <vector>

#include "launch.hpp"
#include "validate.hpp"

using namespace k8v4;

static thread_local char g_last_hip_error[256] = "no error";
static thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;

namespace k8v4 {
void set_last_hip_error(hipError_t e) {
  snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
}

int launch_status() {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return KV_OK;
  set_last_hip_error(e);
  return KV_ERR_LAUNCH;
}

void take_launch_events(hipEvent_t *start, hipEvent_t *stop) {
  *start = g_ev_start;
  *stop = g_ev_stop;
  g_ev_start = g_ev_stop = nullptr;
}
}  // namespace k8v4

// ---------------------------------------------------------------- scratch
// Split-K partials of attn_decode_noalloc (see there).  A decode plan has
// about one split-K workgroup per compute unit, each writing 8 rows of
// 258 floats, so KV_SCRATCH_BYTES (4 MiB) holds the partials of any decode on
// a GPU of up to ~500 compute units.
static __device__ __align__(256) unsigned char scratch[KV_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` per device, set under g_scratch_mu

// Device address of `scratch` on the current device (looked up on the first
// call on that device).  KV_ERR_LAUNCH if the runtime cannot resolve it.
int scratch_of_current_device(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
  if (e == hipSuccess) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
      void *p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e == hipSuccess && !p) e = hipErrorInvalidSymbol;
      if (e == hipSuccess) g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    set_last_hip_error(e);
    return KV_ERR_LAUNCH;
  }
  return KV_OK;
}
}  // namespace

namespace {
// Scope of one entry-point call that may launch work.  On entry it clears
// the HIP runtime's per-thread error slot, so a KV_ERR_LAUNCH returned by
// this call is this call's own failure and never one left behind by an
// earlier, unrelated HIP call.  On every return path it disarms a
// kv_time_next_launch hook that this call did not consume (errors, empty
// work), so the events never attach to a later, unrelated launch.
struct CallScope {
  CallScope() { (void)hipGetLastError(); }
  ~CallScope() {
    hipEvent_t a, b;
    take_launch_events(&a, &b);
  }
  CallScope(const CallScope &) = delete;
  CallScope &operator=(const CallScope &) = delete;
};
}  // namespace

extern "C" {

size_t kv_cell_bytes(int fmt, int n_kv_heads, int head_dim) {
  return cell_bytes(fmt, n_kv_heads, head_dim);
}

size_t kv_run_bytes(int fmt, int run, int n_pages, int page_size, int n_kv_heads, int head_dim) {
  if (run < 0 || run > 3) return 0;
  return run_bytes(fmt, run, n_pages, page_size, n_kv_heads, head_dim);
}

const char *kv_strerror(int code) {
  switch (code) {
    case KV_OK: return "ok";
    case KV_ERR_NULL: return "a required pointer is NULL";
    case KV_ERR_SHAPE: return "inconsistent sizes";
    case KV_ERR_RANGE: return "positions or context outside the page table or pool";
    case KV_ERR_DTYPE: return "unknown dtype";
    case KV_ERR_UNSUPPORTED: return "unsupported format, head_dim, GQA ratio or page size";
    case KV_ERR_WORKSPACE: return "workspace missing or too small";
    case KV_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case KV_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown error";
  }
}

const char *kv_last_hip_error(void) { return g_last_hip_error; }

int kv_time_next_launch(void *start_event, void *stop_event) {
  if (!start_event || !stop_event) return KV_ERR_NULL;
  g_ev_start = (hipEvent_t)start_event;
  g_ev_stop = (hipEvent_t)stop_event;
  return KV_OK;
}

int kv_append_k8v4(const kv_pool *pool, const kv_seq *seq, const void *k, const void *v,
                   int dtype, int32_t pos0, int32_t n_tokens, void *stream) {
  CallScope scope;
  if (int e = check_pool(pool, KV_FMT_K8V4)) return e;
  if (int e = check_seq(seq, pool)) return e;
  if (!k || !v) return KV_ERR_NULL;
  if (int e = check_dtype(dtype)) return e;
  if (int e = check_range(pool, seq, pos0, n_tokens)) return e;
  if (check_aligned16(k) || check_aligned16(v)) return KV_ERR_ALIGN;
  if (n_tokens == 0) return KV_OK;
  return launch_append(pool, seq, k, v, dtype, pos0, n_tokens, (hipStream_t)stream);
}

int kv_append(const kv_pool *pool, const kv_seq *seq, const void *k, const void *v, int dtype, int32_t pos0,
              int32_t n_tokens, void *stream) {
  CallScope scope;
  if (int e = check_pool(pool, 0)) return e;
  if (int e = check_seq(seq, pool)) return e;
  if (!k || !v) return KV_ERR_NULL;
  if (int e = check_dtype(dtype)) return e;
  if (int e = check_range(pool, seq, pos0, n_tokens)) return e;
  if (check_aligned16(k) || check_aligned16(v)) return KV_ERR_ALIGN;
  if (n_tokens == 0) return KV_OK;
  return launch_append(pool, seq, k, v, dtype, pos0, n_tokens, (hipStream_t)stream);
}

int kv_gather(const kv_pool *pool, const kv_seq *seq, int32_t pos0, int32_t n, void *k_codes,
              void *k_scales, void *v_blocks, void *stream) {
  CallScope scope;
  if (int e = check_pool(pool, KV_FMT_K8V4)) return e;
  if (int e = check_seq(seq, pool)) return e;
  if (!k_codes || !k_scales || !v_blocks) return KV_ERR_NULL;
  if (int e = check_range(pool, seq, pos0, n)) return e;
  if (check_aligned16(k_codes) || ((uintptr_t)k_scales & 7u)) return KV_ERR_ALIGN;
  if (n == 0) return KV_OK;
  void *const out[4] = {k_codes, k_scales, v_blocks, nullptr};
  return launch_gather(pool, seq, pos0, n, out, (hipStream_t)stream);
}

int kv_gather_runs(const kv_pool *pool, const kv_seq *seq, int32_t pos0, int32_t n, void *out0, void *out1,
                   void *out2, void *out3, void *stream) {
  CallScope scope;
  if (int e = check_pool(pool, 0)) return e;
  if (int e = check_seq(seq, pool)) return e;
  const int fmt = pool->fmt;
  void *const out[4] = {out0, out1, out2, out3};
  // int8-coded halves: codes (16-byte aligned) + scales (8-byte aligned);
  // q4_0-coded halves: one block array (any alignment)
  // fp16 halves: one [n][H][256] fp16 array each (16-byte aligned)
  const bool k_int8 = fmt == KV_FMT_INT8 || fmt == KV_FMT_K8V4, v_int8 = fmt == KV_FMT_INT8;
  if (!out0 || !out2 || (k_int8 && !out1) || (v_int8 && !out3)) return KV_ERR_NULL;
  if (int e = check_range(pool, seq, pos0, n)) return e;
  if (fmt == KV_FMT_F16 && (check_aligned16(out0) || check_aligned16(out2))) return KV_ERR_ALIGN;
  if (k_int8 && (check_aligned16(out0) || ((uintptr_t)out1 & 7u))) return KV_ERR_ALIGN;
  if (v_int8 && (check_aligned16(out2) || ((uintptr_t)out3 & 7u))) return KV_ERR_ALIGN;
  if (n == 0) return KV_OK;
  return launch_gather(pool, seq, pos0, n, out, (hipStream_t)stream);
}

size_t attn_workspace_bytes(const kv_pool *pool, int n_q_heads, int32_t n_q, int32_t max_ctx) {
  if (!pool || pool->n_kv_heads <= 0 || n_q < 1 || n_q > kMaxQ || max_ctx < 1) return 0;
  if (n_q_heads != kGqa * pool->n_kv_heads) return 0;
  return ws_bytes_bound(pool->n_kv_heads, n_q * kGqa, max_ctx);
}

int kv_workspace_init(void *ws, size_t ws_bytes, void *stream) {
  CallScope scope;
  if (!ws) return KV_ERR_NULL;
  if (check_aligned16(ws)) return KV_ERR_ALIGN;
  return launch_fill_zero(ws, ws_bytes, (hipStream_t)stream);
}

int kv_copy_pages(const kv_pool *dst, const kv_pool *src, const int32_t *dst_pages, const int32_t *src_pages,
                  int32_t n, void *stream) {
  CallScope scope;
  if (int e = check_pool(dst, 0)) return e;
  if (int e = check_pool(src, 0)) return e;
  if (dst->fmt != src->fmt || dst->n_kv_heads != src->n_kv_heads || dst->page_size != src->page_size)
    return KV_ERR_SHAPE;
  if (n < 0) return KV_ERR_RANGE;
  if (n == 0) return KV_OK;
  if (!dst_pages || !src_pages) return KV_ERR_NULL;
  return launch_page_copy(dst, src, dst_pages, src_pages, n, (hipStream_t)stream);
}

int kv_probe_read(const void *buf, size_t bytes, void *sink, void *stream) {
  CallScope scope;
  if (!buf || !sink) return KV_ERR_NULL;
  if (check_aligned16(buf) || check_aligned16(sink)) return KV_ERR_ALIGN;
  return launch_probe_read(buf, bytes, sink, (hipStream_t)stream);
}

static int check_attn_common(const kv_pool *pool, const kv_seq *seq, const void *q, int q_dtype,
                             int n_q_heads, const float *out, int need_fmt) {
  if (int e = check_pool(pool, need_fmt)) return e;
  if (int e = check_seq(seq, pool)) return e;
  if (!q || !out) return KV_ERR_NULL;
  if (int e = check_dtype(q_dtype)) return e;
  if (n_q_heads != kGqa * pool->n_kv_heads) return KV_ERR_UNSUPPORTED;
  if (check_aligned16(q) || check_aligned16(out)) return KV_ERR_ALIGN;
  return KV_OK;
}

static float pick_scale(float scale) {
  return scale > 0.0f ? scale : 1.0f / std::sqrt((float)kHeadDim);
}

static int decode_call(const kv_pool *pool, const kv_seq *seq, const void *q, int q_dtype, int n_q_heads,
                       int32_t n_ctx, float scale, float *out, void *ws, size_t ws_bytes, void *stream) {
  AttnCall c;
  c.pool = pool;
  c.seq = seq;
  c.q = q;
  c.q_dtype = q_dtype;
  c.n_q_heads = n_q_heads;
  c.n_q = 1;
  for (int i = 0; i < kMaxQ; i++) c.limits[i] = 0;
  c.limits[0] = n_ctx;
  c.max_limit = n_ctx;
  c.scale = pick_scale(scale);
  c.out = out;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = (hipStream_t)stream;
  return launch_attn_splitk(c);
}

int attn_decode(const kv_pool *pool, const kv_seq *seq, const void *q, int q_dtype,
                int n_q_heads, int32_t n_ctx, float scale, float *out, void *ws,
                size_t ws_bytes, void *stream) {
  CallScope scope;
  if (int e = check_attn_common(pool, seq, q, q_dtype, n_q_heads, out, 0)) return e;
  if (n_ctx < 1) return KV_ERR_RANGE;
  if (int e = check_range(pool, seq, 0, n_ctx)) return e;
  if (!ws) return KV_ERR_WORKSPACE;
  if (check_aligned16(ws)) return KV_ERR_ALIGN;
  return decode_call(pool, seq, q, q_dtype, n_q_heads, n_ctx, scale, out, ws, ws_bytes, stream);
}

int attn_decode_append(const kv_pool *pool, const kv_seq *seq, const void *k_new, const void *v_new,
                       int kv_dtype, const void *q, int q_dtype, int n_q_heads, int32_t pos, float scale,
                       float *out, void *ws, size_t ws_bytes, void *stream) {
  CallScope scope;
  if (int e = check_attn_common(pool, seq, q, q_dtype, n_q_heads, out, KV_FMT_K8V4)) return e;
  if (!k_new || !v_new) return KV_ERR_NULL;
  if (int e = check_dtype(kv_dtype)) return e;
  if (check_aligned16(k_new) || check_aligned16(v_new)) return KV_ERR_ALIGN;
  if (pos < 0) return KV_ERR_RANGE;
  if (int e = check_range(pool, seq, 0, (int64_t)pos + 1)) return e;
  if (!ws) return KV_ERR_WORKSPACE;
  if (check_aligned16(ws)) return KV_ERR_ALIGN;
  AttnCall c;
  c.pool = pool;
  c.seq = seq;
  c.q = q;
  c.q_dtype = q_dtype;
  c.n_q_heads = n_q_heads;
  c.n_q = 1;
  for (int i = 0; i < kMaxQ; i++) c.limits[i] = 0;
  c.limits[0] = pos;  // cells streamed from the pool; the new one is added by the kernel
  c.max_limit = pos;
  c.scale = pick_scale(scale);
  c.out = out;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = (hipStream_t)stream;
  c.k_new = k_new;
  c.v_new = v_new;
  c.kv_dtype = kv_dtype;
  c.append_pos = pos;
  return launch_attn_splitk(c);
}

int attn_decode_batch(const kv_pool *pool, const kv_seq *seqs, int32_t n_seq, const void *q, int q_dtype,
                      int n_q_heads, const int32_t *n_ctx, float scale, float *out, void *ws, size_t ws_bytes,
                      void *stream) {
  CallScope scope;
  if (!seqs || !n_ctx) return KV_ERR_NULL;
  if (n_seq < 1 || n_seq > kMaxQ) return KV_ERR_SHAPE;
  if (int e = check_attn_common(pool, &seqs[0], q, q_dtype, n_q_heads, out, 0)) return e;
  if (!ws) return KV_ERR_WORKSPACE;
  if (check_aligned16(ws)) return KV_ERR_ALIGN;
  AttnCall c;
  c.batch = true;
  c.max_limit = 0;
  for (int i = 0; i < kMaxQ; i++) c.limits[i] = 0;
  for (int i = 0; i < n_seq; i++) {
    if (int e = check_seq(&seqs[i], pool)) return e;
    if (n_ctx[i] < 1) return KV_ERR_RANGE;
    if (int e = check_range(pool, &seqs[i], 0, n_ctx[i])) return e;
    c.limits[i] = n_ctx[i];
    c.pts[i] = seqs[i].page_table;
    if (n_ctx[i] > c.max_limit) c.max_limit = n_ctx[i];
  }
  c.pool = pool;
  c.seq = &seqs[0];
  c.q = q;
  c.q_dtype = q_dtype;
  c.n_q_heads = n_q_heads;
  c.n_q = n_seq;
  c.scale = pick_scale(scale);
  c.out = out;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = (hipStream_t)stream;
  return launch_attn_splitk(c);
}

int attn_verify(const kv_pool *pool, const kv_seq *seq, const void *q, int q_dtype,
                int n_q_heads, int32_t n_q, const int32_t *n_visible, float scale, float *out,
                void *ws, size_t ws_bytes, void *stream) {
  CallScope scope;
  if (int e = check_attn_common(pool, seq, q, q_dtype, n_q_heads, out, 0)) return e;
  if (!n_visible) return KV_ERR_NULL;
  if (n_q < 1 || n_q > kMaxQ) return KV_ERR_SHAPE;
  if (!ws) return KV_ERR_WORKSPACE;
  if (check_aligned16(ws)) return KV_ERR_ALIGN;
  AttnCall c;
  c.max_limit = 0;
  for (int i = 0; i < kMaxQ; i++) c.limits[i] = 0;
  for (int i = 0; i < n_q; i++) {
    if (n_visible[i] < 1) return KV_ERR_RANGE;
    if (int e = check_range(pool, seq, 0, n_visible[i])) return e;
    c.limits[i] = n_visible[i];
    if (n_visible[i] > c.max_limit) c.max_limit = n_visible[i];
  }
  c.pool = pool;
  c.seq = seq;
  c.q = q;
  c.q_dtype = q_dtype;
  c.n_q_heads = n_q_heads;
  c.n_q = n_q;
  c.scale = pick_scale(scale);
  c.out = out;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = (hipStream_t)stream;
  return launch_attn_splitk(c);
}

int attn_prefill_chunk(const kv_pool *pool, const kv_seq *seq, const void *q, int q_dtype,
                       int n_q_heads, int32_t pos0, int32_t n_new, float scale, float *out,
                       void *ws, size_t ws_bytes, void *stream) {
  CallScope scope;
  if (int e = check_attn_common(pool, seq, q, q_dtype, n_q_heads, out, 0)) return e;
  if (pos0 < 0 || n_new < 0) return KV_ERR_RANGE;
  if (int e = check_range(pool, seq, 0, (int64_t)pos0 + n_new)) return e;
  if (n_new == 0) return KV_OK;
  if (!ws || ws_bytes < prefill_workspace_bytes(pool, (int64_t)pos0 + n_new)) return KV_ERR_WORKSPACE;
  if (int e = check_aligned16(ws)) return e;
  return launch_attn_prefill(pool, seq, q, q_dtype, n_q_heads, pos0, n_new, pick_scale(scale), out, ws,
                             (hipStream_t)stream);
}

size_t attn_prefill_workspace_bytes(const kv_pool *pool, int32_t n_cells) {
  if (!pool || pool->n_kv_heads <= 0 || n_cells <= 0) return 0;
  return prefill_workspace_bytes(pool, n_cells);
}

int kv_check_page_table(const kv_pool *pool, const kv_seq *seq, int32_t n_cells, int32_t *n_bad) {
  CallScope scope;
  if (int e = check_pool(pool, 0)) return e;
  if (int e = check_seq(seq, pool)) return e;
  if (!n_bad) return KV_ERR_NULL;
  if (int e = check_range(pool, seq, 0, n_cells)) return e;
  const int n_pages_used = (int)(((int64_t)n_cells + pool->page_size - 1) / pool->page_size);
  std::vector<int32_t> host(n_pages_used > 0 ? n_pages_used : 1);
  if (n_pages_used > 0 &&
      hipMemcpy(host.data(), seq->page_table, sizeof(int32_t) * n_pages_used, hipMemcpyDeviceToHost) !=
          hipSuccess)
    return KV_ERR_LAUNCH;
  std::vector<unsigned char> seen(pool->n_pages, 0);
  int bad = 0;
  for (int i = 0; i < n_pages_used; i++) {
    const int p = host[i];
    if (p < 0 || p >= pool->n_pages || seen[p]) {
      bad++;
      continue;
    }
    seen[p] = 1;
  }
  *n_bad = bad;
  return KV_OK;
}

// ---------------------------------------------------------------- streamed cache

static int check_stream(const kv_stream *s) {
  if (!s) return KV_ERR_NULL;
  if (int e = check_pool(&s->window, 0)) return e;
  if (int e = check_pool(&s->mirror, 0)) return e;
  if (s->window.fmt != s->mirror.fmt || s->window.n_kv_heads != s->mirror.n_kv_heads ||
      s->window.page_size != s->mirror.page_size)
    return KV_ERR_SHAPE;
  if (!s->mirror_table || !s->window_map || !s->window_owner || !s->stats || !s->fetch_list) return KV_ERR_NULL;
  if (s->n_table < 0) return KV_ERR_SHAPE;
  if ((int64_t)s->n_table * s->window.page_size > ((int64_t)1 << 31) - 1) return KV_ERR_RANGE;
  return KV_OK;
}

static kv_seq stream_seq(const kv_stream *s) {
  kv_seq q;
  q.page_table = s->window_map;
  q.n_table = s->n_table;
  q.reserved = 0;
  return q;
}

int kv_stream_append(const kv_stream *s, const void *k, const void *v, int dtype, int32_t pos0, int32_t n_tokens,
                     void *stream) {
  CallScope scope;
  if (int e = check_stream(s)) return e;
  if (!k || !v) return KV_ERR_NULL;
  if (int e = check_dtype(dtype)) return e;
  kv_seq mq;
  mq.page_table = s->mirror_table;
  mq.n_table = s->n_table;
  mq.reserved = 0;
  if (int e = check_range(&s->mirror, &mq, pos0, n_tokens)) return e;
  if (check_aligned16(k) || check_aligned16(v)) return KV_ERR_ALIGN;
  if (n_tokens == 0) return KV_OK;
  return launch_append(&s->mirror, &mq, k, v, dtype, pos0, n_tokens, (hipStream_t)stream, &s->window, s->window_map);
}

int kv_stream_fetch(const kv_stream *s, int32_t first_page, int32_t n_pages, void *stream) {
  CallScope scope;
  if (int e = check_stream(s)) return e;
  if (first_page < 0 || n_pages < 0 || (int64_t)first_page + n_pages > s->n_table) return KV_ERR_RANGE;
  if (n_pages == 0) return KV_OK;
  return launch_stream_fetch(s, first_page, n_pages, (hipStream_t)stream);
}

int attn_decode_stream(const kv_stream *s, const void *q, int q_dtype, int n_q_heads, int32_t n_ctx, float scale,
                       float *out, void *ws, size_t ws_bytes, void *stream) {
  CallScope scope;
  if (int e = check_stream(s)) return e;
  const kv_seq seq = stream_seq(s);
  if (int e = check_attn_common(&s->window, &seq, q, q_dtype, n_q_heads, out, 0)) return e;
  if (n_ctx < 1) return KV_ERR_RANGE;
  if (int e = check_range(&s->window, &seq, 0, n_ctx)) return e;
  if (!ws) return KV_ERR_WORKSPACE;
  if (check_aligned16(ws)) return KV_ERR_ALIGN;
  AttnCall c;
  c.pool = &s->window;
  c.seq = &seq;
  c.q = q;
  c.q_dtype = q_dtype;
  c.n_q_heads = n_q_heads;
  c.n_q = 1;
  for (int i = 0; i < kMaxQ; i++) c.limits[i] = 0;
  c.limits[0] = n_ctx;
  c.max_limit = n_ctx;
  c.scale = pick_scale(scale);
  c.out = out;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = (hipStream_t)stream;
  c.stream_s = s;
  return launch_attn_splitk(c);
}

int attn_verify_stream(const kv_stream *s, const void *q, int q_dtype, int n_q_heads, int32_t n_q,
                       const int32_t *n_visible, float scale, float *out, void *ws, size_t ws_bytes, void *stream) {
  CallScope scope;
  if (int e = check_stream(s)) return e;
  const kv_seq seq = stream_seq(s);
  if (int e = check_attn_common(&s->window, &seq, q, q_dtype, n_q_heads, out, 0)) return e;
  if (!n_visible) return KV_ERR_NULL;
  if (n_q < 1 || n_q > kMaxQ) return KV_ERR_SHAPE;
  if (!ws) return KV_ERR_WORKSPACE;
  if (check_aligned16(ws)) return KV_ERR_ALIGN;
  AttnCall c;
  c.max_limit = 0;
  for (int i = 0; i < kMaxQ; i++) c.limits[i] = 0;
  for (int i = 0; i < n_q; i++) {
    if (n_visible[i] < 1) return KV_ERR_RANGE;
    if (int e = check_range(&s->window, &seq, 0, n_visible[i])) return e;
    c.limits[i] = n_visible[i];
    if (n_visible[i] > c.max_limit) c.max_limit = n_visible[i];
  }
  c.pool = &s->window;
  c.seq = &seq;
  c.q = q;
  c.q_dtype = q_dtype;
  c.n_q_heads = n_q_heads;
  c.n_q = n_q;
  c.scale = pick_scale(scale);
  c.out = out;
  c.ws = ws;
  c.ws_bytes = ws_bytes;
  c.stream = (hipStream_t)stream;
  c.stream_s = s;
  return launch_attn_splitk(c);
}

// attn_decode for callers that cannot allocate device memory: the split-K
// partials go to `scratch`, a file-scope device array that every GPU the
// library runs on holds (its own copy, at its own address) until the
// process ends.  On the host the name `scratch` is only a stand-in for the
// device symbol, never a device address: host code uses the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device on the first call there and kept in g_scratch.
int attn_decode_noalloc(const kv_pool *pool, const kv_seq *seq, const void *q, int q_dtype, int n_q_heads,
                        int32_t n_ctx, float scale, float *out, void *stream) {
  CallScope scope;
  if (int e = check_attn_common(pool, seq, q, q_dtype, n_q_heads, out, 0)) return e;
  if (n_ctx < 1) return KV_ERR_RANGE;
  if (int e = check_range(pool, seq, 0, n_ctx)) return e;
  void *ws = nullptr;
  if (int e = scratch_of_current_device(&ws)) return e;
  // the launcher checks the plan's partials against this size and returns
  // KV_ERR_WORKSPACE before launching when they do not fit
  return decode_call(pool, seq, q, q_dtype, n_q_heads, n_ctx, scale, out, ws, KV_SCRATCH_BYTES, stream);
}

}  // extern "C"
