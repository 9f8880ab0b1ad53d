// Kernel launchers of libk8v4 (host side; arguments already validated).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "validate.hpp"

namespace k8v4 {

// KV_OK after a successful launch, else KV_ERR_LAUNCH (the HIP error is kept
// per thread for kv_last_hip_error).
int launch_status();

// Record e as the calling thread's HIP error for kv_last_hip_error.
void set_last_hip_error(hipError_t e);

// Start/stop events armed by kv_time_next_launch for the calling thread's
// next kernel launch (both NULL when none); taking them disarms the hook.
void take_launch_events(hipEvent_t *start, hipEvent_t *stop);

// Enqueue `kernel` on stream s (static shared memory only), recording the
// armed timing events around it if any.
template <typename Kernel, typename... Args>
inline void launch(Kernel kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  hipEvent_t e0, e1;
  take_launch_events(&e0, &e1);
  hipExtLaunchKernelGGL(kernel, grid, block, 0, s, e0, e1, 0, args...);
}

// pool2 / pt2 (optional): a second copy of the same cells (a streamed
// cache's window), written from the same quantization
int launch_append(const kv_pool *pool, const kv_seq *seq, const void *k, const void *v, int dtype, int pos0,
                  int n, hipStream_t s, const kv_pool *pool2 = nullptr, const int32_t *pt2 = nullptr);
int launch_gather(const kv_pool *pool, const kv_seq *seq, int pos0, int n, void *const out[4], hipStream_t s);
int launch_fill_zero(void *p, size_t bytes, hipStream_t s);
int launch_page_copy(const kv_pool *dst, const kv_pool *src, const int32_t *dst_pages, const int32_t *src_pages,
                     int n, hipStream_t s);
// kv_stream_fetch: ring placement of logical pages [first, first + n) in the
// window (bookkeeping kernel), then the page copies it lists
int launch_stream_fetch(const kv_stream *st, int first, int n, hipStream_t s);
int launch_probe_read(const void *buf, size_t bytes, void *sink, hipStream_t s);

// Decode / verify: n_q query rows of 8 heads per KV head, row i of query
// q_index attends to cells [0, limits[i]).
struct AttnCall {
  const kv_pool *pool;
  const kv_seq *seq;
  const void *q;
  int q_dtype;
  int n_q_heads;
  int n_q;
  int limits[kMaxQ];
  int max_limit;
  float scale;
  float *out;
  void *ws;
  size_t ws_bytes;
  hipStream_t stream;
  // fused append (decode of a k8v4 pool only): token [H][256] of kv_dtype
  // stored at cell append_pos = max_limit before attending; -1 for none
  const void *k_new = nullptr;
  const void *v_new = nullptr;
  int kv_dtype = 0;
  int append_pos = -1;
  // batch decode: n_q independent sequences (8 rows each), sequence i with
  // table pts[i] and length limits[i]; seq is then unused
  bool batch = false;
  const int32_t *pts[kMaxQ] = {};
  // streamed cache (decode / verify): pool is the window, seq's table the
  // window map; pages not resident are read from the mirror
  const kv_stream *stream_s = nullptr;
};
int launch_attn_splitk(const AttnCall &c);

// Target number of split-K workgroups per KV head on the current device.
int attn_target_splits(int n_kv_heads, int n_rows);

// Prefill: a staging kernel writes each 32-cell tile of every KV head as
// the attention kernel's LDS image into ws (prefill_workspace_bytes for
// pos0 + n_new cells), then the attention kernel copies tiles from there.
size_t prefill_workspace_bytes(const kv_pool *pool, int64_t n_cells);
int launch_attn_prefill(const kv_pool *pool, const kv_seq *seq, const void *q, int q_dtype,
                        int n_q_heads, int pos0, int n_new, float scale, float *out, void *ws,
                        hipStream_t s);

}  // namespace k8v4
