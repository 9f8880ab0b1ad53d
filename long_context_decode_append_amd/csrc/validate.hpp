// Host-side argument checks and launch planning for libk8v4 (pure C++:
// no HIP calls, so every rule here can be exercised without a GPU).
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/k8v4.h"

namespace k8v4 {

constexpr int kHeadDim = 256;
constexpr int kGqa = 8;          // query heads per KV head
constexpr int kStep = 32;        // cells per attention step of one wave
constexpr int kWaves = 4;        // waves per attention workgroup
constexpr int kMaxRows = 128;    // verify: at most 16 queries x 8 heads
constexpr int kMaxQ = 16;
constexpr int kMaxSplitsPerHead = 256;
constexpr int kMaxPasses = 8;    // row passes (16 rows each) of one verify call

int check_pool(const kv_pool *pool, int need_fmt);
int check_seq(const kv_seq *seq, const kv_pool *pool);
int check_dtype(int dtype);
int check_range(const kv_pool *pool, const kv_seq *seq, int64_t pos0, int64_t n);
int check_aligned16(const void *p);

// Split-K plan for decode/verify over cells [0, n_ctx).
struct SplitPlan {
  int steps_per_split;  // kStep-cell steps per split (a multiple of kWaves)
  int n_splits;         // splits per KV head
};
SplitPlan plan_splits(int64_t n_ctx, int target_splits_per_head);

// Workspace layout (byte offsets) for n_rows query rows and a plan.
struct WsLayout {
  size_t part_ml;   // float2 [H][n_splits][n_rows]
  size_t part_o;    // float  [H][n_splits][n_rows][256]
  size_t total;
};
WsLayout ws_layout(int n_kv_heads, int n_rows, int n_splits);

// Upper bound used by attn_workspace_bytes: the largest plan any device
// can choose for max_ctx cells.
size_t ws_bytes_bound(int n_kv_heads, int n_rows, int64_t max_ctx);

size_t cell_bytes(int fmt, int n_kv_heads, int head_dim);
size_t run_bytes(int fmt, int run, int n_pages, int page_size, int n_kv_heads, int head_dim);

}  // namespace k8v4
