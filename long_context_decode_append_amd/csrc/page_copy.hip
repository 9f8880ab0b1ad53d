// Whole-page copies between two pools of one format, for gfx950.
//
// "kv: --kv k8v4 streams with --kv-resident" (What, How, Tests): a streamed
// cache keeps every page in host memory and a window of pages in device
// memory, and moves a page as the list of its byte runs; for k8v4 these are
// three (K codes, K scales, V q4_0).  Every run of a page is copied: the
// pages' trap was a writer that tested one pointer for presence and silently
// skipped the other half's host copy.
//
// In every run a page is one contiguous block (runs are laid out
// [page][kv head][slot]), so a copy is a block move.  One kernel moves all
// runs of n pages: workgroup (i, run, chunk) copies 16 KiB of page pair i's
// block of that run with 16-byte loads and stores.  Either pool may live in
// device memory or in mapped pinned host memory (the copy then crosses the
// host link inside the kernel).
#include "device.hpp"
#include "launch.hpp"

namespace k8v4 {

constexpr int kCopyChunk = 16384;  // bytes per workgroup

struct PageCopyArgs {
  const uint8_t *src[4];
  uint8_t *dst[4];
  size_t page_bytes[4];   // bytes of one page in each run (0: run unused)
  const int32_t *src_pages;
  const int32_t *dst_pages;
  int src_n_pages, dst_n_pages;
};

__global__ __launch_bounds__(256) void page_copy_kernel(const PageCopyArgs a) {
  const int i = blockIdx.x, run = blockIdx.y;
  const size_t pb = a.page_bytes[run];
  const size_t off0 = (size_t)blockIdx.z * kCopyChunk;
  if (off0 >= pb) return;
  const int s = a.src_pages[i], d = a.dst_pages[i];
  if (s < 0 || s >= a.src_n_pages || d < 0 || d >= a.dst_n_pages) return;  // never outside a pool
  const u32x4 *src = reinterpret_cast<const u32x4 *>(a.src[run] + (size_t)s * pb + off0);
  u32x4 *dst = reinterpret_cast<u32x4 *>(a.dst[run] + (size_t)d * pb + off0);
  const size_t n16 = (pb - off0 < (size_t)kCopyChunk ? pb - off0 : (size_t)kCopyChunk) / 16;
  for (size_t k = threadIdx.x; k < n16; k += 256) dst[k] = src[k];
}

int launch_page_copy(const kv_pool *dst, const kv_pool *src, const int32_t *dst_pages, const int32_t *src_pages,
                     int n, hipStream_t s) {
  PageCopyArgs a;
  size_t max_pb = 0;
  for (int r = 0; r < 4; r++) {
    a.src[r] = (const uint8_t *)src->run[r];
    a.dst[r] = (uint8_t *)dst->run[r];
    a.page_bytes[r] = run_bytes(src->fmt, r, 1, src->page_size, src->n_kv_heads, src->head_dim);
    if (a.page_bytes[r] > max_pb) max_pb = a.page_bytes[r];
  }
  a.src_pages = src_pages;
  a.dst_pages = dst_pages;
  a.src_n_pages = src->n_pages;
  a.dst_n_pages = dst->n_pages;
  const unsigned chunks = (unsigned)((max_pb + kCopyChunk - 1) / kCopyChunk);
  launch(page_copy_kernel, dim3((unsigned)n, 4, chunks), dim3(256), s, a);
  return launch_status();
}

// Miss service of a streamed cache (kv_stream_fetch): the last n_place
// pages of the requested range, logical pages [first, first + n_place), are
// placed in the window as a ring, page i in slot i % W.  A page already in
// its slot stays; otherwise the slot's previous page becomes non-resident,
// page i takes the slot and the pair (slot, its mirror page) is listed for
// the copy kernel that follows (-1 pairs are skipped there).  One thread
// per placed page: n_place <= W consecutive pages have distinct slots, and
// a slot's previous page (the only other page the thread writes) lies
// outside the placed range, so no two threads touch one entry.  A page
// whose mirror entry is out of range is left non-resident (the attention
// then reads it from the mirror, where it gives NaN rows).
__global__ __launch_bounds__(256) void stream_place_kernel(int32_t *window_map, int32_t *owner,
                                                           const int32_t *mirror_table, int m_n_pages, int first,
                                                           int n_place, int W, int32_t *dst_list, int32_t *src_list) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= n_place) return;
  const int i = first + k;
  const int slot = i % W;
  const int mp = mirror_table[i];
  const bool fetchable = mp >= 0 && mp < m_n_pages;
  int dst = -1, src = -1;
  if (window_map[i] != slot || owner[slot] != i) {
    const int old = owner[slot];
    if (old >= 0 && old != i) window_map[old] = -1;
    owner[slot] = fetchable ? i : -1;
    window_map[i] = fetchable ? slot : -1;
    if (fetchable) {
      dst = slot;
      src = mp;
    }
  }
  dst_list[k] = dst;
  src_list[k] = src;
}

int launch_stream_fetch(const kv_stream *st, int first, int n, hipStream_t s) {
  const int W = st->window.n_pages;
  const int n_place = n < W ? n : W;
  if (n_place <= 0) return KV_OK;
  int32_t *dst_list = st->fetch_list, *src_list = st->fetch_list + W;
  launch(stream_place_kernel, dim3((unsigned)((n_place + 255) / 256)), dim3(256), s, st->window_map, st->window_owner,
         st->mirror_table, st->mirror.n_pages, first + n - n_place, n_place, W, dst_list, src_list);
  if (int e = launch_status()) return e;
  return launch_page_copy(&st->window, &st->mirror, dst_list, src_list, n_place, s);
}

}  // namespace k8v4
