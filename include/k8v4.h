/*
 * k8v4.h -- C ABI of libk8v4.so: the hybrid "k8v4" quantized KV cache
 * (INT8 K + Walsh-Hadamard-rotated Q4_0 V) and the fused attention that
 * reads it, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the pages
 *   "#120 --kv k8v4: hybrid KV cache -- INT8 K + Hadamard-rotated Q4_0 V
 *    (816 B/cell)"  (sections What, How, Tests)  and
 *   "kv: --kv k8v4 streams with --kv-resident" (section How: a k8v4 block
 *    is moved as three byte runs -- K codes, K scales, V q4_0).
 * The int8 and q4_0 formats those pages compare against run through the
 * same entry points (kv_append, kv_gather_runs, attention).
 *
 * Conventions for every call below:
 *   - Pointers named "device" are HIP device memory owned by the caller;
 *     "host" pointers are read during the call only.  The library never
 *     allocates or frees memory (attn_decode_noalloc uses a fixed
 *     file-scope device array instead of a workspace) and never
 *     synchronizes, except the debug call kv_check_page_table, which copies
 *     the table to the host.
 *   - Calls that take a stream only enqueue work on it (a hipStream_t, or
 *     NULL for the null stream) and return; device faults surface at the
 *     caller's next synchronization.
 *   - Every call returns KV_OK (0) or a negative KV_ERR_* code and launches
 *     nothing when it returns an error found by its argument checks.  A HIP
 *     error left by earlier, unrelated HIP calls on the calling thread is
 *     cleared on entry, so KV_ERR_LAUNCH always reports the call's own
 *     launch (kv_last_hip_error names it).  A required pointer that is NULL is
 *     an error (KV_ERR_NULL), never a silent skip: the pages report silent
 *     wrong output from writers that tested a pointer for presence and
 *     skipped the write.
 *   - Shapes supported: head_dim 256, query heads = 8 * KV heads (GQA 8),
 *     page_size a positive multiple of 16.  Anything else is
 *     KV_ERR_UNSUPPORTED.
 *   - Page-table contents live in device memory and are the caller's
 *     contract: entries must lie in [0, n_pages) and be distinct.  The
 *     kernels never access memory through an out-of-range entry: appends
 *     through one write nothing, attention rows that meet one return NaN.
 *     kv_check_page_table() validates a table synchronously.
 */
#ifndef K8V4_H
#define K8V4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* KV formats.  The numbering keeps k8v4 = 3, the number the pages give it
 * in the engine's format enum ("kv: --kv k8v4 streams with --kv-resident",
 * How).  1 and 2 are the int8 and q4_0 formats the pages compare against. */
enum { KV_FMT_F16 = 0, KV_FMT_INT8 = 1, KV_FMT_Q4_0 = 2, KV_FMT_K8V4 = 3 };

/* element type of K/V/q inputs */
enum { KV_DTYPE_F16 = 0, KV_DTYPE_F32 = 1 };

enum {
  KV_OK = 0,
  KV_ERR_NULL = -1,        /* a required pointer is NULL                       */
  KV_ERR_SHAPE = -2,       /* inconsistent sizes (negative counts, ...)         */
  KV_ERR_RANGE = -3,       /* positions / context outside the table or pool     */
  KV_ERR_DTYPE = -4,       /* unknown dtype code                                */
  KV_ERR_UNSUPPORTED = -5, /* format / head_dim / GQA / page size not supported */
  KV_ERR_WORKSPACE = -6,   /* workspace missing or too small                    */
  KV_ERR_ALIGN = -7,       /* a device pointer is not 16-byte aligned           */
  KV_ERR_LAUNCH = -8       /* the HIP runtime refused a launch                  */
};

/*
 * A paged cell pool.  Each run is one device allocation indexed
 * [physical page][kv head][slot], P = page_size slots per page, D = 256.
 *
 * k8v4 (fmt 3), 816 bytes per cell for 2 KV heads (408 per head):
 *   run[0] K codes  int8, 256 per head-cell hc = (page*H + g)*P + slot,
 *                   in 4096-byte blocks of 16 head-cells laid out
 *                   [dim quarter][hc % 16][64 codes]: code c of hc at
 *                   (hc/16)*4096 + (c/64)*1024 + (hc%16)*64 + c%64 (so a
 *                   16-byte load per lane of 16 cells x 64 dims reads 1 KB
 *                   of consecutive bytes)
 *   run[1] K scales fp32, element ((page*H + g)*P + slot)*2 + j, one scale
 *                   per 128 dims (j = c / 128)
 *   run[2] V q4_0   one tile of 144*P bytes per (page, head) at
 *                   (page*H + g)*144*P: the 16 nibble bytes of block b
 *                   (dims 32b..32b+31, rotated basis) of a slot at
 *                   slot*128 + b*16 (byte i = element i | element i+16 << 4),
 *                   and the block's fp16 scale after the 128*P nibble
 *                   bytes, grouped by 16 slots:
 *                   128*P + (slot/16)*256 + b*32 + (slot%16)*2.
 *   run[3] unused (may be NULL).
 * Keeping the scales apart from the nibbles (rather than in front of each
 * block) keeps every load 8- or 16-byte aligned, and grouping them by 16
 * slots makes the scales of 16 consecutive cells one 256-byte read;
 * kv_gather returns the conventional 18-byte blocks.
 *
 * The comparison formats of the same pages ("#120", Measured) use the same
 * two kinds of half:
 * int8 (fmt 1), 1056 bytes per cell: run[0]/run[1] K codes/scales laid out
 *   like k8v4's and run[2]/run[3] V codes/scales (V by the K rule,
 *   unrotated): V codes as plain rows, code c of hc at hc*256 + c, V scales
 *   like the K scales.
 * q4_0 (fmt 2), 576 bytes per cell: run[0] K and run[2] V, each a q4_0 tile
 *   run like k8v4's run[2] (both halves rotated); run[1], run[3] unused.
 * fp16 (fmt 0), 2048 bytes per cell, no quantization and no rotation (the
 *   reference without dequantization): run[0] K and run[2] V as fp16 (inputs
 *   rounded to nearest even), 8192 bytes per 16 head-cells each, laid out as
 *   the attention kernel's matrix-core operands; with c = hc % 16:
 *     K element d at (hc/16)*8192 + (d/32)*1024 + ((d%32)/8)*256 + c*16 + (d%8)*2
 *     V element d at (hc/16)*8192 + ((d%16)/2)*1024 + (c/4)*256 + (d/16)*16
 *                    + (d%2)*8 + (c%4)*2
 *   run[1], run[3] unused.  Every any-format entry point takes it.
 */
typedef struct kv_pool {
  int32_t fmt;        /* KV_FMT_*                               */
  int32_t n_pages;    /* physical pages held by each run        */
  int32_t page_size;  /* cells per page, a multiple of 16       */
  int32_t n_kv_heads; /* H                                      */
  int32_t head_dim;   /* D, must be 256                         */
  int32_t reserved;   /* set to 0                               */
  void *run[4];       /* device pointers, 256-byte aligned      */
} kv_pool;

/* One sequence: logical page i of the sequence lives in physical page
 * page_table[i].  Logical cell p is slot p % P of logical page p / P.   */
typedef struct kv_seq {
  const int32_t *page_table; /* device, [n_table] entries in [0, n_pages) */
  int32_t n_table;           /* number of entries                         */
  int32_t reserved;          /* set to 0                                  */
} kv_seq;

/* Bytes per cell for all KV heads: 816 (k8v4), 1056 (int8), 576 (q4_0) at
 * 2 heads x 256 dims ("#120 --kv k8v4: hybrid KV cache", What).  0 when
 * the format or head_dim is not supported. */
size_t kv_cell_bytes(int fmt, int n_kv_heads, int head_dim);

/* Bytes of run `run` (0..3) of a pool; 0 for an unused run. */
size_t kv_run_bytes(int fmt, int run, int n_pages, int page_size, int n_kv_heads, int head_dim);

/*
 * Append n_tokens tokens at logical cells [pos0, pos0 + n_tokens) of a k8v4
 * pool ("#120 --kv k8v4: hybrid KV cache", What and How; Tests: bitwise
 * append through a non-identity page table).
 *   k, v: device, [n_tokens][n_kv_heads][256], fp16 or fp32 (dtype), the
 *         keys after any positional encoding.
 * K per 128-dim group: d = max|x| / 127, code = round-half-even(x * (1/d))
 * clamped to +-127 (d = 0 gives codes 0), stored unrotated with fp32 d.
 * V per head: rotated by the 256-point Walsh-Hadamard transform scaled by
 * 1/16 (butterflies in ascending stride order, fp32), then per 32-block:
 * m = value of largest magnitude (first on ties), d = m / -8,
 * code = min(15, trunc(y * (1/d) + 8.5)), fp16 d (round to nearest even).
 * Errors: KV_ERR_NULL, _UNSUPPORTED (fmt != 3), _DTYPE, _RANGE (pos0 < 0,
 * n_tokens < 0, or pos0 + n_tokens > n_table * page_size).
 * n_tokens == 0 is a no-op returning KV_OK.
 */
int kv_append_k8v4(const kv_pool *pool, const kv_seq *seq, const void *k, const void *v,
                   int dtype, int32_t pos0, int32_t n_tokens, void *stream);

/*
 * The same append for a pool of any of the four formats (fmt 0, 1, 2, 3):
 * each half follows its kind's rule above (int8: K and V by the INT8 rule;
 * q4_0: K and V both rotated and Q4_0-coded; k8v4: as kv_append_k8v4;
 * fp16: K and V rounded to fp16, unrotated).
 * Same arguments and errors as kv_append_k8v4, _UNSUPPORTED for an unknown
 * format.
 */
int kv_append(const kv_pool *pool, const kv_seq *seq, const void *k, const void *v, int dtype,
              int32_t pos0, int32_t n_tokens, void *stream);

/*
 * Copy the stored bytes of cells [pos0, pos0 + n) of a k8v4 pool, in
 * logical order, to contiguous device buffers ("#120 --kv k8v4: hybrid KV
 * cache", Tests: bitwise gather through a non-identity page table):
 *   k_codes  int8  [n][H][256]
 *   k_scales fp32  [n][H][2]
 *   v_blocks uint8 [n][H][8][18]  (fp16 scale little-endian, then 16 bytes)
 * Errors: KV_ERR_NULL, _UNSUPPORTED, _RANGE.
 */
int kv_gather(const kv_pool *pool, const kv_seq *seq, int32_t pos0, int32_t n, void *k_codes,
              void *k_scales, void *v_blocks, void *stream);

/*
 * kv_gather for any format: stored bytes of cells [pos0, pos0 + n) in
 * logical order.  An int8-coded half goes to a codes array int8 [n][H][256]
 * (16-byte aligned) and a scales array fp32 [n][H][2] (8-byte aligned); a
 * q4_0-coded half to one block array uint8 [n][H][8][18].
 *   k8v4: out0 K codes, out1 K scales, out2 V blocks (out3 unused)
 *   int8: out0 K codes, out1 K scales, out2 V codes, out3 V scales
 *   q4_0: out0 K blocks, out2 V blocks (out1, out3 unused)
 *   fp16: out0 K, out2 V, each fp16 [n][H][256], 16-byte aligned (out1,
 *         out3 unused)
 * A table entry outside [0, n_pages) gives 0xff bytes and NaN scales for
 * its cells.  Errors: KV_ERR_NULL (a required output), _ALIGN, _RANGE.
 */
int kv_gather_runs(const kv_pool *pool, const kv_seq *seq, int32_t pos0, int32_t n, void *out0,
                   void *out1, void *out2, void *out3, void *stream);

/*
 * Device workspace needed by attn_decode / attn_decode_append (n_q = 1),
 * attn_verify (n_q queries) and attn_decode_batch (n_q = n_seq) over at
 * most max_ctx cells: the split-K partial results (with room for the fused
 * append's extra partial).  Its contents need no initialization and are
 * overwritten by every call; calls that share a workspace must be ordered
 * on one stream.  0 for an unsupported request.
 */
size_t attn_workspace_bytes(const kv_pool *pool, int n_q_heads, int32_t n_q, int32_t max_ctx);

/* Zero-fill a workspace of ws_bytes bytes with a small fill kernel on
 * `stream` (optional: the attention calls do not need it). */
int kv_workspace_init(void *ws, size_t ws_bytes, void *stream);

/*
 * Copy whole pages between two pools of the same format, KV-head count and
 * page size ("kv: --kv k8v4 streams with --kv-resident", How: a streamed
 * cache keeps all pages in host memory and a window in device memory, and
 * moves a page as its byte runs -- three for k8v4): page src_pages[i] of src
 * becomes page dst_pages[i] of dst, every run of it.  Either pool's runs may
 * be device memory or mapped pinned host memory (hipHostMalloc); the copy is
 * one kernel on `stream`.
 *   dst_pages, src_pages: device int32 [n]; an entry outside its pool's
 *   [0, n_pages) skips that pair.  No page may be both read and written.
 * Errors: KV_ERR_NULL (a run of either pool, or a page list with n > 0),
 * _UNSUPPORTED, _ALIGN, _SHAPE (pools that differ in format or shape),
 * _RANGE (n < 0).  n == 0 is a no-op.
 */
int kv_copy_pages(const kv_pool *dst, const kv_pool *src, const int32_t *dst_pages, const int32_t *src_pages,
                  int32_t n, void *stream);

/* Measurement aid, not part of the method: one plain streaming read of the
 * first bytes / 16 16-byte words of buf (device, 16-byte aligned) with
 * non-temporal loads from 512 workgroups, each streaming its own contiguous
 * share, the yardstick against which the
 * attention kernels' bytes per second are read.  sink: device, 16-byte
 * aligned, 4 KiB, written only in a case a repeated-byte fill cannot produce.
 * Returns KV_ERR_NULL / KV_ERR_ALIGN before launching. */
int kv_probe_read(const void *buf, size_t bytes, void *sink, void *stream);

/*
 * One decode step: the query attends to cells [0, n_ctx)
 * ("#120 --kv k8v4: hybrid KV cache", How: the fused attention gathers the
 * pages, reads K through the INT8 path and V through the rotated q4_0 path,
 * and rotates the output back; q is never rotated).
 *   q:   device, [n_q_heads][256], fp16 or fp32 (q_dtype)
 *   out: device fp32 [n_q_heads][256]; head h uses KV head h / 8.
 *   scale: softmax scale; <= 0 selects 1/sqrt(256).
 * out = H/16 * softmax(scale * q K^T) V_rot, with K = code * d and
 * V_rot = (code - 8) * d16 (fp32 accumulation).
 * The comparison formats run through the same entry: int8 scores q against
 * K = code * d and returns softmax(.) V with V = code * d (no rotation);
 * q4_0 scores (H q / 16) against the rotated K_rot = (code - 8) * d16 and
 * rotates the output back as k8v4 does; fp16 returns softmax(scale q K^T) V
 * over the stored fp16 K and V.
 * Errors: KV_ERR_NULL, _UNSUPPORTED, _DTYPE, _RANGE (n_ctx < 1 or beyond
 * the table), _WORKSPACE.
 */
int attn_decode(const kv_pool *pool, const kv_seq *seq, const void *q, int q_dtype,
                int n_q_heads, int32_t n_ctx, float scale, float *out, void *ws,
                size_t ws_bytes, void *stream);

/* Size of the library's per-device scratch array (attn_decode_noalloc):
 * 4 MiB.  A decode's split-K partials take about 8 KiB per split-K
 * workgroup and the plan launches about one per compute unit, so this holds
 * any decode on a GPU of up to ~500 compute units (MI355X: 256, ~2 MiB). */
#define KV_SCRATCH_BYTES ((size_t)4 << 20)

/*
 * attn_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops that forbid allocation, harnesses that
 * forbid hipMalloc.  Same arguments, result and errors as attn_decode,
 * without the workspace: the split-K partials go to a scratch array of
 * KV_SCRATCH_BYTES that the library keeps in each GPU's memory (one copy per
 * device, held until the process ends, looked up on the first call on a
 * device).  The call allocates and frees nothing.
 *   - All calls on one GPU share that GPU's array, which keeps the last
 *     call's partials (they need no clearing: every call overwrites what it
 *     reads).  Calls that overlap on one GPU (on different streams, or from
 *     different threads without ordering) race on it: order them on one
 *     stream.
 *   - KV_ERR_WORKSPACE (before launching) when the call's split plan needs
 *     more than KV_SCRATCH_BYTES;
 *     KV_ERR_LAUNCH if the runtime cannot resolve the array on the current
 *     device.
 */
int attn_decode_noalloc(const kv_pool *pool, const kv_seq *seq, const void *q, int q_dtype,
                        int n_q_heads, int32_t n_ctx, float scale, float *out, void *stream);

/*
 * One decode step with its append fused in ("#120 --kv k8v4: hybrid KV
 * cache", How: a decode step appends the new token's K/V, then attends over
 * the cache including it).  Equivalent to kv_append_k8v4(pool, seq, k_new,
 * v_new, kv_dtype, pos, 1) followed by attn_decode(..., n_ctx = pos + 1):
 * the cell pos receives exactly the bytes kv_append_k8v4 would write, and
 * the token enters the attention through the same dequantization as a
 * stored cell (its score summed in a different order, so the output agrees
 * with the two-call sequence to rounding, not bitwise).  One launch fewer
 * per step: the last split-K workgroup of each KV head quantizes the token.
 *   k_new, v_new: device, [n_kv_heads][256], fp16 or fp32 (kv_dtype),
 *                 16-byte aligned
 *   q, out, scale, ws: as attn_decode; ws sized for n_ctx = pos + 1.
 *   pos >= 0, within the table (pos = 0 attends to the new token alone).
 * k8v4 pools only (_UNSUPPORTED otherwise).  An out-of-range table entry for
 * cell pos leaves the pool unwritten and gives NaN rows.
 * Errors: KV_ERR_NULL, _UNSUPPORTED, _DTYPE, _ALIGN, _RANGE, _WORKSPACE.
 */
int attn_decode_append(const kv_pool *pool, const kv_seq *seq, const void *k_new, const void *v_new,
                       int kv_dtype, const void *q, int q_dtype, int n_q_heads, int32_t pos, float scale,
                       float *out, void *ws, size_t ws_bytes, void *stream);

/*
 * One decode step for a batch of n_seq independent sequences in one launch
 * sequence (the engine decodes two sequences at once in the RTX 5090 field
 * report of "kv: --kv k8v4 streams with --kv-resident"): sequence i has its own page
 * table seqs[i] into the shared pool and attends its query to its cells
 * [0, n_ctx[i]).  Each sequence's output equals attn_decode on it alone,
 * to rounding (the split plan differs).
 *   seqs:  host array [n_seq] of tables into `pool`;  n_ctx: host [n_seq]
 *   q:     device, [n_seq][n_q_heads][256];  out: device fp32 [n_seq][n_q_heads][256]
 *   ws:    attn_workspace_bytes(pool, n_q_heads, n_seq, max n_ctx) bytes
 *   1 <= n_seq <= 16.  Any format.
 * Errors as attn_decode, plus KV_ERR_SHAPE for n_seq outside [1, 16].
 */
int attn_decode_batch(const kv_pool *pool, const kv_seq *seqs, int32_t n_seq, const void *q, int q_dtype,
                      int n_q_heads, const int32_t *n_ctx, float scale, float *out, void *ws, size_t ws_bytes,
                      void *stream);

/*
 * Verify window of speculative decoding: n_q query rows read the cache
 * once, row i attending to cells [0, n_visible[i]) -- the batched form with
 * a per-query step array ("#120 --kv k8v4: hybrid KV cache", Tests).
 *   q:   device, [n_q][n_q_heads][256];  out: device fp32 [n_q][n_q_heads][256]
 *   n_visible: host, [n_q], each in [1, n_table * page_size]
 *   1 <= n_q <= 16.
 * Errors as attn_decode, plus KV_ERR_SHAPE for n_q outside [1, 16].
 */
int attn_verify(const kv_pool *pool, const kv_seq *seq, const void *q, int q_dtype,
                int n_q_heads, int32_t n_q, const int32_t *n_visible, float scale, float *out,
                void *ws, size_t ws_bytes, void *stream);

/*
 * Causal attention of a chunk of n_new new queries at logical positions
 * [pos0, pos0 + n_new) over the cache, whose cells [0, pos0 + n_new) must
 * already be appended; row i attends to cells [0, pos0 + i]
 * ("#120 --kv k8v4: hybrid KV cache", How: the same fused attention serves
 * prefill).  Dense contractions on the matrix cores (fp16 inputs, fp32
 * accumulation).
 *   q:   device, [n_new][n_q_heads][256];  out: device fp32 [n_new][n_q_heads][256]
 *   ws:  device, attn_prefill_workspace_bytes(pool, pos0 + n_new) bytes,
 *        16-byte aligned; overwritten by the call (no initialisation needed;
 *        calls that share it must be ordered).  Two kernels run: the first
 *        dequantizes every 32-cell tile of each KV head once into ws, the
 *        second computes the attention from there.  An armed timing pair
 *        (kv_time_next_launch) brackets both.
 * Any of the four formats, with the same rules as attn_decode (q4_0 scores
 * the rotated query against rotated keys; int8 and fp16 return
 * softmax(.) V unrotated).  A page-table entry outside [0, n_pages) makes
 * the rows whose window reaches its cells NaN (the reads stay in the pool).
 * Errors: KV_ERR_NULL, _UNSUPPORTED, _DTYPE, _RANGE, _ALIGN, _WORKSPACE
 * (ws NULL or smaller than attn_prefill_workspace_bytes).
 */
int attn_prefill_chunk(const kv_pool *pool, const kv_seq *seq, const void *q, int q_dtype,
                       int n_q_heads, int32_t pos0, int32_t n_new, float scale, float *out,
                       void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes of attn_prefill_chunk over n_cells = pos0 + n_new cells:
 * n_kv_heads * ceil(n_cells / 32) tile images of 32,768 bytes (fp16 K,
 * scaled, and fp16 V of 32 cells, in 16-byte chunks).
 * 0 for a NULL pool or n_cells < 1. */
size_t attn_prefill_workspace_bytes(const kv_pool *pool, int32_t n_cells);

/*
 * A streamed cache ("kv: --kv k8v4 streams with --kv-resident", What and
 * How; "#1188 --kv k8v4 produces degenerate repetition when --kv-resident
 * streams", the engine log: a window of cells per layer in device memory,
 * the whole K/V in pinned host memory).  Two pools of one format, KV-head
 * count and page size hold the same logical pages:
 *   mirror: every page of the context, in mapped pinned host memory
 *           (hipHostMalloc); logical page i is mirror page mirror_table[i];
 *   window: a device pool of fewer pages; logical page i is resident in
 *           window slot window_map[i], or not resident when that is -1.
 * window_owner[s] is the logical page in window slot s (-1: free).  The two
 * maps are the caller's memory and state, written only by kv_stream_fetch
 * (set them to -1 before first use).  stats accumulates [lookups, misses]
 * of the streamed attention calls; fetch_list is scratch of
 * 2 * window.n_pages int32 for kv_stream_fetch.  All device pointers.
 */
typedef struct kv_stream {
  kv_pool window;
  kv_pool mirror;
  const int32_t *mirror_table; /* device [n_table]: logical page -> mirror page       */
  int32_t *window_map;         /* device [n_table]: logical page -> window slot or -1  */
  int32_t *window_owner;       /* device [window.n_pages]: slot -> logical page or -1  */
  int32_t *stats;              /* device [2]: lookups, misses (accumulated)            */
  int32_t *fetch_list;         /* device [2 * window.n_pages]: kv_stream_fetch scratch  */
  int32_t n_table;             /* logical pages of the sequence                        */
  int32_t reserved;            /* set to 0                                             */
} kv_stream;

/*
 * Append n_tokens tokens at logical cells [pos0, pos0 + n_tokens) of a
 * streamed cache: one kernel quantizes each token once (the format's rules,
 * as kv_append) and writes every run of the cell to the mirror, and also to
 * the window when the cell's page is resident.  Both copies of a cell are
 * the same bytes.  Every run of both pools is required: a NULL run is
 * KV_ERR_NULL, never a skipped copy -- the pages' bug was a writer that
 * tested one half's pointer for presence and silently left out the host
 * write of the other.
 * Errors: as kv_append, plus KV_ERR_SHAPE (the pools differ in format,
 * heads or page size).
 */
int kv_stream_append(const kv_stream *s, const void *k, const void *v, int dtype, int32_t pos0,
                     int32_t n_tokens, void *stream);

/*
 * Miss service: make logical pages [first_page, first_page + n_pages)
 * resident, as many as fit, the last ones first: page i goes to window slot
 * i % window.n_pages (a ring over the window), whose previous page becomes
 * non-resident; a page already in its slot is not copied; the others are
 * copied from the mirror, every run (one kernel, as kv_copy_pages).  With
 * n_pages > window.n_pages only the last window.n_pages pages are brought
 * in.  Errors: KV_ERR_NULL, _SHAPE, _RANGE (pages outside [0, n_table)).
 */
int kv_stream_fetch(const kv_stream *s, int32_t first_page, int32_t n_pages, void *stream);

/*
 * attn_decode and attn_verify over a streamed cache: each 16-cell half of a
 * page is read from the window when its page is resident and from the
 * mirror otherwise (across the host link, inside the kernel), so the result
 * is bitwise the result over a resident pool holding the same bytes (the
 * split plan depends only on the context length).  Each call first counts,
 * on the device, one lookup per logical page it reads and one miss per page
 * not resident, into s->stats.  Same arguments, results and errors as
 * attn_decode / attn_verify; ws as attn_workspace_bytes for the window
 * pool.
 */
int attn_decode_stream(const kv_stream *s, const void *q, int q_dtype, int n_q_heads, int32_t n_ctx,
                       float scale, float *out, void *ws, size_t ws_bytes, void *stream);
int attn_verify_stream(const kv_stream *s, const void *q, int q_dtype, int n_q_heads, int32_t n_q,
                       const int32_t *n_visible, float scale, float *out, void *ws, size_t ws_bytes,
                       void *stream);

/*
 * Debug check of a page table (synchronous: copies the table to the host).
 * Counts entries of the first ceil(n_cells / page_size) that are out of
 * [0, n_pages) or repeated; writes the count to *n_bad.
 * Errors: KV_ERR_NULL, _RANGE, _LAUNCH (copy failed).
 */
int kv_check_page_table(const kv_pool *pool, const kv_seq *seq, int32_t n_cells, int32_t *n_bad);

/* Static description of an error code. */
const char *kv_strerror(int code);

/* Name and description of the HIP error behind the calling thread's most
 * recent KV_ERR_LAUNCH ("no error" if there was none). */
const char *kv_last_hip_error(void);

/*
 * Measurement aid, not part of the method.  Profiling hook: the calling
 * thread's next kernel launch by this library records start_event when the
 * kernel starts and stop_event when it ends (hipExtLaunchKernelGGL), so
 * hipEventElapsedTime gives that one kernel's duration.  Both are hipEvent_t
 * created by the caller on the device of the launch.  What it brackets, per
 * entry point: attn_decode, attn_decode_append, attn_decode_batch,
 * attn_verify and attn_decode_noalloc launch the split kernel and then a
 * small combine kernel, so the hook times the split kernel;
 * attn_decode_stream and attn_verify_stream launch a page-lookup kernel
 * first, which is what the hook times; attn_prefill_chunk's two kernels are
 * bracketed together (start of the staging kernel to the end of the
 * attention kernel); every other entry point launches one kernel.  The hook
 * applies to the next entry-point call only: a call that returns before
 * launching (an error, empty work) disarms it.  Errors: KV_ERR_NULL.
 */
int kv_time_next_launch(void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* K8V4_H */
