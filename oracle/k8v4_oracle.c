/*
 * k8v4_oracle.c -- plain, slow, obviously-correct CPU oracle for the hybrid
 * "k8v4" KV cache (INT8 K + Walsh-Hadamard-rotated Q4_0 V) and the attention
 * that reads it, plus the int8 and q4_0 comparison formats and an unquantized
 * fp16 format (K and V rounded to fp16, the reference without dequantization;
 * "#729 KV int8 vs fp16 KLD compare at 240K context" uses fp16 KV as its
 * baseline).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or constant generator with the HIP path
 * (long_context_decode_append_amd/csrc); neither side includes the other.
 *
 * Sources (the pages; cited by title and section):
 *   [PR120] "#120 --kv k8v4: hybrid KV cache -- INT8 K + Hadamard-rotated
 *           Q4_0 V (816 B/cell)", sections What / How / Tests.
 *   [PR711] "kv: --kv k8v4 streams with --kv-resident", section How
 *           (a k8v4 block is three byte runs: K codes, K scales, V q4_0).
 *
 * Arithmetic rules (each is a reading of the pages, see the readings list
 * in the design notes of the repository):
 *   - quantizers run in IEEE fp32 with every operation rounded as written
 *     (build with -ffp-contract=off, no fast-math);
 *   - fp16 conversion is this file's own round-to-nearest-even routine,
 *     subnormals included;
 *   - attention is fp64 and written as its plain definition (scores, max,
 *     exponentials, weighted average, then the explicit Hadamard matrix).
 *
 * Parity pins: every function here is pinned by a -m "not gpu" test in
 * tests/test_oracle_*.py against something other than itself (numpy's
 * float16 rounding, scipy's Sylvester Hadamard matrix, crafted values,
 * brute force, closed forms, the byte counts the pages print).  The
 * quantizer conventions that the pages leave open (K scale group of 128 with
 * an fp32 scale, Q4_0 rounding, tie and zero rules, nibble order, FWHT
 * stage order) are "parity unpinned" against the pages' own engine: the
 * pages carry no code or test vectors for them.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_D 256          /* head_dim: the only one the pages use        */
#define ORC_KGROUP 128     /* INT8 K scale group (two scales per head)    */
#define ORC_QBLK 32        /* Q4_0 block length                           */
#define ORC_QBYTES 18      /* Q4_0 block: fp16 scale + 16 nibble bytes    */

/* ------------------------------------------------------------------ */
/* fp16 <-> fp32, written from the IEEE 754 binary16 definition.       */
/* ------------------------------------------------------------------ */

uint16_t orc_f32_to_f16(float f) {
  uint32_t bits;
  memcpy(&bits, &f, 4);
  uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
  if (isnan(f)) return (uint16_t)(sign | 0x7e00u);
  double a = fabs((double)f); /* exact */
  if (isinf(f) || a >= 65520.0) return (uint16_t)(sign | 0x7c00u);
  if (a < 6.103515625e-05) { /* below 2^-14: subnormal range, step 2^-24 */
    double q = nearbyint(a * 16777216.0); /* exact scale, RNE */
    return (uint16_t)(sign | (uint16_t)q); /* q == 1024 is the min normal */
  }
  int e;
  (void)frexp(a, &e);         /* a = m * 2^e, m in [0.5, 1) */
  int E = e - 1;              /* a in [2^E, 2^(E+1)) */
  double q = nearbyint(ldexp(a, 10 - E)); /* in [1024, 2048], RNE */
  if (q >= 2048.0) { q = 1024.0; E += 1; }
  if (E + 15 >= 31) return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024.0));
}

float orc_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return (float)(sign ? -v : v);
}

/* inputs arrive as fp16 bit patterns (dtype 0) or fp32 (dtype 1) */
static float load_in(const void *p, int dtype, size_t i) {
  if (dtype == 0) return orc_f16_to_f32(((const uint16_t *)p)[i]);
  return ((const float *)p)[i];
}

/* ------------------------------------------------------------------ */
/* INT8 K rule [PR120, What + Tests: K stays INT8, unrotated, ties to  */
/* even].  Per group of 128 values: d = max|x| / 127, r = 1/d (0 when  */
/* d is 0), code = clamp(round_half_even(x * r), -127, 127).           */
/* ------------------------------------------------------------------ */

void orc_quant_int8_group(const float *x, int n, int8_t *codes, float *d_out) {
  float amax = 0.0f;
  for (int i = 0; i < n; i++) {
    float ax = fabsf(x[i]);
    if (ax > amax) amax = ax;
  }
  float d = amax / 127.0f;
  float r = (d != 0.0f) ? 1.0f / d : 0.0f;
  for (int i = 0; i < n; i++) {
    float t = x[i] * r;
    float q = nearbyintf(t); /* default rounding mode: nearest, ties even */
    if (q > 127.0f) q = 127.0f;
    if (q < -127.0f) q = -127.0f;
    codes[i] = (int8_t)q;
  }
  *d_out = d;
}

/* ------------------------------------------------------------------ */
/* Walsh-Hadamard rotation [PR120, What + How: V and the attention     */
/* output are rotated, q and K are not].  Sylvester (natural) order    */
/* over the full 256-wide head, butterflies (a+b, a-b) with strides    */
/* 1, 2, 4, ... 128 in ascending order, then times 1/16 so the map is  */
/* orthonormal.  Each butterfly output is one fp32 add or subtract.    */
/* ------------------------------------------------------------------ */

void orc_fwht256(float *y) {
  for (int s = 1; s < ORC_D; s <<= 1) {
    for (int c = 0; c < ORC_D; c++) {
      if (c & s) continue;
      float a = y[c], b = y[c + s];
      y[c] = a + b;
      y[c + s] = a - b;
    }
  }
  for (int c = 0; c < ORC_D; c++) y[c] = y[c] * 0.0625f;
}

/* ------------------------------------------------------------------ */
/* Q4_0 rule for one 32-value block [PR120, What: rotated q4_0].       */
/* m = the value of largest magnitude (first such index), d = m / -8,  */
/* r = 1/d (0 when d is 0), code = min(15, trunc(x * r + 8.5)); the    */
/* block is stored as fp16(d) little-endian followed by 16 bytes,      */
/* byte i = code[i] | code[i+16] << 4.                                 */
/* ------------------------------------------------------------------ */

void orc_quant_q4_block(const float *y, uint8_t *out) {
  int best = 0;
  float bmag = fabsf(y[0]);
  for (int i = 1; i < ORC_QBLK; i++) {
    float a = fabsf(y[i]);
    if (a > bmag) { bmag = a; best = i; }
  }
  float m = y[best];
  float d = m / -8.0f;
  float r = (d != 0.0f) ? 1.0f / d : 0.0f;
  uint8_t code[ORC_QBLK];
  for (int i = 0; i < ORC_QBLK; i++) {
    float t = y[i] * r;
    float u = t + 8.5f;
    int c = (int)u; /* truncation toward zero; u is never negative here */
    if (c > 15) c = 15;
    code[i] = (uint8_t)c;
  }
  uint16_t h = orc_f32_to_f16(d);
  out[0] = (uint8_t)(h & 0xff);
  out[1] = (uint8_t)(h >> 8);
  for (int i = 0; i < 16; i++) out[2 + i] = (uint8_t)(code[i] | (code[i + 16] << 4));
}

/* dequantized value of element i of a canonical 18-byte block */
static double q4_value(const uint8_t *blk, int i) {
  uint16_t h = (uint16_t)(blk[0] | (blk[1] << 8));
  int byte = blk[2 + (i & 15)];
  int code = (i < 16) ? (byte & 15) : (byte >> 4);
  return (double)(code - 8) * (double)orc_f16_to_f32(h);
}

/* ------------------------------------------------------------------ */
/* Sizes [PR120, What: 816 B per cell against 1,056 for int8 and 576   */
/* for q4_0; Measured: V costs 144 against 256 B per head per cell].   */
/* ------------------------------------------------------------------ */

static long k_int8_head_bytes(int D) { return D + 4L * (D / ORC_KGROUP); }
static long q4_head_bytes(int D) { return (D / ORC_QBLK) * (long)ORC_QBYTES; }

long orc_cell_bytes(int fmt, int n_kv_heads, int D) {
  if (D % ORC_KGROUP) return -1;
  switch (fmt) {
    case 0: return (long)n_kv_heads * 2 * 2L * D;
    case 1: return (long)n_kv_heads * 2 * k_int8_head_bytes(D);
    case 2: return (long)n_kv_heads * 2 * q4_head_bytes(D);
    case 3: return (long)n_kv_heads * (k_int8_head_bytes(D) + q4_head_bytes(D));
    default: return -1;
  }
}

/* ------------------------------------------------------------------ */
/* Pool placement [PR711, How: a k8v4 block is three byte runs -- K    */
/* codes, K scales, V q4_0 -- moved as whole pages].  The pages fix    */
/* the runs and the bytes per cell, not the order of bytes inside a    */
/* page; this image takes the plain order.  Every run is indexed       */
/* [physical page][kv head][slot], and a head-cell                     */
/* hc = (page * H + head) * P + slot holds, in each run, one record:   */
/*   INT8 codes:   256 int8, code c at byte hc * 256 + c               */
/*   INT8 scales:  two fp32 (dims 0..127, 128..255) at hc * 8          */
/*   Q4_0 blocks:  8 conventional 18-byte blocks (fp16 scale, then 16  */
/*                 nibble bytes) at hc * 144 + b * 18                  */
/*   fp16 values:  256 fp16 (little-endian) at hc * 512 + 2 d          */
/* A logical cell p lives in physical page pt[p / P] at slot p % P.    */
/* Run use per format: k8v4 = K codes, K scales, V blocks; int8 = K    */
/* codes, K scales, V codes, V scales; q4_0 = K blocks, -, V blocks;   */
/* fp16 = K values, -, V values.  (A library may order the bytes       */
/* inside a page differently; its tests map its image onto this one.)  */
/* ------------------------------------------------------------------ */

#define ORC_NSC (ORC_D / ORC_KGROUP)                 /* scales per head   */
#define ORC_QHEAD ((ORC_D / ORC_QBLK) * ORC_QBYTES)  /* 144 B per head    */

static size_t head_cell(int page, int g, int H, int P, int slot) {
  return ((size_t)page * H + g) * P + slot;
}

static void put_int8_head(uint8_t *codes_run, uint8_t *scales_run, size_t hc, const int8_t *codes,
                          const float *scales) {
  memcpy(codes_run + hc * ORC_D, codes, ORC_D);
  memcpy(scales_run + hc * ORC_NSC * 4, scales, ORC_NSC * 4);
}

static void get_int8_head(const uint8_t *codes_run, const uint8_t *scales_run, size_t hc, uint8_t *codes,
                          uint8_t *scales) {
  memcpy(codes, codes_run + hc * ORC_D, ORC_D);
  memcpy(scales, scales_run + hc * ORC_NSC * 4, ORC_NSC * 4);
}

/* one head of the fp16 format: each value rounded to fp16 (RNE) */
static void put_f16_head(uint8_t *run, size_t hc, const float *x) {
  for (int d = 0; d < ORC_D; d++) {
    const uint16_t h = orc_f32_to_f16(x[d]);
    run[hc * 2 * ORC_D + 2 * d] = (uint8_t)(h & 0xff);
    run[hc * 2 * ORC_D + 2 * d + 1] = (uint8_t)(h >> 8);
  }
}

/* quantize one head's K (int8 rule) */
static void quant_k_int8(const float *x, int8_t *codes, float *scales) {
  for (int j = 0; j < ORC_D / ORC_KGROUP; j++)
    orc_quant_int8_group(x + j * ORC_KGROUP, ORC_KGROUP, codes + j * ORC_KGROUP, scales + j);
}

/* rotate then Q4_0-quantize one head */
static void quant_rot_q4(const float *x, uint8_t *blocks) {
  float y[ORC_D];
  memcpy(y, x, sizeof y);
  orc_fwht256(y);
  for (int b = 0; b < ORC_D / ORC_QBLK; b++) orc_quant_q4_block(y + b * ORC_QBLK, blocks + b * ORC_QBYTES);
}

/*
 * Append n tokens at logical positions [pos0, pos0+n) [PR120, How: the
 * append entry points take separate K and V pointers; Tests: bitwise
 * append through a non-identity page table].  k, v: [n][H][256] as fp16
 * bits (dtype 0) or fp32 (dtype 1).  Returns 0, or -1 on a bad argument.
 */
int orc_append(int fmt, int n_pages, int P, int H, uint8_t *run0, uint8_t *run1, uint8_t *run2,
               uint8_t *run3, const int32_t *pt, int n_table, const void *k, const void *v,
               int dtype, int pos0, int n) {
  if (P <= 0 || pos0 < 0 || n < 0 || (long)pos0 + n > (long)n_table * P) return -1;
  float kx[ORC_D], vx[ORC_D];
  int8_t codes[ORC_D];
  float scales[ORC_D / ORC_KGROUP];
  for (int t = 0; t < n; t++) {
    int p = pos0 + t;
    int page = pt[p / P], slot = p % P;
    if (page < 0 || page >= n_pages) return -1;
    for (int g = 0; g < H; g++) {
      size_t base = ((size_t)t * H + g) * ORC_D;
      for (int c = 0; c < ORC_D; c++) {
        kx[c] = load_in(k, dtype, base + c);
        vx[c] = load_in(v, dtype, base + c);
      }
      const size_t hc = head_cell(page, g, H, P, slot);
      if (fmt == 0) {
        put_f16_head(run0, hc, kx);
        put_f16_head(run2, hc, vx);
      } else if (fmt == 3) {
        quant_k_int8(kx, codes, scales);
        put_int8_head(run0, run1, hc, codes, scales);
        quant_rot_q4(vx, run2 + hc * ORC_QHEAD);
      } else if (fmt == 1) {
        quant_k_int8(kx, codes, scales);
        put_int8_head(run0, run1, hc, codes, scales);
        quant_k_int8(vx, codes, scales);
        put_int8_head(run2, run3, hc, codes, scales);
      } else if (fmt == 2) {
        quant_rot_q4(kx, run0 + hc * ORC_QHEAD);
        quant_rot_q4(vx, run2 + hc * ORC_QHEAD);
      } else {
        return -1;
      }
    }
  }
  return 0;
}

/*
 * Gather cells [pos0, pos0+n) in logical order into canonical arrays
 * [PR120, Tests: bitwise gather through a non-identity page table]:
 *   int8-coded half:  codes [n][H][256] int8, scales [n][H][2] fp32
 *   q4_0-coded half:  blocks [n][H][8][18] (fp16 scale then 16 bytes)
 * k8v4: out0 = K codes, out1 = K scales, out2 = V blocks.
 * int8: out0..out3 = K codes, K scales, V codes, V scales.
 * q4_0: out0 = K blocks, out2 = V blocks.
 * fp16: out0 = K, out2 = V, each [n][H][256] fp16 bits.
 */
int orc_gather(int fmt, int n_pages, int P, int H, const uint8_t *run0, const uint8_t *run1,
               const uint8_t *run2, const uint8_t *run3, const int32_t *pt, int n_table,
               int pos0, int n, uint8_t *out0, uint8_t *out1, uint8_t *out2, uint8_t *out3) {
  if (P <= 0 || pos0 < 0 || n < 0 || (long)pos0 + n > (long)n_table * P) return -1;
  for (int t = 0; t < n; t++) {
    int p = pos0 + t;
    int page = pt[p / P], slot = p % P;
    if (page < 0 || page >= n_pages) return -1;
    for (int g = 0; g < H; g++) {
      const size_t hc = head_cell(page, g, H, P, slot);
      const size_t o = (size_t)t * H + g;
      if (fmt == 0) {
        memcpy(out0 + o * 2 * ORC_D, run0 + hc * 2 * ORC_D, 2 * ORC_D);
        memcpy(out2 + o * 2 * ORC_D, run2 + hc * 2 * ORC_D, 2 * ORC_D);
        continue;
      }
      if (fmt == 1 || fmt == 3) get_int8_head(run0, run1, hc, out0 + o * ORC_D, out1 + o * ORC_NSC * 4);
      else memcpy(out0 + o * ORC_QHEAD, run0 + hc * ORC_QHEAD, ORC_QHEAD);
      if (fmt == 1) get_int8_head(run2, run3, hc, out2 + o * ORC_D, out3 + o * ORC_NSC * 4);
      else memcpy(out2 + o * ORC_QHEAD, run2 + hc * ORC_QHEAD, ORC_QHEAD);
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Dequantization of gathered cells into fp64 [n][H][256].             */
/* int8 half: code * scale of its 128-group.  q4_0 half: (code - 8) *  */
/* fp16 scale, still in the rotated basis.                             */
/* ------------------------------------------------------------------ */

void orc_dequant_int8(const int8_t *codes, const float *scales, long n_heads_total, double *out) {
  for (long o = 0; o < n_heads_total; o++)
    for (int c = 0; c < ORC_D; c++)
      out[o * ORC_D + c] = (double)codes[o * ORC_D + c] * (double)scales[o * 2 + c / ORC_KGROUP];
}

void orc_dequant_q4(const uint8_t *blocks, long n_heads_total, double *out) {
  const size_t qb = (ORC_D / ORC_QBLK) * ORC_QBYTES;
  for (long o = 0; o < n_heads_total; o++)
    for (int c = 0; c < ORC_D; c++)
      out[o * ORC_D + c] = q4_value(blocks + o * qb + (c / ORC_QBLK) * ORC_QBYTES, c % ORC_QBLK);
}

/* Sylvester Hadamard entry: (-1)^popcount(a & b) */
static double hentry(int a, int b) { return (__builtin_popcount((unsigned)(a & b)) & 1) ? -1.0 : 1.0; }

/* out = (1/16) * H * in, as the explicit matrix-vector product */
void orc_hadamard_apply_f64(const double *in, double *out) {
  for (int a = 0; a < ORC_D; a++) {
    double s = 0.0;
    for (int b = 0; b < ORC_D; b++) s += hentry(a, b) * in[b];
    out[a] = s / 16.0;
  }
}

typedef struct {
  const double *kd, *vd;
  int n_cells, H;
  const void *q;
  int q_dtype, rows, Hq;
  const int32_t *n_vis;
  double scale;
  int q_rotate, v_rotated;
  double *out;
} attn_job;

/* one (row, query head) pair of orc_attention; s: n_cells doubles of scratch */
static void attend_one(const attn_job *J, int r, int h, double *s) {
  const int G = J->Hq / J->H, g = h / G, n = J->n_vis[r];
  double qv[ORC_D], qr[ORC_D], u[ORC_D];
  size_t qoff = ((size_t)r * J->Hq + h) * ORC_D;
  for (int c = 0; c < ORC_D; c++) qv[c] = (double)load_in(J->q, J->q_dtype, qoff + c);
  const double *qq = qv;
  if (J->q_rotate) { orc_hadamard_apply_f64(qv, qr); qq = qr; }
  double smax = -INFINITY;
  for (int t = 0; t < n; t++) {
    const double *kt = J->kd + ((size_t)t * J->H + g) * ORC_D;
    double acc = 0.0;
    for (int c = 0; c < ORC_D; c++) acc += qq[c] * kt[c];
    s[t] = J->scale * acc;
    if (s[t] > smax) smax = s[t];
  }
  double wsum = 0.0;
  for (int c = 0; c < ORC_D; c++) u[c] = 0.0;
  for (int t = 0; t < n; t++) {
    double w = exp(s[t] - smax);
    wsum += w;
    const double *vt = J->vd + ((size_t)t * J->H + g) * ORC_D;
    for (int c = 0; c < ORC_D; c++) u[c] += w * vt[c];
  }
  for (int c = 0; c < ORC_D; c++) u[c] /= wsum;
  double *o = J->out + ((size_t)r * J->Hq + h) * ORC_D;
  if (J->v_rotated) orc_hadamard_apply_f64(u, o);
  else memcpy(o, u, sizeof u);
}

typedef struct {
  const attn_job *J;
  int first, stride;  /* this worker's (row, head) pairs: first, first + stride, ... */
  int rc;
} attn_worker;

static void *attn_worker_run(void *arg) {
  attn_worker *w = (attn_worker *)arg;
  const attn_job *J = w->J;
  double *s = (double *)malloc(sizeof(double) * (J->n_cells > 0 ? J->n_cells : 1));
  if (!s) { w->rc = -1; return NULL; }
  for (long i = w->first; i < (long)J->rows * J->Hq; i += w->stride) attend_one(J, (int)(i / J->Hq), (int)(i % J->Hq), s);
  free(s);
  w->rc = 0;
  return NULL;
}

/*
 * Exact fp64 attention over dequantized K/V, by definition [PR120, How:
 * the fused decode/prefill/verify attention; Tests: step and batched
 * forms, the batched one with a per-query step array].
 *
 *   kd: [n_cells][H][256] fp64 keys in the basis q lives in.
 *   vd: [n_cells][H][256] fp64 values (rotated basis when v_rotated).
 *   q:  [rows][Hq][256] fp16 bits or fp32 (q_dtype), never rotated here;
 *       when q_rotate is set (q4_0 format: K is stored rotated) the scores
 *       use (1/16) H q instead of q.
 *   n_vis: [rows] number of leading cells row r attends to (>= 1).
 *   out: [rows][Hq][256] fp64.  Row r, head h uses kv head h / (Hq / H).
 *   For row r, head h: s_t = scale * <q, k_t>, w_t = exp(s_t - max s),
 *   u = sum w_t v_t / sum w_t, and out = (1/16) H u when v_rotated.
 * The (row, head) pairs are independent; n_threads > 1 hands them out
 * round robin to that many threads, each computing its pairs exactly as
 * one thread would (the result is bitwise the same).
 */
int orc_attention_threads(const double *kd, const double *vd, int n_cells, int H, const void *q,
                          int q_dtype, int rows, int Hq, const int32_t *n_vis, double scale,
                          int q_rotate, int v_rotated, double *out, int n_threads) {
  if (H <= 0 || Hq % H) return -1;
  for (int r = 0; r < rows; r++)
    if (n_vis[r] < 1 || n_vis[r] > n_cells) return -1;
  attn_job J = {kd, vd, n_cells, H, q, q_dtype, rows, Hq, n_vis, scale, q_rotate, v_rotated, out};
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  attn_worker w[256];
  pthread_t tid[256];
  int started = 0, rc = 0;
  for (int i = 0; i < n_threads; i++) {
    w[i].J = &J;
    w[i].first = i;
    w[i].stride = n_threads;
    w[i].rc = -1;
  }
  for (int i = 1; i < n_threads; i++) {
    if (pthread_create(&tid[i], NULL, attn_worker_run, &w[i]) != 0) break;
    started = i;
  }
  if (started < n_threads - 1) {
    /* could not start them all: the calling thread does every pair itself */
    for (int i = 1; i <= started; i++) pthread_join(tid[i], NULL);
    w[0].stride = 1;
    attn_worker_run(&w[0]);
    return w[0].rc;
  }
  attn_worker_run(&w[0]);
  for (int i = 1; i < n_threads; i++) pthread_join(tid[i], NULL);
  for (int i = 0; i < n_threads; i++) rc |= w[i].rc;
  return rc ? -1 : 0;
}

int orc_attention(const double *kd, const double *vd, int n_cells, int H, const void *q,
                  int q_dtype, int rows, int Hq, const int32_t *n_vis, double scale,
                  int q_rotate, int v_rotated, double *out) {
  return orc_attention_threads(kd, vd, n_cells, H, q, q_dtype, rows, Hq, n_vis, scale, q_rotate, v_rotated,
                               out, 1);
}

/* ------------------------------------------------------------------ */
/* Array helpers for the ctypes wrapper (loops over the rules above).  */
/* ------------------------------------------------------------------ */

void orc_f32_to_f16_array(const float *in, uint16_t *out, long n) {
  for (long i = 0; i < n; i++) out[i] = orc_f32_to_f16(in[i]);
}

void orc_f16_to_f32_array(const uint16_t *in, float *out, long n) {
  for (long i = 0; i < n; i++) out[i] = orc_f16_to_f32(in[i]);
}

void orc_fwht256_rows(float *y, long rows) {
  for (long r = 0; r < rows; r++) orc_fwht256(y + r * ORC_D);
}

void orc_quant_int8_groups(const float *x, long n_groups, int8_t *codes, float *d) {
  for (long i = 0; i < n_groups; i++)
    orc_quant_int8_group(x + i * ORC_KGROUP, ORC_KGROUP, codes + i * ORC_KGROUP, d + i);
}

void orc_quant_q4_blocks(const float *y, long n_blocks, uint8_t *out) {
  for (long i = 0; i < n_blocks; i++) orc_quant_q4_block(y + i * ORC_QBLK, out + i * ORC_QBYTES);
}
