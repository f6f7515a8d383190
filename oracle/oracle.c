/*
 * oracle.c -- plain, slow CPU definition of the zero-copy MoE
 * dispatch -> expert -> combine path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library under combine_symmetric_memory_amd/) never calls it and
 * shares no code, header or constant with it.
 *
 * Sources (cited by page title and section):
 *   [blog]  "MORI CCO: Next-Generation Collective Communication Object for
 *           GPUs" (AMD technical article), sections "What is MORI CCO?"
 *           (slot address arithmetic) and "Zero-copy MoE dispatch -> expert
 *           -> combine" (the dataflow: dispatch lands rows in the receive
 *           region, the expert reads it and writes the combine staging
 *           region row for row, combine gathers and weights).
 *   The pages do not define routing order, the expert function or the
 *   combine arithmetic.  The readings taken here are:
 *     - expert e lives in slot e / (E/S) (contiguous blocks of experts);
 *     - inside a slot, rows are grouped by ascending expert id, and inside
 *       an expert by the flat index t*K + j (a stable counting sort);
 *     - one row per (token, k) pair, duplicates included;
 *     - the expert is a SwiGLU MLP, h = silu(x Wg^T) * (x Wu^T) stored as
 *       bf16, y = h Wd^T stored as bf16;
 *     - combine is out[t] = bf16( sum_j w[t][j] * y_j ) accumulated in fp32
 *       with one fused multiply-add per j in j = 0..K-1 order;
 *     - after an 8-bit dispatch the expert reads each value as
 *       bf16( binary32( e4m3(q) * scale ) ), the scale of the value's block
 *       of H / ns (orc_dequant_e4m3_rows).
 *
 * Precision: the GEMM-like sums are accumulated in double; h and y are
 * rounded to bf16 (round to nearest even) because the path stores them in
 * bf16.  Combine uses fp32 fma because the path fixes fp32 accumulation in
 * fixed k order.
 *
 * Parity pins (tests/test_oracle_pins.py) check every function here against
 * brute force, library routines (numpy stable argsort, bincount, float64
 * matmul, torch bf16 and float8_e4m3fn conversions), exact rationals and
 * closed forms.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* status codes returned by orc_plan */
#define ORC_OK 0
#define ORC_BAD_EXPERT 1
#define ORC_CAPACITY 2

/* ---------------------------------------------------------------- bf16 --- */

/* bf16 is the top 16 bits of an IEEE binary32. */
static float orc_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round a binary32 to the nearest bf16, ties to even.  NaN stays a quiet NaN. */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) /* NaN */
    return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t upper = u >> 16;
  uint32_t lower = u & 0xffffu;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

/* Round a binary64 straight to the nearest bf16, ties to even (no double
 * rounding through binary32: a binary32 tie is resolved by the sign of the
 * part that the binary32 conversion dropped). */
uint16_t orc_f64_to_bf16(double d) {
  if (isnan(d)) return (uint16_t)0x7fc0u;
  float f = (float)d; /* nearest binary32 */
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0xffffu) == 0x8000u && (double)f != d) {
    /* f sits exactly half-way between two bf16 values but d does not:
     * round toward the side d lies on. */
    uint32_t upper = u >> 16;
    double rest = d - (double)f; /* exact in binary64 */
    int away = (rest > 0.0) == (f > 0.0f || (f == 0.0f && d > 0.0));
    if (away) upper += 1u;
    return (uint16_t)upper;
  }
  return orc_f32_to_bf16(f);
}

/* ---------------------------------------------------------------- plan --- */

/*
 * Routing plan ([blog] "Zero-copy MoE dispatch": dispatch returns a receive
 * count per rank and a routing object that combine reuses).
 *
 * idx[T][K]   expert id chosen by token t in column j
 * counts[E]   rows routed to each expert
 * expert_off[E]  first row of expert e inside its slot (slot-local)
 * slot_total[S]  rows received by each slot (the per-rank receive count)
 * pos[T][K]   row inside slot(idx[t][j]) that receives the pair (t, j), or
 *             -1 when that row would be at or past cap (the pair is dropped:
 *             a slot holds cap rows, and the status says it overflowed)
 *
 * Returns ORC_BAD_EXPERT if an id is outside [0, E) (outputs then undefined),
 * ORC_CAPACITY if a slot would receive more than cap rows.
 */
int orc_plan(const int32_t *idx, int64_t T, int32_t K, int32_t E, int32_t S,
             int64_t cap, int32_t *counts, int32_t *expert_off,
             int32_t *slot_total, int32_t *pos) {
  int64_t n = T * (int64_t)K;
  int32_t eps = E / S; /* experts per slot */
  int64_t f;
  int32_t e, s;

  /* 1. every id must name an expert */
  for (f = 0; f < n; ++f)
    if (idx[f] < 0 || idx[f] >= E) return ORC_BAD_EXPERT;

  /* 2. count rows per expert, then per slot */
  for (e = 0; e < E; ++e) counts[e] = 0;
  for (f = 0; f < n; ++f) counts[idx[f]] += 1;
  for (s = 0; s < S; ++s) slot_total[s] = 0;
  for (e = 0; e < E; ++e) slot_total[e / eps] += counts[e];

  /* 3. slot-local offsets: experts of a slot are laid out in id order */
  for (s = 0; s < S; ++s) {
    int32_t run = 0;
    for (e = s * eps; e < (s + 1) * eps; ++e) {
      expert_off[e] = run;
      run += counts[e];
    }
  }

  /* 4. positions: walk the pairs in flat (t, j) order; each expert hands out
   * its rows in that order (stable counting sort by expert id). */
  {
    int32_t *next = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (f = 0; f < n; ++f) {
      e = idx[f];
      pos[f] = expert_off[e] + next[e];
      next[e] += 1;
      if ((int64_t)pos[f] >= cap) pos[f] = -1; /* past the slot: dropped */
    }
    free(next);
  }

  for (s = 0; s < S; ++s)
    if ((int64_t)slot_total[s] > cap) return ORC_CAPACITY;
  return ORC_OK;
}

/* ------------------------------------------------------------- dispatch --- */

/*
 * Dispatch ([blog] "Zero-copy MoE dispatch": each token goes to the slot of
 * every expert it selected and lands straight in that slot's receive region).
 *
 * disp_x is [S][cap][H] bf16: disp_x[slot(e)][pos[t][j]] = x[t], bit for bit.
 * meta_* are [S][cap]: source pair t*K+j, its routing weight, its expert id.
 * Dropped pairs (pos -1) move nothing.
 */
void orc_dispatch(const uint16_t *x, const float *w, const int32_t *idx,
                  const int32_t *pos, int64_t T, int32_t K, int64_t H,
                  int32_t E, int32_t S, int64_t cap, uint16_t *disp_x,
                  int32_t *meta_src, float *meta_w, int32_t *meta_e) {
  int32_t eps = E / S;
  int64_t t;
  int32_t j;
  for (t = 0; t < T; ++t) {
    for (j = 0; j < K; ++j) {
      int64_t f = t * K + j;
      int32_t e = idx[f];
      if (pos[f] < 0) continue;
      int64_t row = (int64_t)(e / eps) * cap + pos[f];
      memcpy(disp_x + row * H, x + t * H, (size_t)H * sizeof(uint16_t));
      meta_src[row] = (int32_t)f;
      meta_w[row] = w[f];
      meta_e[row] = e;
    }
  }
}

/*
 * OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits; exponent 0 holds the subnormals m * 2^-9; exponent 15 with
 * mantissa 7 is NaN, and there are no infinities.  The value is exact in
 * binary32.
 */
static float e4m3_to_f32(uint8_t b) {
  int sign = b >> 7, ex = (b >> 3) & 15, m = b & 7;
  float v;
  if (ex == 15 && m == 7) return NAN;
  if (ex == 0)
    v = ldexpf((float)m, -9);
  else
    v = ldexpf((float)(8 + m), ex - 10);
  return sign ? -v : v;
}

/*
 * The expert's input when the dispatch moved 8-bit tokens (the pages hand
 * the received scales on with the received tokens and leave their use to
 * the expert): each receive row holds H e4m3 values and then ns fp32
 * scales, scale i covering the values [i*H/ns, (i+1)*H/ns).  A value is
 * decoded, multiplied by its scale in binary32 (one rounding to nearest
 * even), and rounded to bf16 (nearest even) -- the bf16 the matrix cores
 * then read.  ns == 0: no scales, the decoded value itself (exact in bf16).
 * rows: n rows of 2H bytes; out: n rows of H bf16.
 */
void orc_dequant_e4m3_rows(const uint8_t *rows, int64_t n, int64_t H, int32_t ns,
                           uint16_t *out) {
  int64_t r, k;
  int64_t blk = ns > 0 ? H / ns : H;
  for (r = 0; r < n; ++r) {
    const uint8_t *q = rows + r * 2 * H;
    for (k = 0; k < H; ++k) {
      float v = e4m3_to_f32(q[k]);
      if (ns > 0) {
        float sc;
        memcpy(&sc, q + H + 4 * (k / blk), 4);
        v = v * sc;
      }
      out[r * H + k] = orc_f32_to_bf16(v);
    }
  }
}

/*
 * Dispatch of tokens the caller has already quantized to 8 bits, with their
 * scales ([blog] "Zero-copy MoE dispatch": the op's dispatch takes the
 * tokens, their routing weights, their scales and the expert ids, and hands
 * back the received tokens, weights and scales).  The pages fix no layout
 * for the received scales; this library's reading: a receive row keeps its
 * 2H bytes, the token's H bytes fill the first half and its ns fp32 scales
 * the 4*ns bytes after them; the rest of the row is not written.
 *
 * rows is [S][cap][2H] bytes; meta_* as in orc_dispatch.
 */
void orc_dispatch_fp8(const uint8_t *x, const float *scales, int32_t ns, const float *w,
                      const int32_t *idx, const int32_t *pos, int64_t T, int32_t K,
                      int64_t H, int32_t E, int32_t S, int64_t cap, uint8_t *rows,
                      int32_t *meta_src, float *meta_w, int32_t *meta_e) {
  int32_t eps = E / S;
  int64_t t;
  int32_t j;
  for (t = 0; t < T; ++t) {
    for (j = 0; j < K; ++j) {
      int64_t f = t * K + j;
      int32_t e = idx[f];
      if (pos[f] < 0) continue;
      int64_t row = (int64_t)(e / eps) * cap + pos[f];
      uint8_t *r = rows + row * 2 * H;
      memcpy(r, x + t * H, (size_t)H);
      memcpy(r + H, scales + t * ns, (size_t)ns * sizeof(float));
      meta_src[row] = (int32_t)f;
      meta_w[row] = w[f];
      meta_e[row] = e;
    }
  }
}

/* --------------------------------------------------------------- expert --- */

/*
 * One SwiGLU expert on n rows ([blog] "Zero-copy MoE dispatch": the expert
 * reads the receive region and writes row i of its output for row i of its
 * input).
 *
 * X   [n][H] bf16           rows of this expert
 * w13 [2I][H] bf16          rows 0..I-1 gate weights, rows I..2I-1 up weights
 * w2  [H][I] bf16           down weights
 * Y   [n][H] bf16 (output)
 *
 * g_i = sum_h x_h Wg[i][h],  u_i = sum_h x_h Wu[i][h]       (double)
 * a_i = bf16( silu(g_i) * u_i ),  silu(z) = z / (1 + e^-z)  (double, rounded once)
 * y_o = bf16( sum_i a_i Wd[o][i] )                          (double, rounded once)
 */
static void orc_swiglu_one_row(const uint16_t *xr, int64_t H, int64_t I,
                               const uint16_t *w13, const uint16_t *w2,
                               uint16_t *yr, float *a /* [I] scratch */) {
  int64_t i, h, o;
  for (i = 0; i < I; ++i) {
    const uint16_t *wg = w13 + i * H;
    const uint16_t *wu = w13 + (I + i) * H;
    double g = 0.0, u = 0.0;
    for (h = 0; h < H; ++h) {
      double xv = (double)orc_bf16_to_f32(xr[h]);
      g += xv * (double)orc_bf16_to_f32(wg[h]);
      u += xv * (double)orc_bf16_to_f32(wu[h]);
    }
    double silu = g / (1.0 + exp(-g));
    a[i] = orc_bf16_to_f32(orc_f64_to_bf16(silu * u));
  }
  for (o = 0; o < H; ++o) {
    const uint16_t *wd = w2 + o * I;
    double y = 0.0;
    for (i = 0; i < I; ++i) y += (double)a[i] * (double)orc_bf16_to_f32(wd[i]);
    yr[o] = orc_f64_to_bf16(y);
  }
}

typedef struct {
  const uint16_t *X;
  int64_t n, H, I;
  const uint16_t *w13, *w2;
  uint16_t *Y;
  int tid, nthreads;
} orc_swiglu_job;

static void *orc_swiglu_worker(void *arg) {
  orc_swiglu_job *jb = (orc_swiglu_job *)arg;
  float *a = (float *)malloc((size_t)jb->I * sizeof(float));
  int64_t r;
  for (r = jb->tid; r < jb->n; r += jb->nthreads)
    orc_swiglu_one_row(jb->X + r * jb->H, jb->H, jb->I, jb->w13, jb->w2,
                       jb->Y + r * jb->H, a);
  free(a);
  return NULL;
}

/* Rows are independent, so threads split them; the arithmetic of a row does
 * not depend on the thread count. */
void orc_swiglu_rows(const uint16_t *X, int64_t n, int64_t H, int64_t I,
                     const uint16_t *w13, const uint16_t *w2, uint16_t *Y,
                     int nthreads) {
  int t;
  if (n <= 0) return;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > n) nthreads = (int)n;
  pthread_t th[256];
  orc_swiglu_job jobs[256];
  for (t = 0; t < nthreads; ++t) {
    jobs[t].X = X; jobs[t].n = n; jobs[t].H = H; jobs[t].I = I;
    jobs[t].w13 = w13; jobs[t].w2 = w2; jobs[t].Y = Y;
    jobs[t].tid = t; jobs[t].nthreads = nthreads;
    pthread_create(&th[t], NULL, orc_swiglu_worker, &jobs[t]);
  }
  for (t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* -------------------------------------------------------------- combine --- */

/*
 * Combine for a list of tokens ([blog] "Zero-copy MoE dispatch": each token's
 * rows are read back from the slots that own its experts and summed with its
 * routing weights).
 *
 * src is [S][cap][H] bf16 (the expert outputs, or the receive region itself
 * when the experts are the identity).  tokens[nt] lists the tokens to
 * produce; out is [nt][H] bf16.
 *   acc = 0; for j in 0..K-1: acc = fmaf(w[t][j], y_j[h], acc); out = bf16(acc)
 * A dropped pair (pos -1) contributes nothing.
 */
void orc_combine_tokens(const uint16_t *src, const float *w, const int32_t *idx,
                        const int32_t *pos, const int64_t *tokens, int64_t nt,
                        int32_t K, int64_t H, int32_t E, int32_t S,
                        int64_t cap, uint16_t *out) {
  int32_t eps = E / S;
  int64_t q, h;
  int32_t j;
  for (q = 0; q < nt; ++q) {
    int64_t t = tokens[q];
    for (h = 0; h < H; ++h) {
      float acc = 0.0f;
      for (j = 0; j < K; ++j) {
        int64_t f = t * K + j;
        if (pos[f] < 0) continue;
        int64_t row = (int64_t)(idx[f] / eps) * cap + pos[f];
        acc = fmaf(w[f], orc_bf16_to_f32(src[row * H + h]), acc);
      }
      out[q * H + h] = orc_f32_to_bf16(acc);
    }
  }
}

/* Same arithmetic, rows given as direct pointers: rows[q*K + j] is the bf16
 * row that token q's pair j reads.  Used on sampled tokens of large shapes,
 * where the slot arrays are not materialised on the host. */
void orc_combine_rows(const uint16_t *const *rows, const float *w, int64_t nt,
                      int32_t K, int64_t H, uint16_t *out) {
  int64_t q, h;
  int32_t j;
  for (q = 0; q < nt; ++q)
    for (h = 0; h < H; ++h) {
      float acc = 0.0f;
      for (j = 0; j < K; ++j)
        acc = fmaf(w[q * K + j], orc_bf16_to_f32(rows[q * K + j][h]), acc);
      out[q * H + h] = orc_f32_to_bf16(acc);
    }
}
