/*
 * Runs every function of oracle/oracle.c once on small inputs, for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py).
 * Exit status 0 when all calls returned what their definitions say.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t orc_f32_to_bf16(float f);
uint16_t orc_f64_to_bf16(double d);
int orc_plan(const int32_t *idx, int64_t T, int32_t K, int32_t E, int32_t S, int64_t cap,
             int32_t *counts, int32_t *expert_off, int32_t *slot_total, int32_t *pos);
void orc_dispatch(const uint16_t *x, const float *w, const int32_t *idx, const int32_t *pos,
                  int64_t T, int32_t K, int64_t H, int32_t E, int32_t S, int64_t cap,
                  uint16_t *disp_x, int32_t *meta_src, float *meta_w, int32_t *meta_e);
void orc_dispatch_fp8(const uint8_t *x, const float *scales, int32_t ns, const float *w,
                      const int32_t *idx, const int32_t *pos, int64_t T, int32_t K, int64_t H,
                      int32_t E, int32_t S, int64_t cap, uint8_t *rows, int32_t *meta_src,
                      float *meta_w, int32_t *meta_e);
void orc_swiglu_rows(const uint16_t *X, int64_t n, int64_t H, int64_t I, const uint16_t *w13,
                     const uint16_t *w2, uint16_t *Y, int nthreads);
void orc_combine_tokens(const uint16_t *src, const float *w, const int32_t *idx,
                        const int32_t *pos, const int64_t *tokens, int64_t nt, int32_t K,
                        int64_t H, int32_t E, int32_t S, int64_t cap, uint16_t *out);
void orc_combine_rows(const uint16_t *const *rows, const float *w, int64_t nt, int32_t K,
                      int64_t H, uint16_t *out);

#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                               \
    }                                                         \
  } while (0)

static uint32_t rng_state = 12345u;
static uint32_t rnd(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 17;
  rng_state ^= rng_state << 5;
  return rng_state;
}

int main(void) {
  enum { T = 37, K = 3, E = 8, S = 4, H = 64, I = 32, NS = 5 };
  const int64_t cap = (int64_t)T * K;
  int32_t *idx = malloc(sizeof(int32_t) * T * K), *pos = malloc(sizeof(int32_t) * T * K);
  int32_t counts[E], off[E], tot[S];
  float *w = malloc(sizeof(float) * T * K);
  uint16_t *x = malloc(2 * T * H);
  uint8_t *x8 = malloc(T * H);
  float *sc = malloc(sizeof(float) * T * NS);
  int64_t i;
  for (i = 0; i < T * K; ++i) {
    idx[i] = (int32_t)(rnd() % E);
    w[i] = (float)(rnd() % 1000) / 1000.0f;
  }
  for (i = 0; i < T * H; ++i) {
    x[i] = orc_f32_to_bf16((float)((int)(rnd() % 2001) - 1000) / 500.0f);
    x8[i] = (uint8_t)rnd();
  }
  for (i = 0; i < T * NS; ++i) sc[i] = (float)(rnd() % 100) / 7.0f;

  /* rounding special cases */
  CHECK(orc_f32_to_bf16(1.0f) == 0x3F80);
  CHECK((orc_f32_to_bf16(NAN) & 0x7FC0) == 0x7FC0);
  CHECK(orc_f32_to_bf16(INFINITY) == 0x7F80);
  CHECK(orc_f32_to_bf16(1e-40f) == 0x0001 || orc_f32_to_bf16(1e-40f) == 0x0000 ||
        orc_f32_to_bf16(1e-40f) == 0x0001);
  CHECK(orc_f64_to_bf16(-2.0) == 0xC000);
  CHECK(orc_f64_to_bf16(1e300) == 0x7F80);

  /* plan: success, a bad id, a slot overflow */
  CHECK(orc_plan(idx, T, K, E, S, cap, counts, off, tot, pos) == 0);
  {
    int64_t sum = 0;
    for (i = 0; i < E; ++i) sum += counts[i];
    CHECK(sum == (int64_t)T * K);
  }
  idx[5] = E;
  CHECK(orc_plan(idx, T, K, E, S, cap, counts, off, tot, pos) != 0);
  idx[5] = 0;
  CHECK(orc_plan(idx, T, K, E, S, 1, counts, off, tot, pos) != 0);
  CHECK(orc_plan(idx, T, K, E, S, cap, counts, off, tot, pos) == 0);
  CHECK(orc_plan(idx, 0, K, E, S, cap, counts, off, tot, pos) == 0);
  CHECK(orc_plan(idx, T, K, E, S, cap, counts, off, tot, pos) == 0);

  /* dispatch, bf16 and 8-bit */
  uint16_t *dx = calloc((size_t)S * cap * H, 2);
  uint8_t *rows8 = calloc((size_t)S * cap * 2 * H, 1);
  int32_t *ms = malloc(sizeof(int32_t) * S * cap), *me = malloc(sizeof(int32_t) * S * cap);
  float *mw = malloc(sizeof(float) * S * cap);
  orc_dispatch(x, w, idx, pos, T, K, H, E, S, cap, dx, ms, mw, me);
  orc_dispatch_fp8(x8, sc, NS, w, idx, pos, T, K, H, E, S, cap, rows8, ms, mw, me);
  for (i = 0; i < T * K; ++i) {
    const int64_t row = (int64_t)(idx[i] / (E / S)) * cap + pos[i];
    CHECK(memcmp(dx + row * H, x + (i / K) * H, 2 * H) == 0);
    CHECK(memcmp(rows8 + row * 2 * H, x8 + (i / K) * H, H) == 0);
    CHECK(memcmp(rows8 + row * 2 * H + H, sc + (i / K) * NS, 4 * NS) == 0);
    CHECK(ms[row] == (int32_t)i);
  }

  /* expert: SwiGLU on every slot's rows, two threads */
  uint16_t *w13 = malloc(2 * 2 * I * H), *w2 = malloc(2 * H * I);
  for (i = 0; i < 2 * I * H; ++i) w13[i] = orc_f32_to_bf16((float)((int)(rnd() % 201) - 100) / 2000.0f);
  for (i = 0; i < H * I; ++i) w2[i] = orc_f32_to_bf16((float)((int)(rnd() % 201) - 100) / 2000.0f);
  uint16_t *y = calloc((size_t)S * cap * H, 2);
  for (i = 0; i < S; ++i) orc_swiglu_rows(dx + i * cap * H, tot[i], H, I, w13, w2, y + i * cap * H, 2);
  orc_swiglu_rows(dx, 0, H, I, w13, w2, y, 4);

  /* combine: all tokens, and the same tokens through row pointers */
  int64_t *tok = malloc(sizeof(int64_t) * T);
  for (i = 0; i < T; ++i) tok[i] = i;
  uint16_t *out = malloc(2 * T * H), *out2 = malloc(2 * T * H);
  const uint16_t **rp = malloc(sizeof(uint16_t *) * T * K);
  orc_combine_tokens(y, w, idx, pos, tok, T, K, H, E, S, cap, out);
  for (i = 0; i < T * K; ++i) rp[i] = y + ((int64_t)(idx[i] / (E / S)) * cap + pos[i]) * H;
  orc_combine_rows(rp, w, T, K, H, out2);
  CHECK(memcmp(out, out2, 2 * T * H) == 0);

  free(idx); free(pos); free(w); free(x); free(x8); free(sc); free(dx); free(rows8);
  free(ms); free(me); free(mw); free(w13); free(w2); free(y); free(tok); free(out);
  free(out2); free(rp);
  printf("oracle sanitizer driver ok\n");
  return 0;
}
