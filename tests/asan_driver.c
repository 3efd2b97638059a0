/*
 * asan_driver.c -- host-side memory checks, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_asan_cpu.py.  No GPU is used.
 *
 * Part 1 drives the HIP library's host code (compiled host-only with the
 * sanitizers): every argument check that returns before a launch, the
 * workspace sizing over a sweep of shapes, status strings.  Part 2 drives the
 * CPU oracle (test infrastructure, compiled with the same sanitizers) over
 * small random cases in both dtypes, and compares the metadata it returns with
 * a brute-force stable sort written here.  Any out-of-bounds access, use after
 * free, leak or undefined operation aborts the run with a report.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lora_mi355x.h"

/* the oracle's entry points (oracle/lora_oracle.c) */
int oracle_prepare_meta(const int32_t *token_slot, int64_t T, int32_t S, int32_t *sorted, int32_t *seg_slot,
                        int32_t *seg_count, int32_t *seg_start, int32_t *num_segments, int32_t *no_lora,
                        int32_t *num_bad);
int oracle_lora_rows(int dtype, const void *x, int64_t ldx, int64_t d_in, const int32_t *token_slot, int32_t S,
                     int32_t n_slices, const void *const *A, const int64_t *a_slot_stride, int32_t r_max,
                     const void *const *B, const int64_t *b_slot_stride, const int64_t *width,
                     const int64_t *offset, double scale, const float *slot_scale, const void *y0, int64_t ldy,
                     int add, const int64_t *rows, int64_t n_rows, double *y_out, double *u_out);
int oracle_expand_rows(int dtype, const float *u, int64_t ldu, const int32_t *token_slot, int32_t S,
                       int32_t n_slices, int32_t r_max, const void *const *B, const int64_t *b_slot_stride,
                       const int64_t *width, const int64_t *offset, const void *y0, int64_t ldy, int add,
                       const int64_t *rows, int64_t n_rows, double *y_out);
int oracle_moe_keys(const int32_t *topk_ids, int64_t T, int32_t topk, const int32_t *token_slot, int32_t S,
                    int32_t E_global, int32_t E_local, const int32_t *expert_map, int32_t *keys);

static int failures = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {  /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float next_f32(void) { return (float)((int)(next_u32() % 2001) - 1000) / 1000.0f; }

/* ------------------------------------------------------------ part 1: library */

/* A fake device address: the checks under test return before any launch, so
 * nothing dereferences it. */
static void *fake(uintptr_t misalign) { return (void *)((uintptr_t)0x7f0000000000ull + misalign); }

static lora_meta fake_meta(int64_t T, int32_t S) {
  lora_meta m;
  memset(&m, 0, sizeof m);
  m.num_tokens = T;
  m.num_slots = S;
  m.x_row_div = 1;
  m.sorted = m.sorted_slot = m.seg_slot = m.seg_count = m.seg_start = m.info = m.tiles = (int32_t *)fake(0);
  return m;
}

static void library_checks(void) {
  CHECK(lora_abi_version() > 0);
  for (int s = -1; s <= 6; ++s) {
    const char *msg = lora_status_string((lora_status)s);
    CHECK(msg != NULL && strlen(msg) > 0);
  }
  size_t b = 0;
  CHECK(lora_meta_workspace_bytes(-1, 4, &b) == LORA_ERR_INVALID_ARG);
  CHECK(lora_meta_workspace_bytes(10, 1024, &b) == LORA_ERR_UNSUPPORTED);
  CHECK(lora_meta_workspace_bytes(10, 4, NULL) == LORA_ERR_INVALID_ARG);

  /* workspace sizing over a sweep: succeeds for every supported rank, grows
   * with the token count, never below the rendezvous words */
  const int64_t Ts[] = {0, 1, 7, 64, 256, 4096, 17705, 1 << 20};
  const int32_t Ss[] = {1, 8, 128, 1023};
  const int64_t dins[] = {8, 4096, 14336};
  for (size_t ti = 0; ti < sizeof Ts / sizeof Ts[0]; ++ti)
    for (size_t si = 0; si < sizeof Ss / sizeof Ss[0]; ++si)
      for (size_t di = 0; di < sizeof dins / sizeof dins[0]; ++di)
        for (int32_t r = 0; r <= 136; r += 4)
          for (int dt = 0; dt < 2; ++dt)
            for (int mode = 0; mode < 3; ++mode)
              for (int32_t n = 1; n <= 8; n += 7) {
                size_t wa = 0, ws = 0, wm = 0;
                const lora_status sa =
                    lora_apply_workspace_bytes(Ts[ti], Ss[si], dins[di], n, r, (lora_dtype)dt, (lora_mode)mode, &wa);
                const lora_status ss =
                    lora_shrink_workspace_bytes(Ts[ti], Ss[si], dins[di], n, r, (lora_dtype)dt, (lora_mode)mode, &ws);
                const int ok_rank = r >= 8 && r <= 128 && r % 8 == 0;
                CHECK((sa == LORA_OK) == ok_rank);
                CHECK((ss == LORA_OK) == ok_rank);
                if (ok_rank) {
                  CHECK(wa >= LORA_APPLY_SYNC_BYTES + 4u * (size_t)n * (size_t)Ts[ti] * (size_t)r);
                  CHECK(ws % 256 == 0);
                }
                CHECK(lora_meta_workspace_bytes(Ts[ti], Ss[si], &wm) == LORA_OK && wm > 0);
              }

  /* argument checks of the compute calls (all return before a launch) */
  lora_meta m = fake_meta(64, 4);
  lora_weight A[9], B[9];
  memset(A, 0, sizeof A);
  memset(B, 0, sizeof B);
  for (int s = 0; s < 9; ++s) {
    A[s].ptr = fake(0);
    A[s].slot_stride = 64 * 16;
    B[s].ptr = fake(0);
    B[s].slot_stride = 16 * 64;
  }
  int64_t width[2] = {64, 32}, offset[2] = {0, 64};
  const float one = 1.0f;
  (void)one;
  CHECK(lora_shrink(NULL, fake(0), 64, 64, LORA_BF16, 1, A, 16, 1.f, NULL, NULL, (float *)fake(0), LORA_MODE_AUTO,
                    fake(0), 1 << 15, NULL) == LORA_ERR_INVALID_ARG);
  CHECK(lora_shrink(&m, fake(0), 64, 64, LORA_BF16, 1, A, 12, 1.f, NULL, NULL, (float *)fake(0), LORA_MODE_AUTO,
                    fake(0), 1 << 15, NULL) == LORA_ERR_UNSUPPORTED);
  CHECK(lora_shrink(&m, fake(0), 64, 64, LORA_BF16, 9, A, 16, 1.f, NULL, NULL, (float *)fake(0), LORA_MODE_AUTO,
                    fake(0), 1 << 15, NULL) == LORA_ERR_UNSUPPORTED);
  CHECK(lora_shrink(&m, fake(0), 64, 64, (lora_dtype)7, 1, A, 16, 1.f, NULL, NULL, (float *)fake(0), LORA_MODE_AUTO,
                    fake(0), 1 << 15, NULL) == LORA_ERR_UNSUPPORTED);
  CHECK(lora_shrink(&m, fake(0), 64, 64, LORA_BF16, 1, A, 16, 1.f, NULL, NULL, (float *)fake(0), (lora_mode)-3,
                    fake(0), 1 << 15, NULL) == LORA_ERR_UNSUPPORTED);
  CHECK(lora_expand(&m, (const float *)fake(0), 2, B, width, offset, 16, NULL, fake(0), 96, (lora_dtype)-1, 1,
                    LORA_MODE_AUTO, NULL) == LORA_ERR_UNSUPPORTED);
  CHECK(lora_apply(&m, fake(0), 64, 64, LORA_BF16, 1, A, B, width, offset, 16, 1.f, NULL, NULL, fake(0), 96, 1,
                   (lora_mode)9, fake(0), 1 << 22, NULL) == LORA_ERR_UNSUPPORTED);
  /* rank-major A: bf16, r_max >= 16, AUTO or SGMV, every slice alike; B default only */
  A[0].layout = LORA_LAYOUT_RANK_ROWS;
  CHECK(lora_shrink(&m, fake(0), 64, 64, LORA_F32, 1, A, 16, 1.f, NULL, NULL, (float *)fake(0), LORA_MODE_AUTO,
                    fake(0), 1 << 15, NULL) == LORA_ERR_UNSUPPORTED);
  CHECK(lora_shrink(&m, fake(0), 64, 64, LORA_BF16, 1, A, 16, 1.f, NULL, NULL, (float *)fake(0), LORA_MODE_BGMV,
                    fake(0), 1 << 15, NULL) == LORA_ERR_UNSUPPORTED);
  CHECK(lora_shrink(&m, fake(0), 64, 64, LORA_BF16, 1, A, 8, 1.f, NULL, NULL, (float *)fake(0), LORA_MODE_AUTO,
                    fake(0), 1 << 15, NULL) == LORA_ERR_UNSUPPORTED);
  CHECK(lora_shrink(&m, fake(0), 64, 64, LORA_BF16, 2, A, 16, 1.f, NULL, NULL, (float *)fake(0), LORA_MODE_AUTO,
                    fake(0), 1 << 15, NULL) == LORA_ERR_INVALID_ARG);  /* slices differ */
  A[0].layout = 7;
  CHECK(lora_shrink(&m, fake(0), 64, 64, LORA_BF16, 1, A, 16, 1.f, NULL, NULL, (float *)fake(0), LORA_MODE_AUTO,
                    fake(0), 1 << 15, NULL) == LORA_ERR_UNSUPPORTED);
  A[0].layout = LORA_LAYOUT_DEFAULT;
  A[0].reserved = 1;
  CHECK(lora_shrink(&m, fake(0), 64, 64, LORA_BF16, 1, A, 16, 1.f, NULL, NULL, (float *)fake(0), LORA_MODE_AUTO,
                    fake(0), 1 << 15, NULL) == LORA_ERR_INVALID_ARG);
  A[0].reserved = 0;
  B[1].layout = LORA_LAYOUT_OUT_ROWS;  /* slices differ */
  CHECK(lora_expand(&m, (const float *)fake(0), 2, B, width, offset, 16, NULL, fake(0), 96, LORA_BF16, 1,
                    LORA_MODE_AUTO, NULL) == LORA_ERR_INVALID_ARG);
  B[0].layout = B[1].layout = LORA_LAYOUT_RANK_ROWS;
  CHECK(lora_expand(&m, (const float *)fake(0), 2, B, width, offset, 16, NULL, fake(0), 96, LORA_BF16, 1,
                    LORA_MODE_AUTO, NULL) == LORA_ERR_UNSUPPORTED);
  B[0].layout = B[1].layout = LORA_LAYOUT_OUT_ROWS;
  CHECK(lora_expand(&m, (const float *)fake(0), 2, B, width, offset, 16, NULL, fake(0), 96, LORA_F32, 1,
                    LORA_MODE_AUTO, NULL) == LORA_ERR_UNSUPPORTED);
  CHECK(lora_expand(&m, (const float *)fake(0), 2, B, width, offset, 16, NULL, fake(0), 96, LORA_BF16, 1,
                    LORA_MODE_BGMV, NULL) == LORA_ERR_UNSUPPORTED);
  B[0].layout = B[1].layout = LORA_LAYOUT_DEFAULT;
  CHECK(lora_shrink(&m, fake(2), 64, 64, LORA_BF16, 1, A, 16, 1.f, NULL, NULL, (float *)fake(0), LORA_MODE_AUTO,
                    fake(0), 1 << 15, NULL) == LORA_ERR_INVALID_ARG);
  CHECK(lora_expand(&m, (const float *)fake(0), 2, B, width, offset, 16, NULL, fake(0), 90, LORA_BF16, 1,
                    LORA_MODE_AUTO, NULL) == LORA_ERR_INVALID_ARG);
  offset[1] = 32;  /* windows overlap */
  CHECK(lora_expand(&m, (const float *)fake(0), 2, B, width, offset, 16, NULL, fake(0), 96, LORA_BF16, 1,
                    LORA_MODE_AUTO, NULL) == LORA_ERR_INVALID_ARG);
  offset[1] = 64;
  CHECK(lora_expand(&m, (const float *)fake(0), 2, B, width, offset, 20, NULL, fake(0), 96, LORA_BF16, 1,
                    LORA_MODE_AUTO, NULL) == LORA_ERR_UNSUPPORTED);
  /* lora_apply: workspace too small, misaligned, null meta */
  CHECK(lora_apply(&m, fake(0), 64, 64, LORA_BF16, 1, A, B, width, offset, 16, 1.f, NULL, NULL, fake(0), 96, 1,
                   LORA_MODE_AUTO, fake(0), 16, NULL) == LORA_ERR_WORKSPACE);
  CHECK(lora_apply(&m, fake(0), 64, 64, LORA_BF16, 1, A, B, width, offset, 16, 1.f, NULL, NULL, fake(0), 96, 1,
                   LORA_MODE_AUTO, fake(8), 1 << 22, NULL) == LORA_ERR_WORKSPACE);
  CHECK(lora_apply(NULL, fake(0), 64, 64, LORA_BF16, 1, A, B, width, offset, 16, 1.f, NULL, NULL, fake(0), 96, 1,
                   LORA_MODE_AUTO, fake(0), 1 << 22, NULL) == LORA_ERR_INVALID_ARG);
  CHECK(lora_apply_workspace_init(NULL, 1 << 20, NULL) == LORA_ERR_INVALID_ARG);
  CHECK(lora_apply_workspace_init(fake(0), LORA_APPLY_SYNC_BYTES - 16, NULL) == LORA_ERR_WORKSPACE);
  lora_meta huge = fake_meta((int64_t)1 << 22, 4);
  CHECK(lora_apply_noalloc(&huge, fake(0), 64, 64, LORA_BF16, 1, A, B, width, offset, 16, 1.f, NULL, NULL, fake(0),
                           96, 1, LORA_MODE_AUTO, NULL) == LORA_ERR_WORKSPACE);
  CHECK(lora_apply_noalloc(&m, fake(0), 64, 64, LORA_BF16, 1, A, B, width, offset, 12, 1.f, NULL, NULL, fake(0),
                           96, 1, LORA_MODE_AUTO, NULL) == LORA_ERR_UNSUPPORTED);
  size_t mb = 0;
  CHECK(lora_moe_meta_workspace_bytes(16, 8, 4, 32, &mb) == LORA_OK && mb > 0);
  CHECK(lora_moe_meta_workspace_bytes(16, 8, 64, 32, &mb) == LORA_ERR_UNSUPPORTED);
}

/* ------------------------------------------------------------ part 2: oracle */

static uint16_t to_bf16(float f) {  /* round to nearest even; inputs are finite */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static void oracle_meta_checks(void) {
  /* every token_slot in {-1..S-1}^T for T <= 5, S <= 3, against a stable
   * sort written here (insertion sort on (key, index)) */
  for (int32_t S = 1; S <= 3; ++S)
    for (int64_t T = 0; T <= 5; ++T) {
      int64_t combos = 1;
      for (int64_t t = 0; t < T; ++t) combos *= S + 1;
      for (int64_t c = 0; c < combos; ++c) {
        int32_t ts[8], sorted[8], seg_slot[8], seg_count[8], seg_start[8], nseg = 0, no_lora = 0, bad = 0;
        int64_t v = c;
        for (int64_t t = 0; t < T; ++t) {
          ts[t] = (int32_t)(v % (S + 1)) - 1;
          v /= S + 1;
        }
        CHECK(oracle_prepare_meta(ts, T, S, sorted, seg_slot, seg_count, seg_start, &nseg, &no_lora, &bad) == 0);
        int32_t idx[8];
        for (int64_t t = 0; t < T; ++t) idx[t] = (int32_t)t;
        for (int64_t i = 1; i < T; ++i)
          for (int64_t j = i; j > 0 && ts[idx[j - 1]] > ts[idx[j]]; --j) {
            const int32_t tmp = idx[j];
            idx[j] = idx[j - 1];
            idx[j - 1] = tmp;
          }
        for (int64_t t = 0; t < T; ++t) CHECK(sorted[t] == idx[t]);
        CHECK(bad == 0);
        int32_t total = 0;
        for (int32_t g = 0; g < nseg; ++g) total += seg_count[g];
        CHECK(total == T && seg_start[nseg] == T);
      }
    }
}

static void oracle_rows_checks(void) {
  for (int dtype = 0; dtype < 2; ++dtype) {
    const int64_t T = 37, d_in = 40, ldx = 48, ldy = 72;
    const int32_t S = 3, n_slices = 2, r = 24;
    const int64_t width[2] = {32, 24}, offset[2] = {0, 40};
    const size_t es = dtype ? 2 : 4;
    void *x = malloc(es * (size_t)(T * ldx)), *y0 = malloc(es * (size_t)(T * ldy));
    void *A[2], *B[2];
    int64_t astr[2], bstr[2];
    for (int s = 0; s < n_slices; ++s) {
      astr[s] = d_in * r;
      bstr[s] = r * width[s];
      A[s] = malloc(es * (size_t)(S * astr[s]));
      B[s] = malloc(es * (size_t)(S * bstr[s]));
    }
#define FILL(buf, n)                                                          \
  for (int64_t i = 0; i < (n); ++i) {                                         \
    const float f = next_f32();                                               \
    if (dtype) ((uint16_t *)(buf))[i] = to_bf16(f); else ((float *)(buf))[i] = f; \
  }
    FILL(x, T * ldx);
    FILL(y0, T * ldy);
    for (int s = 0; s < n_slices; ++s) {
      FILL(A[s], S * astr[s]);
      FILL(B[s], S * bstr[s]);
    }
#undef FILL
    int32_t ts[37];
    for (int64_t t = 0; t < T; ++t) ts[t] = (int32_t)(next_u32() % (S + 2)) - 1;  /* includes a bad id S */
    int64_t rows[37];
    for (int64_t t = 0; t < T; ++t) rows[t] = T - 1 - t;
    const float slot_scale[3] = {0.5f, 1.0f, 2.0f};
    double *y = malloc(sizeof(double) * (size_t)(T * ldy));
    double *u = malloc(sizeof(double) * (size_t)(T * n_slices * r));
    for (int add = 0; add < 2; ++add) {
      CHECK(oracle_lora_rows(dtype, x, ldx, d_in, ts, S, n_slices, (const void *const *)A, astr, r,
                             (const void *const *)B, bstr, width, offset, 0.75, slot_scale, y0, ldy, add, rows, T, y,
                             u) == 0);
      /* the expand alone from the same u (fp32 copy, layout [slice][token][rank]) */
      float *uf = malloc(sizeof(float) * (size_t)(n_slices * T * r));
      memset(uf, 0, sizeof(float) * (size_t)(n_slices * T * r));
      for (int64_t i = 0; i < T; ++i)
        for (int32_t s = 0; s < n_slices; ++s)
          for (int32_t j = 0; j < r; ++j) uf[((int64_t)s * T + rows[i]) * r + j] = (float)u[(i * n_slices + s) * r + j];
      double *y2 = malloc(sizeof(double) * (size_t)(T * ldy));
      CHECK(oracle_expand_rows(dtype, uf, r, ts, S, n_slices, r, (const void *const *)B, bstr, width, offset, y0,
                               ldy, add, rows, T, y2) == 0);
      /* columns outside every window equal y0 in both */
      for (int64_t i = 0; i < T; ++i)
        for (int64_t c = 32; c < 40; ++c) CHECK(y[i * ldy + c] == y2[i * ldy + c]);
      free(y2);
      free(uf);
    }
    int32_t topk_ids[37 * 2], keys[37 * 2], emap[6] = {0, -1, 1, -1, 2, 0};
    for (int64_t i = 0; i < T * 2; ++i) topk_ids[i] = (int32_t)(next_u32() % 7) - (i == 5);  /* one id -1 */
    CHECK(oracle_moe_keys(topk_ids, T, 2, ts, S, 6, 3, emap, keys) == 0);
    for (int64_t i = 0; i < T * 2; ++i) CHECK(keys[i] >= -2 && keys[i] < S * 3);  /* -2: an id out of range */
    free(u);
    free(y);
    for (int s = 0; s < n_slices; ++s) {
      free(A[s]);
      free(B[s]);
    }
    free(x);
    free(y0);
  }
}

int main(void) {
  library_checks();
  oracle_meta_checks();
  oracle_rows_checks();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("asan driver: all checks passed\n");
  return 0;
}
