/* Test program that runs the CPU oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer: calls every exported oracle function on small
 * seeded inputs, including the edge cases the oracle flags (zero, non-finite
 * and overflowing blocks, out-of-range ids and choices, importance above
 * 2^64, idle experts), with two threads where the oracle runs threads.
 * Built and run by tests/test_oracle_sanitizers.py; exits 0 when every call
 * returned without a sanitizer report. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_geometry(int fmt, int *out5);
uint16_t orc_f32_to_f16(float f);
float orc_f16_to_f32(uint16_t h);
int orc_collect(const float *x, int64_t T, int64_t K, const int32_t *ids, int top_k, int E, double *sums,
                int64_t *counts);
int orc_merge(const float *src, const int64_t *src_counts, int E, int64_t K, float *sums, int64_t *counts);
int orc_hessian_collect(const float *x, int64_t T, int64_t K, const int32_t *ids, int top_k, int E, double *hess);
float orc_mean(const float *m, int64_t K);
int orc_importance(const float *sums, const int64_t *counts, int E, int64_t K, float floor_rel, float *imp);
uint16_t orc_anchor(int fmt, const float *x, int *st);
void orc_pack_flat(int fmt, const int *v, uint8_t *out);
void orc_unpack_flat(int fmt, const uint8_t *in, int *v);
void orc_decode_block(int fmt, const uint8_t *in, const float *grid, float *y);
int orc_encode_block(int fmt, const float *x, const float *a, const float *grid, int grid_n,
                     const uint8_t *choices, int d16_override, uint8_t *out);
int orc_group_minima(int fmt, const float *x, const float *a, const float *grid, int grid_n, uint16_t d16,
                     float *best, int *bestk);
int orc_quantize(int fmt, const float *w, int64_t rows, int64_t cols, int64_t rpe, const int64_t *row_ids,
                 int64_t n_rows, const float *grid, const float *imp, const uint8_t *choices, uint8_t *out,
                 int threads);
int orc_dequantize(int fmt, const uint8_t *packed, int64_t rows, int64_t cols, const float *grid, float *y);
float orc_damping(const float *H, float perc_damp);
int orc_choice_search(int fmt, const float *w, int64_t rows, int64_t cols, int64_t rpe, const int64_t *row_ids,
                      int64_t n_rows, const float *grid, const float *imp, const float *hess, float perc_damp,
                      uint8_t *out, int threads);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void) { /* xorshift64*: test data only */
  state ^= state >> 12; state ^= state << 25; state ^= state >> 27;
  return (uint32_t)((state * 0x2545f4914f6cdd1dull) >> 32);
}
static float uniform(void) { return (float)(next_u32() >> 8) * (1.0f / 16777216.0f); }
static float normalish(void) { return (uniform() + uniform() + uniform() - 1.5f) * 0.03f; }

int main(void) {
  static const int grid_n[5] = {256, 512, 1024, 2048, 2048};
  int geo[5];
  for (int i = 0; i < 70000; i += 7) orc_f16_to_f32(orc_f32_to_f16((float)i * 1.37f - 40000.0f));

  /* collection, merge, Hessian, importance */
  const int T = 37, K = 512, E = 5, TOPK = 3;
  float *x = malloc(sizeof(float) * T * K);
  int32_t ids[37 * 3];
  for (int i = 0; i < T * K; ++i) x[i] = normalish();
  x[5 * K + 9] = INFINITY;
  for (int i = 0; i < T * TOPK; ++i) ids[i] = (int32_t)(next_u32() % (E + 1)) - (i == 4 ? 3 : 0);
  double *sums = calloc((size_t)E * K, sizeof(double));
  int64_t counts[5] = {0};
  orc_collect(x, T, K, ids, TOPK, E, sums, counts);
  orc_collect(x, T, K, NULL, 0, 1, sums, counts);
  float *s32 = malloc(sizeof(float) * E * K), *acc = malloc(sizeof(float) * E * K);
  for (int i = 0; i < E * K; ++i) { s32[i] = (float)sums[i]; acc[i] = uniform(); }
  int64_t acc_counts[5] = {1, 2, 3, 4, 5};
  orc_merge(s32, counts, E, K, acc, acc_counts);
  double *hess = calloc((size_t)E * (K / 256) * 65536, sizeof(double));
  orc_hessian_collect(x, T, K, ids, TOPK, E, hess);
  float *imp = malloc(sizeof(float) * E * K);
  counts[1] = 0;
  orc_importance(s32, counts, E, K, 1e-6f, imp);
  orc_mean(s32, K);

  /* encode, decode, pack for every layout */
  const int rows = 4, cols = 512, nb = cols / 256;
  float *w = malloc(sizeof(float) * rows * cols), *a = malloc(sizeof(float) * 2 * cols);
  for (int i = 0; i < rows * cols; ++i) w[i] = normalish();
  for (int j = 0; j < 256; ++j) w[j] = 0.0f;              /* zero block */
  w[cols + 3] = NAN;                                      /* non-finite block */
  for (int j = 0; j < 256; ++j) w[2 * cols + j] *= 1e9f;  /* fp16 scale overflow */
  for (int i = 0; i < 2 * cols; ++i) a[i] = 0.5f + uniform();
  a[300] = 1e30f;                                         /* importance above 2^64 */
  for (int fmt = 0; fmt < 5; ++fmt) {
    const int N = grid_n[fmt];
    float *grid = malloc(sizeof(float) * N * 8);
    for (int i = 0; i < N * 8; ++i) {
      const uint32_t r = next_u32() % 3;
      grid[i] = fmt < 3 ? (float)(2 * r + 1) : (float)r - 1.0f;
    }
    orc_geometry(fmt, geo);
    const int bytes = geo[0], nunits = 16; /* block bytes; choice buffers sized for the most units */
    uint8_t *out = malloc((size_t)rows * nb * bytes);
    uint8_t *choices = malloc((size_t)rows * nb * nunits);
    for (int i = 0; i < rows * nb * nunits; ++i) choices[i] = (uint8_t)(next_u32() % 17);
    orc_quantize(fmt, w, rows, cols, 2, NULL, rows, grid, a, NULL, out, 2);
    orc_quantize(fmt, w, rows, cols, rows, NULL, rows, grid, NULL, choices, out, 2);
    const int64_t rid[2] = {3, 1};
    orc_quantize(fmt, w, rows, cols, 2, rid, 2, grid, a, NULL, out, 2);
    float *y = malloc(sizeof(float) * rows * cols);
    orc_dequantize(fmt, out, 2, cols, grid, y);
    orc_decode_block(fmt, out, grid, y);
    int st = 0;
    orc_anchor(fmt, w + 3 * cols, &st);
    uint8_t blk[128];
    orc_encode_block(fmt, w + 3 * cols, a, grid, 16, NULL, 0x2c00, blk);
    float best[32 * 16];
    int bestk[32 * 16];
    orc_group_minima(fmt, w + 3 * cols, a, grid, 16, 0x2c00, best, bestk);
    int v[113];
    for (int i = 0; i < 113; ++i) v[i] = (int)(next_u32() % 2048);
    orc_pack_flat(fmt, v, blk);
    orc_unpack_flat(fmt, blk, v);
    float *H = malloc(sizeof(float) * 2 * 65536);
    for (int i = 0; i < 2 * 65536; ++i) H[i] = normalish();
    orc_damping(H, 0.3f);
    uint8_t picks[4 * 2 * 16];
    orc_choice_search(fmt, w + 3 * cols, 1, cols, 1, NULL, 1, grid, a, H, 0.3f, picks, 2);
    free(H); free(y); free(choices); free(out); free(grid);
  }
  free(x); free(sums); free(s32); free(acc); free(hess); free(imp); free(w); free(a);
  printf("oracle sanitizer run ok\n");
  return 0;
}
