/*
 * Plain loops of the oracle: y[r][n] = sum_k deq(W)[n][k] * x[r][k] in double, one
 * thread, for the three stored weight formats of the decode layer.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by oracle/layer.py (tests, smoke, the bench's
 * cpu_baseline leg); shares nothing with the HIP library.
 *
 * Formats ("Mono decode layer for DeepSeek-V4.1-Flash on MI355X", vLLM PR 60397,
 * Design and Layout; element and scale encodings per the OCP MX v1.0 and OFP8
 * specifications):
 *   MXFP8 tile32  e4m3 [N][K] row-major, one E8M0 byte per 32x32 tile [N/32][K/32]
 *   FP8 block128  e4m3 [N][K] row-major, one float per 128x128 block [N/128][K/128]
 *   MXFP4         e2m1 nibbles [N][K/2] (low nibble = even k), one E8M0 per 32 along
 *                 K [N][K/32]
 * Each element is decoded exactly (decode tables built by oracle/formats.py from the
 * bit definitions), multiplied by its block scale, then into each input row, and the
 * products are summed in order of k.  R <= 64 input rows.
 */
#include <stdint.h>

#define MAXR 64

/* x: [R][K] doubles; y: [R][N] doubles (overwritten).  e8m0_table[b] = 2^(b-127). */
void oracle_gemv_mxfp8(const uint8_t *restrict w, const uint8_t *restrict s, int N, int K,
                       const double *restrict e4m3_table, const double *restrict e8m0_table,
                       const double *restrict x, int R, double *restrict y) {
  for (int n = 0; n < N; n++) {
    double acc[MAXR] = {0};
    const uint8_t *row = w + (long)n * K;
    const uint8_t *srow = s + (long)(n / 32) * (K / 32);
    for (int k = 0; k < K; k++) {
      const double v = e4m3_table[row[k]] * e8m0_table[srow[k / 32]];
      for (int r = 0; r < R; r++) acc[r] += v * x[(long)r * K + k];
    }
    for (int r = 0; r < R; r++) y[(long)r * N + n] = acc[r];
  }
}

void oracle_gemv_fp8b128(const uint8_t *restrict w, const float *restrict s, int N, int K,
                         const double *restrict e4m3_table, const double *restrict x, int R,
                         double *restrict y) {
  for (int n = 0; n < N; n++) {
    double acc[MAXR] = {0};
    const uint8_t *row = w + (long)n * K;
    const float *srow = s + (long)(n / 128) * (K / 128);
    for (int k = 0; k < K; k++) {
      const double v = e4m3_table[row[k]] * (double)srow[k / 128];
      for (int r = 0; r < R; r++) acc[r] += v * x[(long)r * K + k];
    }
    for (int r = 0; r < R; r++) y[(long)r * N + n] = acc[r];
  }
}

void oracle_gemv_mxfp4(const uint8_t *restrict w, const uint8_t *restrict s, int N, int K,
                       const double *restrict e2m1_table, const double *restrict e8m0_table,
                       const double *restrict x, int R, double *restrict y) {
  for (int n = 0; n < N; n++) {
    double acc[MAXR] = {0};
    const uint8_t *row = w + (long)n * (K / 2);
    const uint8_t *srow = s + (long)n * (K / 32);
    for (int k = 0; k < K; k++) {
      const uint8_t byte = row[k / 2];
      const int code = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
      const double v = e2m1_table[code] * e8m0_table[srow[k / 32]];
      for (int r = 0; r < R; r++) acc[r] += v * x[(long)r * K + k];
    }
    for (int r = 0; r < R; r++) y[(long)r * N + n] = acc[r];
  }
}
