/*
 * CPU oracle for the MLX-affine quantized row product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code with the HIP library.
 *
 * It computes, plainly and slowly, in fp64:
 *
 *   q[n,k]  = bits [k*b, k*b+b) of row n's little-endian bitstream
 *   w[n,k]  = s[n, k/G] * q[n,k] + bias[n, k/G]
 *   y[m,n]  = sum_k w[n,k] * x[m,k]            (sequential fp64 sum)
 *   abs[m,n]   = sum_k |w[n,k] * x[m,k]|
 *   terms[m,n] = sum_k (|s*q*x| + |bias*x|)
 *
 * Sources (page titles and sections as they appear on the pages):
 *  - "Qwen3.8-Flash-Next faster kernels in Zig engine - #788", commit
 *    "...row kernel at every MLX width": 3- and 5-bit rows unpack eight codes
 *    from three or five bytes, low code first, as MLX packs them, and a row
 *    ends on a 32-bit word; the check compares against an fp64 product from
 *    the MLX reference dequantization.
 *  - same page, commit "tf-affine-ref": the reference dequantizes the same
 *    codes in float64 and multiplies in float64; a reference with its scales
 *    1% off must exceed the bound (the scale multiplier below).
 *  - same page, commit "2-bit prompt product": codes enter as themselves,
 *    with no offset.
 *  - affine dequantization s*q + bias per group along K: the MLX affine
 *    format named throughout the pages (codes, scales, biases per group of
 *    32, 64 or 128).
 *
 * Exactness of the fp64 steps: a bf16 scale (8 significant bits) times a
 * code (<= 8 bits) plus a bf16 bias fits in 53 bits at these magnitudes, so
 * w is exact; w times a bf16 x is exact unless w spans more than 45 bits,
 * and the sequential fp64 sum is within (K-1)*2^-53*abs of the exact value.
 */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Status values of the oracle's own validation (independent of the library). */
#define ORACLE_OK 0
#define ORACLE_BAD_BITS 1
#define ORACLE_BAD_GROUP 2
#define ORACLE_BAD_SHAPE 3

static double bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Admission rules: widths 2,3,4,5,6,8; groups 32,64,128; the group divides
 * K; a row of K codes ends on a 32-bit word. */
int oracle_check_shape(int bits, int group, int64_t n, int64_t k) {
  if (!(bits == 2 || bits == 3 || bits == 4 || bits == 5 || bits == 6 || bits == 8))
    return ORACLE_BAD_BITS;
  if (!(group == 32 || group == 64 || group == 128)) return ORACLE_BAD_GROUP;
  if (n < 1 || k < 1 || k % group != 0 || (k * bits) % 32 != 0) return ORACLE_BAD_SHAPE;
  return ORACLE_OK;
}

/* Code kk of one row, read from the row's bytes: take the bytes that hold
 * bits [kk*bits, kk*bits+bits), little-endian, shift and mask. */
unsigned oracle_code(const uint8_t *row, int bits, int64_t kk) {
  int64_t p = kk * (int64_t)bits;
  int64_t first = p / 8;
  int shift = (int)(p % 8);
  int nbytes = (shift + bits + 7) / 8;
  uint32_t window = 0;
  for (int i = 0; i < nbytes; i++) window |= (uint32_t)row[first + i] << (8 * i);
  return (window >> shift) & ((1u << bits) - 1u);
}

/* codes[n][k] of an N x K matrix stored as words[N][K*bits/32]. */
int oracle_unpack(int bits, int64_t n, int64_t k, const uint32_t *words, uint8_t *codes) {
  if (!(bits == 2 || bits == 3 || bits == 4 || bits == 5 || bits == 6 || bits == 8))
    return ORACLE_BAD_BITS;
  if (n < 1 || k < 1 || (k * bits) % 32 != 0) return ORACLE_BAD_SHAPE;
  const int64_t row_bytes = k * bits / 8;
  const uint8_t *base = (const uint8_t *)words;
  for (int64_t r = 0; r < n; r++) {
    const uint8_t *row = base + r * row_bytes;
    for (int64_t kk = 0; kk < k; kk++) codes[r * k + kk] = (uint8_t)oracle_code(row, bits, kk);
  }
  return ORACLE_OK;
}

/*
 * Rows [n0, n1) of y = x * dequant(W)^T for an m-row window.
 *   words  [N][K*bits/32], scales/biases [N][K/group] (bf16 bits), x [m][K].
 *   Outputs are [m][ldo] doubles; column n is written at [i*ldo + n].
 *   scale_mult multiplies every scale in fp64 (1.0 for the product itself,
 *   1.01 for the negative control); it is never re-rounded.
 *   abs_out / terms_out may be NULL.
 */
int oracle_gemv(int bits, int group, int64_t n_total, int64_t k, const uint32_t *words,
                const uint16_t *scales, const uint16_t *biases, int64_t m, const uint16_t *x,
                double scale_mult, int64_t n0, int64_t n1, int64_t ldo, double *y_out,
                double *abs_out, double *terms_out) {
  int rc = oracle_check_shape(bits, group, n_total, k);
  if (rc != ORACLE_OK) return rc;
  if (m < 0 || n0 < 0 || n1 > n_total || n0 > n1 || ldo < n_total) return ORACLE_BAD_SHAPE;
  const int64_t row_bytes = k * bits / 8;
  const int64_t groups = k / group;
  const uint8_t *base = (const uint8_t *)words;

  /* one dequantized row: w = s*q + bias, kept with its two parts */
  double *w = (double *)malloc(sizeof(double) * (size_t)k * 3);
  if (!w) return ORACLE_BAD_SHAPE;
  double *sq = w + k, *bb = w + 2 * k;

  for (int64_t r = n0; r < n1; r++) {
    const uint8_t *row = base + r * row_bytes;
    for (int64_t kk = 0; kk < k; kk++) {
      const int64_t g = kk / group;
      const double s = bf16_value(scales[r * groups + g]) * scale_mult;
      const double b = bf16_value(biases[r * groups + g]);
      const double q = (double)oracle_code(row, bits, kk);
      sq[kk] = s * q;
      bb[kk] = b;
      w[kk] = sq[kk] + b;
    }
    for (int64_t i = 0; i < m; i++) {
      const uint16_t *xr = x + i * k;
      double acc = 0.0, mag = 0.0, terms = 0.0;
      for (int64_t kk = 0; kk < k; kk++) {
        const double xv = bf16_value(xr[kk]);
        const double prod = w[kk] * xv;
        acc += prod;
        mag += fabs(prod);
        terms += fabs(sq[kk] * xv) + fabs(bb[kk] * xv);
      }
      y_out[i * ldo + r] = acc;
      if (abs_out) abs_out[i * ldo + r] = mag;
      if (terms_out) terms_out[i * ldo + r] = terms;
    }
  }
  free(w);
  return ORACLE_OK;
}

/* relu2 epilogue on fp64 values: y*y where y > 0, y itself where y is NaN,
 * else +0 ("relu2" option of the row kernel, commit "...row kernel at every
 * MLX width" on "Qwen3.8-Flash-Next faster kernels in Zig engine - #788"). */
void oracle_relu2(const double *y, int64_t count, double *out) {
  for (int64_t i = 0; i < count; i++) {
    const double v = y[i];
    out[i] = v > 0.0 ? v * v : (v != v ? v : 0.0);
  }
}

/* Gate/up pair of a gated MLP, the experts' "gate/up (through silu)" class
 * of P788 "tf-flashnext-widths": out = silu(g) * u with silu(g) = g / (1 +
 * exp(-g)), in fp64. */
void oracle_silu_gateup(const double *g, const double *u, int64_t count, double *out) {
  for (int64_t i = 0; i < count; i++) out[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
}
