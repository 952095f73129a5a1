/*
 * rope_oracle.c -- CPU oracle for rotary position embedding (RoPE).
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, scalar statement of
 * what the GPU library computes. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it; no product code links, includes or
 * calls it, and it shares no source, header or constant with the GPU library.
 *
 * What it computes (binary64 scalar loops, nothing blocked or fused):
 *
 *   freq_i = theta^(-2i/R), i = 0 .. R/2-1
 *       rotary-embedding-torch docs, Key Parameters: `theta` is the base of
 *       the frequencies (default 10000) and `dim` is the width of the part
 *       being rotated, so the exponent runs over the rotary dim R.
 *   angle  = (p / interpolate_factor) * freq_i for the token's position p
 *       "Rotary Embedding Kernel", Overview: applied per position along the
 *       sequence. rotary-embedding-torch docs, Key Parameters:
 *       `interpolate_factor` scales sequence positions (default 1.0); read
 *       here as a divisor (a factor k > 1 squeezes k times more positions
 *       into the same angles, i.e. position interpolation). The division is
 *       one binary64 operation, exact for factor 1.
 *   (x1, x2) -> (x1*cos - x2*sin, x1*sin + x2*cos)
 *       "Rotary Embedding Kernel", Overview (the rotation of one pair).
 *   pairs (x[i], x[i + R/2]) or (x[2i], x[2i+1])
 *       "Rotary Embedding Kernel", Paired Element Layout (split-half and
 *       interleaved), applied to the first R dims of each head row.
 *   backward = the same rotation with sin negated
 *       Unsloth page, Frequently Asked Questions (backward reuses the forward
 *       kernels under a flag); the transpose of a rotation is the rotation by
 *       the opposite angle.
 *   p = pos[b * pos_batch_stride + s] when an index tensor is given, else s
 *       Unsloth page, Support for Custom Position IDs; a negative (or
 *       >= table_rows) index leaves the token's row unchanged, which is how
 *       CLS/register tokens are skipped (rotary-embedding-torch docs,
 *       flash_attn_with_rotary).
 *
 * Table contract ("table mode"): cos and sin of the binary64 angle are each
 * rounded once to float32, because that is the precision of the tables the
 * GPU path reads. Each output is then x1*c32 - s*x2*s32 evaluated in binary64
 * (both products are exact there) and rounded once, to nearest-even, into the
 * storage dtype. Rows and dims that are not rotated are copied bit for bit.
 *
 * "Exact mode" (oracle_rope_exact) uses the unrounded binary64 cos/sin and
 * binary64 inputs/outputs; it exists for the invariant checks.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Codes of this file's own interface (mirrored in oracle/__init__.py). */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2 };
enum { ORC_BHSD = 0, ORC_BSHD = 1 };
enum { ORC_SPLIT_HALF = 0, ORC_INTERLEAVED = 1 };

/* ---------------------------------------------------------------- numbers */

/* Exact value of a stored element as binary64. */
static double load_elem(const void *base, int64_t idx, int dtype) {
  if (dtype == ORC_F32) {
    float v;
    memcpy(&v, (const char *)base + 4 * idx, 4);
    return (double)v;
  }
  uint16_t h;
  memcpy(&h, (const char *)base + 2 * idx, 2);
  if (dtype == ORC_BF16) {
    /* bfloat16 is the top half of a float32 */
    uint32_t w = (uint32_t)h << 16;
    float v;
    memcpy(&v, &w, 4);
    return (double)v;
  }
  /* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits */
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1f;
  int fr = h & 0x3ff;
  double mag;
  if (ex == 0)
    mag = ldexp((double)fr, -24); /* subnormal: fr * 2^-24 */
  else if (ex == 31)
    mag = fr ? NAN : INFINITY;
  else
    mag = ldexp((double)(fr + 1024), ex - 25); /* (1 + fr/1024) * 2^(ex-15) */
  return sign ? -mag : mag;
}

/*
 * Round y to the nearest value with `prec` significant bits whose exponent is
 * at least `emin` (values below 2^emin are kept on the fixed grid 2^(emin -
 * prec + 1), i.e. gradual underflow), ties to even. The scaling by a power of
 * two is exact, and nearbyint rounds to nearest-even in the default mode.
 */
static double round_prec(double y, int prec, int emin) {
  if (y == 0.0 || !isfinite(y)) return y;
  int e;
  frexp(y, &e); /* |y| in [2^(e-1), 2^e) */
  int lead = e - 1;
  if (lead < emin) lead = emin;
  int q = lead - (prec - 1); /* exponent of one unit in the last place */
  return ldexp(nearbyint(ldexp(y, -q)), q);
}

/* binary64 -> IEEE binary16 bits, round to nearest-even, overflow to inf. */
static uint16_t to_f16_bits(double y) {
  if (isnan(y)) return 0x7e00;
  uint16_t sign = signbit(y) ? 0x8000 : 0;
  double r = fabs(round_prec(y, 11, -14));
  if (r > 65504.0) return sign | 0x7c00;
  if (r == 0.0) return sign;
  if (r < ldexp(1.0, -14)) /* subnormal: r = m * 2^-24 */
    return sign | (uint16_t)ldexp(r, 24);
  int e;
  double m = frexp(r, &e); /* r = m * 2^e, m in [0.5, 1) */
  uint16_t ex = (uint16_t)(e - 1 + 15);
  uint16_t fr = (uint16_t)(ldexp(m, 11) - 1024.0);
  return sign | (uint16_t)(ex << 10) | fr;
}

/* binary64 -> bfloat16 bits (8 significant bits, float32's exponent range). */
static uint16_t to_bf16_bits(double y) {
  if (isnan(y)) return signbit(y) ? 0xffc0 : 0x7fc0;
  uint16_t sign = signbit(y) ? 0x8000 : 0;
  double r = fabs(round_prec(y, 8, -126));
  double maxfin = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
  if (r > maxfin) return sign | 0x7f80;
  if (r == 0.0) return sign;
  if (r < ldexp(1.0, -126)) /* subnormal: r = m * 2^-133 */
    return sign | (uint16_t)ldexp(r, 133);
  int e;
  double m = frexp(r, &e);
  uint16_t ex = (uint16_t)(e - 1 + 127);
  uint16_t fr = (uint16_t)(ldexp(m, 8) - 128.0);
  return sign | (uint16_t)(ex << 7) | fr;
}

static void store_elem(void *base, int64_t idx, int dtype, double y) {
  if (dtype == ORC_F32) {
    float v = (float)y; /* C conversion: round to nearest-even */
    memcpy((char *)base + 4 * idx, &v, 4);
    return;
  }
  uint16_t h = (dtype == ORC_BF16) ? to_bf16_bits(y) : to_f16_bits(y);
  memcpy((char *)base + 2 * idx, &h, 2);
}

static int64_t elem_size(int dtype) { return dtype == ORC_F32 ? 4 : 2; }

/* ------------------------------------------------------------- the method */

/* freq_i = theta^(-2i/R), the exponent formed in binary64 as -(2i)/R. */
double oracle_freq(double theta, int64_t rotary_dim, int64_t i) {
  double expo = -(2.0 * (double)i) / (double)rotary_dim;
  return pow(theta, expo);
}

/* The angle of position p at frequency i. */
static double angle_of(double theta, double interp, int64_t rotary_dim, int64_t p,
                       int64_t i) {
  return ((double)p / interp) * oracle_freq(theta, rotary_dim, i);
}

/* Table entries of row `p`, column `i`: cos and sin of the angle, each
 * rounded once to float32. */
void oracle_table_entry(double theta, double interp, int64_t rotary_dim, int64_t p,
                        int64_t i, float *c32, float *s32) {
  double angle = angle_of(theta, interp, rotary_dim, p, i);
  *c32 = (float)cos(angle);
  *s32 = (float)sin(angle);
}

/* The whole [rows, R/2] table, row-major (for the table pins). */
void oracle_table(double theta, double interp, int64_t rotary_dim, int64_t rows,
                  float *cos_out, float *sin_out) {
  int64_t half = rotary_dim / 2;
  for (int64_t p = 0; p < rows; ++p)
    for (int64_t i = 0; i < half; ++i)
      oracle_table_entry(theta, interp, rotary_dim, p, i, &cos_out[p * half + i],
                         &sin_out[p * half + i]);
}

/* Element offset of row (b, h, s) for the two layouts. */
static int64_t row_offset(int layout, int64_t H, int64_t S, int64_t D, int64_t b,
                          int64_t h, int64_t s) {
  if (layout == ORC_BHSD) return ((b * H + h) * S + s) * D; /* [B,H,S,D] */
  return ((b * S + s) * H + h) * D;                          /* [B,S,H,D] */
}

/* Dims of pair i inside the rotated prefix of R dims. */
static void pair_dims(int pairing, int64_t R, int64_t i, int64_t *j1, int64_t *j2) {
  if (pairing == ORC_SPLIT_HALF) {
    *j1 = i;
    *j2 = i + R / 2;
  } else {
    *j1 = 2 * i;
    *j2 = 2 * i + 1;
  }
}

/* Position of token (b, s), or -1 if the token is left unrotated. */
static int64_t token_position(const int32_t *pos, int64_t pos_batch_stride,
                              int64_t table_rows, int64_t b, int64_t s) {
  int64_t p = pos ? (int64_t)pos[b * pos_batch_stride + s] : s;
  if (p < 0 || p >= table_rows) return -1;
  return p;
}

static int check_args(int dtype, int layout, int pairing, int direction, int64_t B,
                      int64_t H, int64_t S, int64_t D, int64_t R, int64_t table_rows,
                      const int32_t *pos, double interp) {
  if (dtype < ORC_F32 || dtype > ORC_BF16) return -3;
  if (!(interp > 0.0) || !isfinite(interp)) return -2;
  if (layout != ORC_BHSD && layout != ORC_BSHD) return -4;
  if (pairing != ORC_SPLIT_HALF && pairing != ORC_INTERLEAVED) return -4;
  if (direction != 1 && direction != -1) return -2;
  if (B < 0 || H < 0 || S < 0 || D < 0 || R < 0 || R > D || (R & 1)) return -2;
  if (!pos && S > table_rows) return -2;
  return 0;
}

/*
 * Table mode. `x` and `y` hold B*H*S*D elements of `dtype` in `layout`;
 * y receives the rotated copy of x (they may be the same buffer).
 * direction +1 = forward, -1 = backward. Returns 0, or a negative code for
 * arguments it cannot interpret.
 */
int oracle_rope(const void *x, void *y, int dtype, int layout, int pairing,
                int direction, int64_t B, int64_t H, int64_t S, int64_t D, int64_t R,
                double theta, double interp, const int32_t *pos, int64_t pos_batch_stride,
                int64_t table_rows) {
  int rc = check_args(dtype, layout, pairing, direction, B, H, S, D, R, table_rows, pos,
                      interp);
  if (rc) return rc;
  int64_t es = elem_size(dtype);
  if (x != y) memcpy(y, x, (size_t)(B * H * S * D * es)); /* untouched lanes */
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t s = 0; s < S; ++s) {
        int64_t p = token_position(pos, pos_batch_stride, table_rows, b, s);
        if (p < 0) continue; /* masked token: row stays as it was */
        int64_t row = row_offset(layout, H, S, D, b, h, s);
        for (int64_t i = 0; i < R / 2; ++i) {
          float c32, s32;
          oracle_table_entry(theta, interp, R, p, i, &c32, &s32);
          double c = c32, sn = (double)direction * (double)s32;
          int64_t j1, j2;
          pair_dims(pairing, R, i, &j1, &j2);
          double x1 = load_elem(x, row + j1, dtype);
          double x2 = load_elem(x, row + j2, dtype);
          double y1 = x1 * c - x2 * sn;
          double y2 = x1 * sn + x2 * c;
          store_elem(y, row + j1, dtype, y1);
          store_elem(y, row + j2, dtype, y2);
        }
      }
  return 0;
}

/* Exact mode: binary64 in and out, unrounded cos/sin of the binary64 angle. */
int oracle_rope_exact(const double *x, double *y, int layout, int pairing, int direction,
                      int64_t B, int64_t H, int64_t S, int64_t D, int64_t R, double theta,
                      double interp, const int32_t *pos, int64_t pos_batch_stride,
                      int64_t table_rows) {
  int rc = check_args(ORC_F32, layout, pairing, direction, B, H, S, D, R, table_rows, pos,
                      interp);
  if (rc) return rc;
  if (x != y) memcpy(y, x, (size_t)(B * H * S * D) * sizeof(double));
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t s = 0; s < S; ++s) {
        int64_t p = token_position(pos, pos_batch_stride, table_rows, b, s);
        if (p < 0) continue;
        int64_t row = row_offset(layout, H, S, D, b, h, s);
        for (int64_t i = 0; i < R / 2; ++i) {
          double angle = angle_of(theta, interp, R, p, i);
          double c = cos(angle), sn = (double)direction * sin(angle);
          int64_t j1, j2;
          pair_dims(pairing, R, i, &j1, &j2);
          double x1 = y[row + j1], x2 = y[row + j2];
          y[row + j1] = x1 * c - x2 * sn;
          y[row + j2] = x1 * sn + x2 * c;
        }
      }
  return 0;
}

/*
 * XPOS scaling (rotary-embedding-torch docs, Key Parameters: `use_xpos`,
 * Extrapolatable Positional Encoding). The pages name the option and nothing
 * more; its definition is the xPos paper's (Sun et al., "A
 * Length-Extrapolatable Transformer", ACL 2023): after the rotation, pair i
 * of a query at position n is scaled by zeta_i^(n/B) and pair i of a key at m
 * by zeta_i^(-m/B), with zeta_i = (i / (R/2) + gamma) / (1 + gamma), so the
 * query-key product of that pair carries zeta_i^((n - m)/B), a decay in the
 * relative distance. Positions are taken relative to `center` (n - center).
 *
 * Table contract, as for cos/sin: each factor is rounded once to float32;
 * the output is (x1*c32 - s*x2*s32) * z32 evaluated in binary64 and rounded
 * once into the storage dtype.
 */
double oracle_xpos_zeta(double gamma, int64_t rotary_dim, int64_t i) {
  return ((double)i / ((double)rotary_dim / 2.0) + gamma) / (1.0 + gamma);
}

/* The factor of pair i at position p: zeta_i^((p - center)/B) for a query row,
 * the reciprocal power for a key row (binary64, unrounded). */
static double xpos_factor(double scale_base, double gamma, double center, int64_t rotary_dim,
                          int64_t p, int64_t i, int is_key) {
  double e = ((double)p - center) / scale_base;
  return pow(oracle_xpos_zeta(gamma, rotary_dim, i), is_key ? -e : e);
}

/* [rows, R/2] float32 factor tables for query and key rows. */
void oracle_xpos_table(double scale_base, double gamma, double center, int64_t rotary_dim,
                       int64_t rows, float *zq_out, float *zk_out) {
  int64_t half = rotary_dim / 2;
  for (int64_t p = 0; p < rows; ++p)
    for (int64_t i = 0; i < half; ++i) {
      zq_out[p * half + i] = (float)xpos_factor(scale_base, gamma, center, rotary_dim, p, i, 0);
      zk_out[p * half + i] = (float)xpos_factor(scale_base, gamma, center, rotary_dim, p, i, 1);
    }
}

static int check_xpos(double scale_base, double gamma, double center) {
  if (!(scale_base > 0.0) || !isfinite(scale_base)) return -2;
  if (!(gamma > 0.0) || !isfinite(gamma) || !isfinite(center)) return -2;
  return 0;
}

/* Table mode with XPOS factors; is_key selects the key rows' factors. */
int oracle_rope_xpos(const void *x, void *y, int dtype, int layout, int pairing, int direction,
                     int is_key, int64_t B, int64_t H, int64_t S, int64_t D, int64_t R,
                     double theta, double interp, const int32_t *pos, int64_t pos_batch_stride,
                     int64_t table_rows, double scale_base, double gamma, double center) {
  int rc = check_args(dtype, layout, pairing, direction, B, H, S, D, R, table_rows, pos,
                      interp);
  if (!rc) rc = check_xpos(scale_base, gamma, center);
  if (rc) return rc;
  int64_t es = elem_size(dtype);
  if (x != y) memcpy(y, x, (size_t)(B * H * S * D * es)); /* untouched lanes */
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t s = 0; s < S; ++s) {
        int64_t p = token_position(pos, pos_batch_stride, table_rows, b, s);
        if (p < 0) continue; /* skipped token: neither rotated nor scaled */
        int64_t row = row_offset(layout, H, S, D, b, h, s);
        for (int64_t i = 0; i < R / 2; ++i) {
          float cos32, sin32;
          oracle_table_entry(theta, interp, R, p, i, &cos32, &sin32);
          /* the factor as the float32 table holds it */
          double f32 = (float)xpos_factor(scale_base, gamma, center, R, p, i, is_key);
          double cs = cos32, sg = (double)direction * (double)sin32;
          int64_t ja, jb;
          pair_dims(pairing, R, i, &ja, &jb);
          double a1 = load_elem(x, row + ja, dtype);
          double a2 = load_elem(x, row + jb, dtype);
          store_elem(y, row + ja, dtype, (a1 * cs - a2 * sg) * f32);
          store_elem(y, row + jb, dtype, (a1 * sg + a2 * cs) * f32);
        }
      }
  return 0;
}

/* Exact mode with XPOS: binary64 in and out, unrounded cos, sin and factors. */
int oracle_rope_xpos_exact(const double *x, double *y, int layout, int pairing, int direction,
                           int is_key, int64_t B, int64_t H, int64_t S, int64_t D, int64_t R,
                           double theta, double interp, const int32_t *pos,
                           int64_t pos_batch_stride, int64_t table_rows, double scale_base,
                           double gamma, double center) {
  int rc = check_args(ORC_F32, layout, pairing, direction, B, H, S, D, R, table_rows, pos,
                      interp);
  if (!rc) rc = check_xpos(scale_base, gamma, center);
  if (rc) return rc;
  if (x != y) memcpy(y, x, (size_t)(B * H * S * D) * sizeof(double));
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t s = 0; s < S; ++s) {
        int64_t p = token_position(pos, pos_batch_stride, table_rows, b, s);
        if (p < 0) continue;
        int64_t row = row_offset(layout, H, S, D, b, h, s);
        for (int64_t i = 0; i < R / 2; ++i) {
          double ang = angle_of(theta, interp, R, p, i);
          double cs = cos(ang), sg = (double)direction * sin(ang);
          double f = xpos_factor(scale_base, gamma, center, R, p, i, is_key);
          int64_t ja, jb;
          pair_dims(pairing, R, i, &ja, &jb);
          double a1 = y[row + ja], a2 = y[row + jb];
          y[row + ja] = (a1 * cs - a2 * sg) * f;
          y[row + jb] = (a1 * sg + a2 * cs) * f;
        }
      }
  return 0;
}

/*
 * Attention with RoPE applied to the loaded Q and K (rotary-embedding-torch
 * docs, flash_attn_with_rotary: the rotation is applied to Q and K inside the
 * attention computation instead of as a separate pass; GQA repeats the K/V
 * heads; is_causal). Written as the unfused composition it replaces:
 *
 *   Qr = oracle_rope(Q), Kr = oracle_rope(K)      table mode, each element
 *       rounded to the storage dtype, as a separate rotation pass would leave
 *       them (query positions: qpos, or row i at i + Sk - Sq; key positions:
 *       kpos, or row j at j)
 *   s_ij = scale * sum_d Qr[i][d] * Kr[j][d]       binary64
 *   causal: key j is visible to query i when j <= i + (Sk - Sq)
 *       (the last query row lines up with the last key row)
 *   o_i = sum_j softmax_j(s_ij) * V[j]             binary64, max subtracted
 *
 * Query head h uses K/V head h / (Hq / Hk). q [B,Hq,Sq,D], k and v
 * [B,Hk,Sk,D] in `dtype` storage; o [B,Hq,Sq,D] binary64. Returns 0, or a
 * negative code (also for Hq not a multiple of Hk, or causal with Sq > Sk).
 */
int oracle_rope_attention(const void *q, const void *k, const void *v, double *o, int dtype,
                          int pairing, int64_t B, int64_t Hq, int64_t Hk, int64_t Sq,
                          int64_t Sk, int64_t D, int64_t R, double theta, double interp,
                          const int32_t *qpos, int64_t qpos_batch_stride, const int32_t *kpos,
                          int64_t kpos_batch_stride, int64_t table_rows, int causal,
                          double scale) {
  if (Hk <= 0 || Hq % Hk || (causal && Sq > Sk) || Sq < 0 || Sk < 0) return -2;
  int64_t es = elem_size(dtype);
  void *qr = malloc((size_t)(B * Hq * Sq * D * es));
  void *kr = malloc((size_t)(B * Hk * Sk * D * es));
  int32_t *qp = NULL;
  int rc = -5;
  if (!qr || !kr) goto done;
  if (!qpos && Sk != Sq) { /* default query positions i + Sk - Sq, as an index row */
    qp = malloc((size_t)(Sq > 0 ? Sq : 1) * sizeof(int32_t));
    if (!qp) goto done;
    for (int64_t i = 0; i < Sq; ++i) qp[i] = (int32_t)(i + Sk - Sq);
    qpos = qp;
    qpos_batch_stride = 0;
  }
  rc = oracle_rope(q, qr, dtype, ORC_BHSD, pairing, 1, B, Hq, Sq, D, R, theta, interp, qpos,
                   qpos_batch_stride, table_rows);
  if (!rc)
    rc = oracle_rope(k, kr, dtype, ORC_BHSD, pairing, 1, B, Hk, Sk, D, R, theta, interp, kpos,
                     kpos_batch_stride, table_rows);
  if (rc) goto done;
  {
    double *w = malloc((size_t)(Sk > 0 ? Sk : 1) * sizeof(double));
    if (!w) { rc = -5; goto done; }
    for (int64_t b = 0; b < B; ++b)
      for (int64_t h = 0; h < Hq; ++h) {
        int64_t hk = h / (Hq / Hk);
        for (int64_t i = 0; i < Sq; ++i) {
          int64_t qrow = ((b * Hq + h) * Sq + i) * D;
          int64_t last = causal ? i + (Sk - Sq) : Sk - 1; /* last visible key */
          double m = -INFINITY;
          for (int64_t j = 0; j <= last; ++j) {
            int64_t krow = ((b * Hk + hk) * Sk + j) * D;
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d)
              dot += load_elem(qr, qrow + d, dtype) * load_elem(kr, krow + d, dtype);
            w[j] = scale * dot;
            if (w[j] > m) m = w[j];
          }
          double l = 0.0;
          for (int64_t j = 0; j <= last; ++j) {
            w[j] = exp(w[j] - m);
            l += w[j];
          }
          for (int64_t d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int64_t j = 0; j <= last; ++j)
              acc += w[j] * load_elem(v, ((b * Hk + hk) * Sk + j) * D + d, dtype);
            o[qrow + d] = last >= 0 ? acc / l : 0.0;
          }
        }
      }
    free(w);
  }
done:
  free(qr);
  free(kr);
  free(qp);
  return rc;
}

/* Rounding helpers exposed for the pins on the dtype conversions. */
uint16_t oracle_to_bf16_bits(double y) { return to_bf16_bits(y); }
uint16_t oracle_to_f16_bits(double y) { return to_f16_bits(y); }
double oracle_from_bits(uint32_t bits, int dtype) {
  if (dtype == ORC_F32) {
    float v;
    memcpy(&v, &bits, 4);
    return v;
  }
  uint16_t h = (uint16_t)bits;
  return load_elem(&h, 0, dtype);
}
