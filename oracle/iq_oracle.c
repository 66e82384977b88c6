/*
 * iq_oracle.c -- slow, plain CPU oracle for importance-weighted GGML IQ
 * encoding and imatrix collection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library: every constant below is restated here from the
 * pages.
 *
 * Sources (web pages; cited by title and section):
 *  [2735] ModelOpt PR "Add imatrix calibration for the GGML formats and use it
 *         for fused MoE experts" -- description bullets ("What imatrix does",
 *         "Bounded memory", "Idle experts", "Checked up front", "Shared floor").
 *  [2513] ModelOpt PR #2513 (IQ2_XXS / IQ2_S / IQ1_M) -- the three commit
 *         messages and the IQ1_M PR body ("What's distinctive about it",
 *         "A scale-anchor correction", "Testing").
 *  [3157] ModelOpt PR "[1/5] Let the GGML IQ encoders take fixed per-group
 *         choices" -- description and bot review.
 *  [recipes] ModelOpt modelopt_recipes folder page -- IQ1_M CUDA encoder
 *         commit ("The kernel", "Shared with IQ1_S rather than copied").
 *  [coverage] "MoE expert coverage in imatrix calibration" -- Facts list.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared
 * Every fused multiply-add is an explicit fmaf(); every other operation is a
 * single IEEE fp32 operation in the order written.  Collection accumulates in
 * fp64.
 *
 * Readings of the pages that the code below fixes (the pages are silent or
 * ambiguous there); each is named where it is used:
 *  R1  IQ2 anchor ratio r = 1 (the pages print no IQ2 ratio).
 *  R2  d = (r * amax) / Qmax, Qmax = top local multiplier * top grid magnitude:
 *      IQ2 3.875 * 5, IQ1 15 * 1.  Local multipliers (2c+1)/8 (IQ2), 2ls+1 (IQ1).
 *  R3  IQ1_M peak-to-RMS = amax / sqrt(mean x^2) over the 256-value block.
 *  R4  the search runs at the fp16-rounded d.
 *  R5  amax == 0, fp16(d) == 0, non-finite inputs, fp16 overflow and
 *      out-of-range fixed choices give an all-zero block (the all-zero rule of
 *      the [3157] review); the last three also raise a status bit.
 *  R6  imatrix floor: a_j = sqrt(max(E_j, 1e-6 * mean_j E_j)); the mean is the
 *      plain one: the E_j summed in fp64 in ascending j, divided by K in fp64,
 *      rounded to fp32 (orc_mean).
 *  R7  odd sign parity (IQ2_XXS, IQ2_XS): per candidate entry, flip the element
 *      with the least a_j*|x_j|*g_kj (lowest j on ties).
 *  R8  x = -0 counts as positive.
 *  R9  choice ties go to the lowest choice; unit score summed left to right.
 *  R10 IQ1 shift h=0 is +1/8 (the "lower" shift), h=1 is -1/8.
 *  R11 IQ1_S choice c = (h << 3) | ls.
 *  R12 the reduced error: per group t = s*G - 2P, G = sum a_j u_j^2,
 *      P = sum a_j y_j u_j, computed as written in iq2_group/iq1_group.
 *  R13 byte layouts (sizes fixed by [2513]; field positions our own).
 *  R20 a block whose importance holds a value outside [0, 2^64] (NaN, a
 *      negative value, or one no floored square root of a finite fp32 second
 *      moment can reach, since sqrt(FLT_MAX) < 2^64) is refused: all-zero
 *      bytes and the BADIMP status bit.  Within that range and with a finite
 *      fp16 scale every fp32 intermediate of the search stays finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <pthread.h>

enum { ORC_IQ2_XXS = 0, ORC_IQ2_XS = 1, ORC_IQ2_S = 2, ORC_IQ1_S = 3, ORC_IQ1_M = 4 };

/* status bits */
#define ORC_ST_NONFINITE 1
#define ORC_ST_OVERFLOW 2
#define ORC_ST_BADCHOICE 4
#define ORC_ST_BADIMP 8
#define ORC_ST_BADID 16

/* largest accepted importance value (R20): 2^64 */
#define ORC_IMP_MAX 18446744073709551616.0f

typedef struct {
  int block_bytes; /* [2513]: 2.0625 / 2.3125 / 2.5625 / 1.5625 / 1.75 bits per weight */
  int grid_n;      /* codebook entries: 256 / 512 / 1024 / 2048 / 2048            */
  int gpu;         /* groups (8 values) per choice unit                           */
  int units;       /* choice units per 256-value block                            */
  int nchoices;    /* choices per unit                                            */
} orc_geom;

static const orc_geom GEOM[5] = {
    {66, 256, 4, 8, 16},  /* IQ2_XXS: 4-bit scale per 32 values            */
    {74, 512, 2, 16, 16}, /* IQ2_XS : 4-bit scale per 16 values            */
    {82, 1024, 2, 16, 16},/* IQ2_S  : 4-bit scale per 16 values            */
    {50, 2048, 4, 8, 16}, /* IQ1_S  : 3-bit scale + delta sign per 32      */
    {56, 2048, 2, 16, 8}, /* IQ1_M  : 3-bit scale per 16, shift per group  */
};

static int is_iq1(int fmt) { return fmt == ORC_IQ1_S || fmt == ORC_IQ1_M; }

int orc_geometry(int fmt, int *out5) {
  if (fmt < 0 || fmt > 4) return -1;
  out5[0] = GEOM[fmt].block_bytes;
  out5[1] = GEOM[fmt].grid_n;
  out5[2] = GEOM[fmt].gpu;
  out5[3] = GEOM[fmt].units;
  out5[4] = GEOM[fmt].nchoices;
  return 0;
}

/* ------------------------------------------------------------------------- */
/* IEEE binary16 conversion, round to nearest, ties to even                  */
/* ------------------------------------------------------------------------- */
uint16_t orc_f32_to_f16(float f) {
  uint16_t sign = signbit(f) ? 0x8000 : 0;
  if (isnan(f)) return sign | 0x7e00;
  double a = fabs((double)f);
  if (a >= 65520.0) return sign | 0x7c00; /* beyond max + half ulp: inf */
  if (a == 0.0) return sign;
  int e; /* a = m * 2^e, m in [0.5, 1) */
  frexp(a, &e);
  int exp = e - 1;            /* a in [2^exp, 2^(exp+1)) */
  if (exp < -14) exp = -14;   /* subnormal range shares the quantum of 2^-14 */
  double q = ldexp(1.0, exp - 10);
  double n = a / q;           /* exact: power-of-two scaling */
  double fl = floor(n);
  double rem = n - fl;
  double r = fl;
  if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) r = fl + 1.0;
  /* r * q is the rounded magnitude; encode it */
  if (r >= 2048.0) { r /= 2.0; exp += 1; }
  if (exp > 15) return sign | 0x7c00;
  if (r < 1024.0) return sign | (uint16_t)r; /* subnormal (exp == -14) */
  return sign | (uint16_t)(((exp + 15) << 10) | ((int)r - 1024));
}

float orc_f16_to_f32(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 31) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m, -24);
  else v = ldexp((double)(m + 1024), e - 25);
  return (float)(sign ? -v : v);
}

/* ------------------------------------------------------------------------- */
/* imatrix collection  ([2735] "What imatrix does", "Bounded memory";        */
/* [coverage] Facts: squares added only to the experts in a token's top-k,  */
/* one counts entry per expert)                                              */
/* ------------------------------------------------------------------------- */
/* x [T, K] fp32; ids [T, top_k] or NULL (dense: one statistic, count += T).
 * sums [E, K] fp64 and counts [E] are accumulated in place.  Returns status
 * bits: non-finite values seen in a row that reached some expert, bad ids. */
int orc_collect(const float *x, int64_t T, int64_t K, const int32_t *ids, int top_k,
                int num_experts, double *sums, int64_t *counts) {
  int st = 0;
  if (ids == NULL) {
    for (int64_t t = 0; t < T; ++t)
      for (int64_t j = 0; j < K; ++j) {
        double v = (double)x[t * K + j];
        if (!isfinite(v)) st |= ORC_ST_NONFINITE;
        sums[j] += v * v;
      }
    counts[0] += T;
    return st;
  }
  for (int64_t t = 0; t < T; ++t)
    for (int s = 0; s < top_k; ++s) {
      int e = ids[t * top_k + s];
      if (e < 0 || e >= num_experts) { st |= ORC_ST_BADID; continue; }
      counts[e] += 1;
      for (int64_t j = 0; j < K; ++j) {
        double v = (double)x[t * K + j];
        if (!isfinite(v)) st |= ORC_ST_NONFINITE;
        sums[(int64_t)e * K + j] += v * v;
      }
    }
  return st;
}

/* Merging the statistics of two collections ([coverage] Facts: the GGUF
 * imatrix format stores each tensor's in_sum2 and counts so that files can be
 * merged; [2735] "Single rank": statistics of several ranks would be summed).
 * sums[e][j] = sums[e][j] + src_sums[e][j], one fp32 addition; counts[e] +=
 * src_counts[e].  A non-finite source sum of an expert the source touched
 * (src_counts[e] != 0) raises the non-finite bit ([coverage] Facts: only
 * touched experts are checked). */
int orc_merge(const float *src_sums, const int64_t *src_counts, int num_experts, int64_t K, float *sums,
              int64_t *counts) {
  int st = 0;
  for (int e = 0; e < num_experts; ++e) {
    for (int64_t j = 0; j < K; ++j) {
      float v = src_sums[(int64_t)e * K + j];
      if (src_counts[e] != 0 && !isfinite(v)) st |= ORC_ST_NONFINITE;
      sums[(int64_t)e * K + j] = sums[(int64_t)e * K + j] + v;
    }
    counts[e] += src_counts[e];
  }
  return st;
}

/* Hessian blocks for the local-Hessian choice search ([3158]: the layer-output
 * error over the 256-column diagonal blocks of the input Hessian X^T X).
 * hess [E][K/256][256][256] fp64, accumulated in place: for each (t, s) with
 * ids[t][s] == e (dense: every token, E = 1), add x_t,b x_t,b^T to block b. */
int orc_hessian_collect(const float *x, int64_t T, int64_t K, const int32_t *ids, int top_k, int num_experts,
                        double *hess) {
  int st = 0;
  int64_t nb = K / 256;
  for (int64_t t = 0; t < T; ++t) {
    int ns = ids ? top_k : 1;
    for (int s = 0; s < ns; ++s) {
      int e = ids ? ids[t * top_k + s] : 0;
      if (e < 0 || e >= num_experts) { st |= ORC_ST_BADID; continue; }
      for (int64_t b = 0; b < nb; ++b) {
        const float *xb = x + t * K + b * 256;
        double *H = hess + ((int64_t)e * nb + b) * 65536;
        for (int i = 0; i < 256; ++i) {
          if (!isfinite(xb[i])) st |= ORC_ST_NONFINITE;
          for (int j = 0; j < 256; ++j) H[i * 256 + j] += (double)xb[i] * (double)xb[j];
        }
      }
    }
  }
  return st;
}

/* Importance a_j = sqrt(floored E[x_j^2]) per expert  ([2735] "What imatrix
 * does", "Why the square root", "Shared floor"; [coverage] Facts: count 0 ->
 * weight 1 on every channel).  sums are the fp32 statistics.  R6.
 *
 * The floor is floor_rel times the mean of the m_j, taken as the plain mean:
 * the m_j added one after another in fp64, j ascending from 0, the total
 * divided by K in fp64 and rounded to fp32. */
float orc_mean(const float *m, int64_t K) {
  double acc = 0.0;
  for (int64_t j = 0; j < K; ++j) acc += (double)m[j];
  return (float)(acc / (double)K);
}

int orc_importance(const float *sums, const int64_t *counts, int num_experts, int64_t K,
                   float floor_rel, float *imp) {
  int st = 0;
  float *m = (float *)malloc(sizeof(float) * (size_t)K);
  for (int e = 0; e < num_experts; ++e) {
    const float *se = sums + (int64_t)e * K;
    float *ie = imp + (int64_t)e * K;
    int flat = counts[e] <= 0;
    if (!flat) {
      float c = (float)counts[e];
      for (int64_t j = 0; j < K; ++j) {
        m[j] = se[j] / c;
        if (!isfinite(m[j]) || m[j] < 0.0f) { st |= ORC_ST_BADIMP; flat = 1; }
      }
    }
    float mean = flat ? 0.0f : orc_mean(m, K);
    if (flat || mean == 0.0f) { /* idle expert or nothing usable: flat weights */
      for (int64_t j = 0; j < K; ++j) ie[j] = 1.0f;
      continue;
    }
    float fl = floor_rel * mean;
    for (int64_t j = 0; j < K; ++j) ie[j] = sqrtf(fmaxf(m[j], fl));
  }
  free(m);
  return st;
}

/* ------------------------------------------------------------------------- */
/* Super-block scale anchor  ([2513] IQ2_XXS message "fixed anchored         */
/* super-block scale"; IQ1_M body "A scale-anchor correction": IQ1_S flat    */
/* 0.61, IQ1_M clamp(0.58 + 0.035 * peak_to_rms, 0.65, 0.95)).  R1-R5.       */
/* ------------------------------------------------------------------------- */
static float anchor_ratio(int fmt, const float *x, float amax) {
  if (fmt == ORC_IQ1_S) return 0.61f;
  if (fmt == ORC_IQ1_M) {
    float ss = 0.0f;
    for (int j = 0; j < 256; ++j) ss = fmaf(x[j], x[j], ss);
    float rms = sqrtf(ss * (1.0f / 256.0f));
    float p = amax / rms;
    return fminf(fmaxf(fmaf(0.035f, p, 0.58f), 0.65f), 0.95f);
  }
  return 1.0f;
}

/* Returns the fp16 bits of d; 0 means "all-zero block".  *st gets status bits. */
uint16_t orc_anchor(int fmt, const float *x, int *st) {
  float amax = 0.0f;
  for (int j = 0; j < 256; ++j) {
    if (!isfinite(x[j])) { *st |= ORC_ST_NONFINITE; return 0; }
    amax = fmaxf(amax, fabsf(x[j]));
  }
  if (amax == 0.0f) return 0;
  float qmax = is_iq1(fmt) ? 15.0f : 19.375f; /* 15 * 1 ; 3.875 * 5 */
  float r = anchor_ratio(fmt, x, amax);
  float d = (r * amax) / qmax;
  uint16_t h = orc_f32_to_f16(d);
  if ((h & 0x7c00) == 0x7c00) { *st |= ORC_ST_OVERFLOW; return 0; }
  if ((h & 0x7fff) == 0) return 0;
  return h;
}

/* ------------------------------------------------------------------------- */
/* Per-group search                                                          */
/* ------------------------------------------------------------------------- */
/* IQ2 family ([2513] IQ2_XXS and IQ2_S messages: even-parity sign rule for
 * IQ2_XXS/XS with the weakest element flipped; IQ2_S keeps the input signs and
 * compares magnitudes).  For one group of 8 values x with weights a, fill
 * t[c*N + k] = reduced error of entry k under choice c (R12), and flip[k] =
 * the element flipped for entry k (-1 if none).  Local scale of choice c is
 * s_c = d * (2c+1)/8.  */
static void iq2_group(int fmt, const float *x, const float *a, const float *grid, int N,
                      float d, float *t, int *flip) {
  float ax[8], nax[8];
  int neg = 0;
  for (int j = 0; j < 8; ++j) {
    float v = fabsf(x[j]);
    if (x[j] < 0.0f) neg ^= 1;          /* R8: -0 is positive */
    ax[j] = a[j] * v;
    nax[j] = -2.0f * ax[j];
  }
  int odd = (fmt != ORC_IQ2_S) && neg;  /* parity rule only for XXS / XS */
  for (int k = 0; k < N; ++k) {
    const float *g = grid + (int64_t)k * 8;
    float G = 0.0f, P2 = 0.0f;
    for (int j = 0; j < 8; ++j) {
      G = fmaf(a[j], g[j] * g[j], G);   /* sum a_j g_j^2         */
      P2 = fmaf(nax[j], g[j], P2);      /* -2 sum a_j |x_j| g_j  */
    }
    flip[k] = -1;
    if (odd) {                          /* R7: cheapest single flip */
      int jm = 0;
      float F = ax[0] * g[0];
      for (int j = 1; j < 8; ++j) {
        float f = ax[j] * g[j];
        if (f < F) { F = f; jm = j; }
      }
      P2 = fmaf(4.0f, F, P2);           /* -2 (P - 2F) */
      flip[k] = jm;
    }
    for (int c = 0; c < 16; ++c) {
      float s = d * ((float)(2 * c + 1) * 0.125f);
      t[c * N + k] = fmaf(s, G, P2);
    }
  }
}

/* IQ1 family ([2513] IQ1_M body; [recipes] "Shared with IQ1_S rather than
 * copied": per-entry grid terms, then the +-1/8 shift applied).  Values are
 * s * (g + delta_h).  t[(h*8 + ls)*N + k] = reduced error (R12) of entry k with
 * shift h under local scale s_ls = d * (2ls+1).  */
static void iq1_group(const float *x, const float *a, const float *grid, int N, float d,
                      float *t) {
  static const float delta[2] = {0.125f, -0.125f}; /* R10 */
  float nax[8];
  float S2 = 0.0f;
  for (int j = 0; j < 8; ++j) {
    nax[j] = -2.0f * (a[j] * x[j]);
    S2 = S2 + nax[j];                               /* -2 sum a_j x_j */
  }
  for (int k = 0; k < N; ++k) {
    const float *g = grid + (int64_t)k * 8;
    float P2 = 0.0f;
    for (int j = 0; j < 8; ++j) P2 = fmaf(nax[j], g[j], P2); /* -2 sum a_j x_j g_j */
    for (int h = 0; h < 2; ++h) {
      float G = 0.0f;
      for (int j = 0; j < 8; ++j) {
        float u = g[j] + delta[h];
        G = fmaf(a[j], u * u, G);                   /* sum a_j (g_j + delta)^2 */
      }
      float P2h = fmaf(delta[h], S2, P2);           /* -2 sum a_j x_j (g_j + delta) */
      for (int ls = 0; ls < 8; ++ls) {
        float s = d * (float)(2 * ls + 1);
        t[(h * 8 + ls) * N + k] = fmaf(s, G, P2h);
      }
    }
  }
}

/* first minimum over k of row[0..N) (strict <: lower entry wins ties) */
static int first_argmin(const float *row, int N, float *best) {
  int kb = 0;
  float b = row[0];
  for (int k = 1; k < N; ++k)
    if (row[k] < b) { b = row[k]; kb = k; }
  *best = b;
  return kb;
}

/* Decoded fields of one block. */
typedef struct {
  uint16_t d;      /* fp16 bits                           */
  int k[32];       /* grid entry per group                */
  int mask[32];    /* IQ2: 8-bit negative mask per group  */
  int h[32];       /* IQ1: shift per group (1 -> -1/8)    */
  int ls[16];      /* local scale per choice unit         */
} orc_fields;

/* ------------------------------------------------------------------------- */
/* Packing (R13).  Little-endian fields.                                     */
/* ------------------------------------------------------------------------- */
static int parity7(int v) { return __builtin_popcount(v & 0x7f) & 1; }

static void put16(uint8_t *p, unsigned v) { p[0] = v & 0xff; p[1] = (v >> 8) & 0xff; }
static unsigned get16(const uint8_t *p) { return p[0] | (p[1] << 8); }
static void put32(uint8_t *p, uint32_t v) { put16(p, v & 0xffff); put16(p + 2, v >> 16); }
static uint32_t get32(const uint8_t *p) { return get16(p) | ((uint32_t)get16(p + 2) << 16); }

void orc_pack(int fmt, const orc_fields *f, uint8_t *out) {
  memset(out, 0, (size_t)GEOM[fmt].block_bytes);
  switch (fmt) {
  case ORC_IQ2_XXS: /* d | 8 x (4 index bytes, u32: 4 x 7-bit sign index + 4-bit scale) */
    put16(out, f->d);
    for (int ib = 0; ib < 8; ++ib) {
      uint8_t *q = out + 2 + 8 * ib;
      uint32_t w = (uint32_t)f->ls[ib] << 28;
      for (int l = 0; l < 4; ++l) {
        q[l] = (uint8_t)f->k[4 * ib + l];
        w |= (uint32_t)(f->mask[4 * ib + l] & 0x7f) << (7 * l);
      }
      put32(q + 4, w);
    }
    break;
  case ORC_IQ2_XS: /* d | 32 x u16 (9-bit index, 7-bit sign index) | 8 scale bytes */
    put16(out, f->d);
    for (int g = 0; g < 32; ++g) put16(out + 2 + 2 * g, (unsigned)f->k[g] | ((unsigned)(f->mask[g] & 0x7f) << 9));
    for (int ib = 0; ib < 8; ++ib) out[66 + ib] = (uint8_t)(f->ls[2 * ib] | (f->ls[2 * ib + 1] << 4));
    break;
  case ORC_IQ2_S: /* d | 32 low index bytes | 32 sign masks | 8 high-bit bytes | 8 scale bytes */
    put16(out, f->d);
    for (int g = 0; g < 32; ++g) {
      out[2 + g] = (uint8_t)(f->k[g] & 0xff);
      out[34 + g] = (uint8_t)f->mask[g];
      out[66 + g / 4] |= (uint8_t)(((f->k[g] >> 8) & 3) << (2 * (g % 4)));
    }
    for (int ib = 0; ib < 8; ++ib) out[74 + ib] = (uint8_t)(f->ls[2 * ib] | (f->ls[2 * ib + 1] << 4));
    break;
  case ORC_IQ1_S: /* d | 32 low index bytes | 8 x u16 (4 x 3 high bits, 3-bit scale, delta sign) */
    put16(out, f->d);
    for (int g = 0; g < 32; ++g) out[2 + g] = (uint8_t)(f->k[g] & 0xff);
    for (int ib = 0; ib < 8; ++ib) {
      unsigned w = ((unsigned)f->ls[ib] << 12) | ((unsigned)f->h[4 * ib] << 15);
      for (int l = 0; l < 4; ++l) w |= (unsigned)((f->k[4 * ib + l] >> 8) & 7) << (3 * l);
      put16(out + 34 + 2 * ib, w);
    }
    break;
  case ORC_IQ1_M: /* 32 low index bytes | 16 qh bytes | 4 x u16 scale words with d nibbles */
    for (int g = 0; g < 32; ++g) out[g] = (uint8_t)(f->k[g] & 0xff);
    for (int q = 0; q < 16; ++q) {
      unsigned lo = ((f->k[2 * q] >> 8) & 7) | (f->h[2 * q] << 3);
      unsigned hi = ((f->k[2 * q + 1] >> 8) & 7) | (f->h[2 * q + 1] << 3);
      out[32 + q] = (uint8_t)(lo | (hi << 4));
    }
    for (int w = 0; w < 4; ++w) {
      unsigned v = (unsigned)((f->d >> (4 * w)) & 0xf) << 12;
      for (int i = 0; i < 4; ++i) v |= (unsigned)(f->ls[4 * w + i] & 7) << (3 * i);
      put16(out + 48 + 2 * w, v);
    }
    break;
  }
}

void orc_unpack(int fmt, const uint8_t *in, orc_fields *f) {
  memset(f, 0, sizeof *f);
  switch (fmt) {
  case ORC_IQ2_XXS:
    f->d = (uint16_t)get16(in);
    for (int ib = 0; ib < 8; ++ib) {
      const uint8_t *q = in + 2 + 8 * ib;
      uint32_t w = get32(q + 4);
      f->ls[ib] = (int)(w >> 28);
      for (int l = 0; l < 4; ++l) {
        int si = (int)((w >> (7 * l)) & 0x7f);
        f->k[4 * ib + l] = q[l];
        f->mask[4 * ib + l] = si | (parity7(si) << 7);
      }
    }
    break;
  case ORC_IQ2_XS:
    f->d = (uint16_t)get16(in);
    for (int g = 0; g < 32; ++g) {
      unsigned v = get16(in + 2 + 2 * g);
      int si = (int)(v >> 9);
      f->k[g] = (int)(v & 511);
      f->mask[g] = si | (parity7(si) << 7);
    }
    for (int ib = 0; ib < 8; ++ib) { f->ls[2 * ib] = in[66 + ib] & 15; f->ls[2 * ib + 1] = in[66 + ib] >> 4; }
    break;
  case ORC_IQ2_S:
    f->d = (uint16_t)get16(in);
    for (int g = 0; g < 32; ++g) {
      f->k[g] = in[2 + g] | (((in[66 + g / 4] >> (2 * (g % 4))) & 3) << 8);
      f->mask[g] = in[34 + g];
    }
    for (int ib = 0; ib < 8; ++ib) { f->ls[2 * ib] = in[74 + ib] & 15; f->ls[2 * ib + 1] = in[74 + ib] >> 4; }
    break;
  case ORC_IQ1_S:
    f->d = (uint16_t)get16(in);
    for (int ib = 0; ib < 8; ++ib) {
      unsigned w = get16(in + 34 + 2 * ib);
      f->ls[ib] = (int)((w >> 12) & 7);
      for (int l = 0; l < 4; ++l) {
        int g = 4 * ib + l;
        f->k[g] = in[2 + g] | (int)(((w >> (3 * l)) & 7) << 8);
        f->h[g] = (int)(w >> 15);
      }
    }
    break;
  case ORC_IQ1_M: {
    unsigned d = 0;
    for (int w = 0; w < 4; ++w) {
      unsigned v = get16(in + 48 + 2 * w);
      d |= (v >> 12) << (4 * w);
      for (int i = 0; i < 4; ++i) f->ls[4 * w + i] = (int)((v >> (3 * i)) & 7);
    }
    f->d = (uint16_t)d;
    for (int q = 0; q < 16; ++q) {
      int lo = in[32 + q] & 15, hi = in[32 + q] >> 4;
      f->k[2 * q] = in[2 * q] | ((lo & 7) << 8);
      f->h[2 * q] = lo >> 3;
      f->k[2 * q + 1] = in[2 * q + 1] | ((hi & 7) << 8);
      f->h[2 * q + 1] = hi >> 3;
    }
    break;
  }
  }
}

/* Round trip helpers exposed for tests: fields as flat int arrays
 * [d, k[32], mask[32], h[32], ls[16]] (113 ints). */
void orc_pack_flat(int fmt, const int *v, uint8_t *out) {
  orc_fields f;
  f.d = (uint16_t)v[0];
  for (int g = 0; g < 32; ++g) { f.k[g] = v[1 + g]; f.mask[g] = v[33 + g]; f.h[g] = v[65 + g]; }
  for (int u = 0; u < 16; ++u) f.ls[u] = v[97 + u];
  orc_pack(fmt, &f, out);
}

void orc_unpack_flat(int fmt, const uint8_t *in, int *v) {
  orc_fields f;
  orc_unpack(fmt, in, &f);
  v[0] = f.d;
  for (int g = 0; g < 32; ++g) { v[1 + g] = f.k[g]; v[33 + g] = f.mask[g]; v[65 + g] = f.h[g]; }
  for (int u = 0; u < 16; ++u) v[97 + u] = f.ls[u];
}

/* ------------------------------------------------------------------------- */
/* Decoding  ([2513]: decoders validated against llama.cpp's dequantize_row  */
/* semantics; IQ1_M d from the top nibbles of four scale words, one 3-bit    */
/* scale per two groups)                                                     */
/* ------------------------------------------------------------------------- */
void orc_decode_block(int fmt, const uint8_t *in, const float *grid, float *y) {
  orc_fields f;
  orc_unpack(fmt, in, &f);
  float d = orc_f16_to_f32(f.d);
  int gpu = GEOM[fmt].gpu;
  for (int g = 0; g < 32; ++g) {
    int u = g / gpu;
    const float *e = grid + (int64_t)f.k[g] * 8;
    if (is_iq1(fmt)) {
      float s = d * (float)(2 * f.ls[u] + 1);
      float delta = f.h[g] ? -0.125f : 0.125f;
      for (int j = 0; j < 8; ++j) y[8 * g + j] = s * (e[j] + delta);
    } else {
      float s = d * ((float)(2 * f.ls[u] + 1) * 0.125f);
      for (int j = 0; j < 8; ++j) {
        float v = s * e[j];
        y[8 * g + j] = ((f.mask[g] >> j) & 1) ? -v : v;
      }
    }
  }
}

/* ------------------------------------------------------------------------- */
/* One 256-value block: anchor, per-unit choice (searched or fixed), entry   */
/* search under the choice, pack.  ([3157]: one choice per unit by least     */
/* importance-weighted squared error; with fixed choices the scoring sweep   */
/* is skipped and the entry search kept.)                                    */
/* d16_override >= 0 replaces the anchor (used by tests that need an exact   */
/* lattice scale).  chosen (may be NULL) receives each unit's choice (0 for  */
/* an all-zero block).  Returns status bits.                                 */
/* ------------------------------------------------------------------------- */
typedef struct {
  float *t;     /* [16][N] reduced errors of one group */
  int *flip;    /* [N] */
  float *best;  /* [32][16] first-min value per group and slot */
  int *bestk;   /* [32][16] */
} orc_scratch;

static int encode_block(int fmt, const float *x, const float *a, const float *grid, int N,
                        const uint8_t *choices, int d16_override, uint8_t *out, orc_scratch *sc,
                        uint8_t *chosen) {
  const orc_geom *G = &GEOM[fmt];
  int st = 0;
  uint16_t d16;
  int bad_imp = 0;
  for (int j = 0; j < 256; ++j) /* R20: usable weights lie in [0, 2^64] */
    if (!(a[j] >= 0.0f && a[j] <= ORC_IMP_MAX)) bad_imp = 1;
  if (d16_override >= 0) {
    d16 = (uint16_t)d16_override;
    for (int j = 0; j < 256; ++j)
      if (!isfinite(x[j])) { st |= ORC_ST_NONFINITE; d16 = 0; break; }
  } else {
    d16 = orc_anchor(fmt, x, &st);
  }
  if (bad_imp) { st |= ORC_ST_BADIMP; d16 = 0; }
  if (choices)
    for (int u = 0; u < G->units; ++u)
      if (choices[u] >= G->nchoices) { st |= ORC_ST_BADCHOICE; d16 = 0; }
  if (d16 == 0) {
    memset(out, 0, (size_t)G->block_bytes);
    if (chosen) memset(chosen, 0, (size_t)G->units);
    return st;
  }
  float d = orc_f16_to_f32(d16);
  int flips[32][16];

  /* per group: first minimum over entries for each of the 16 slots */
  for (int g = 0; g < 32; ++g) {
    if (is_iq1(fmt)) {
      iq1_group(x + 8 * g, a + 8 * g, grid, N, d, sc->t);
    } else {
      iq2_group(fmt, x + 8 * g, a + 8 * g, grid, N, d, sc->t, sc->flip);
    }
    for (int c = 0; c < 16; ++c) {
      int kb = first_argmin(sc->t + (int64_t)c * N, N, &sc->best[g * 16 + c]);
      sc->bestk[g * 16 + c] = kb;
      flips[g][c] = is_iq1(fmt) ? -1 : sc->flip[kb];
    }
  }

  orc_fields f;
  memset(&f, 0, sizeof f);
  f.d = d16;
  for (int u = 0; u < G->units; ++u) {
    int g0 = u * G->gpu;
    int cu;
    if (choices) {
      cu = choices[u];
    } else { /* R9: unit score = sum over its groups of s_c * best, left to right */
      float bestscore = 0.0f;
      cu = -1;
      for (int c = 0; c < G->nchoices; ++c) {
        float score = 0.0f;
        for (int i = 0; i < G->gpu; ++i) {
          int g = g0 + i;
          float s, b;
          if (fmt == ORC_IQ1_M) {
            float b0 = sc->best[g * 16 + c], b1 = sc->best[g * 16 + 8 + c];
            b = (b1 < b0) ? b1 : b0;    /* tie: lower shift */
            s = d * (float)(2 * c + 1);
          } else if (fmt == ORC_IQ1_S) {
            b = sc->best[g * 16 + c];
            s = d * (float)(2 * (c & 7) + 1);
          } else {
            b = sc->best[g * 16 + c];
            s = d * ((float)(2 * c + 1) * 0.125f);
          }
          float e = s * b;
          score = (i == 0) ? e : score + e;
        }
        if (cu < 0 || score < bestscore) { bestscore = score; cu = c; }
      }
    }
    for (int i = 0; i < G->gpu; ++i) {
      int g = g0 + i;
      int slot = cu;
      if (fmt == ORC_IQ1_M) {
        float b0 = sc->best[g * 16 + cu], b1 = sc->best[g * 16 + 8 + cu];
        slot = (b1 < b0) ? 8 + cu : cu;
      }
      f.k[g] = sc->bestk[g * 16 + slot];
      if (is_iq1(fmt)) {
        f.h[g] = slot >> 3;
      } else {
        int neg = 0;
        for (int j = 0; j < 8; ++j) neg |= (x[8 * g + j] < 0.0f) << j;
        int fj = flips[g][slot];
        f.mask[g] = fj >= 0 ? (neg ^ (1 << fj)) : neg;
      }
    }
    f.ls[u] = (fmt == ORC_IQ1_S) ? (cu & 7) : cu;
    if (chosen) chosen[u] = (uint8_t)cu;
  }
  orc_pack(fmt, &f, out);
  return st;
}

static void scratch_init(orc_scratch *sc, int N) {
  sc->t = (float *)malloc(sizeof(float) * 16 * (size_t)N);
  sc->flip = (int *)malloc(sizeof(int) * (size_t)N);
  sc->best = (float *)malloc(sizeof(float) * 32 * 16);
  sc->bestk = (int *)malloc(sizeof(int) * 32 * 16);
}
static void scratch_free(orc_scratch *sc) { free(sc->t); free(sc->flip); free(sc->best); free(sc->bestk); }

/* One block with an explicit grid size (tests use small hand grids). */
int orc_encode_block(int fmt, const float *x, const float *a, const float *grid, int grid_n,
                     const uint8_t *choices, int d16_override, uint8_t *out) {
  if (fmt < 0 || fmt > 4 || grid_n < 1) return -1;
  orc_scratch sc;
  scratch_init(&sc, grid_n);
  int st = encode_block(fmt, x, a, grid, grid_n, choices, d16_override, out, &sc, NULL);
  scratch_free(&sc);
  return st;
}

/* Per-group slot minima for tests: best[32][16], bestk[32][16]. */
int orc_group_minima(int fmt, const float *x, const float *a, const float *grid, int grid_n,
                     uint16_t d16, float *best, int *bestk) {
  orc_scratch sc;
  scratch_init(&sc, grid_n);
  float d = orc_f16_to_f32(d16);
  for (int g = 0; g < 32; ++g) {
    if (is_iq1(fmt)) iq1_group(x + 8 * g, a + 8 * g, grid, grid_n, d, sc.t);
    else iq2_group(fmt, x + 8 * g, a + 8 * g, grid, grid_n, d, sc.t, sc.flip);
    for (int c = 0; c < 16; ++c)
      bestk[g * 16 + c] = first_argmin(sc.t + (int64_t)c * grid_n, grid_n, &best[g * 16 + c]);
  }
  scratch_free(&sc);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Whole tensor: rows x cols, cols % 256 == 0 ([2735] "Checked up front").   */
/* importance [E, cols] (row r uses expert r / rows_per_expert) or NULL      */
/* (flat).  choices [rows, cols/256, units] or NULL.  Threads split rows.    */
/* ------------------------------------------------------------------------- */
typedef struct {
  int fmt;
  const float *w;
  int64_t rows, cols, rpe;
  const int64_t *row_ids; /* optional: encode only these rows (out is [n, ...]) */
  const float *grid;
  const float *imp;
  const uint8_t *choices;
  uint8_t *out;
  int64_t r0, r1;
  int st;
} orc_job;

static void *quantize_rows(void *p) {
  orc_job *J = (orc_job *)p;
  const orc_geom *G = &GEOM[J->fmt];
  int64_t nb = J->cols / 256;
  orc_scratch sc;
  scratch_init(&sc, G->grid_n);
  float *ones = (float *)malloc(sizeof(float) * 256);
  for (int j = 0; j < 256; ++j) ones[j] = 1.0f;
  for (int64_t i = J->r0; i < J->r1; ++i) {
    int64_t r = J->row_ids ? J->row_ids[i] : i;
    int64_t e = r / J->rpe;
    for (int64_t b = 0; b < nb; ++b) {
      const float *x = J->w + r * J->cols + b * 256;
      const float *a = J->imp ? J->imp + e * J->cols + b * 256 : ones;
      const uint8_t *ch = J->choices ? J->choices + (r * nb + b) * G->units : NULL;
      uint8_t *o = J->out + (i * nb + b) * G->block_bytes;
      J->st |= encode_block(J->fmt, x, a, J->grid, G->grid_n, ch, -1, o, &sc, NULL);
    }
  }
  free(ones);
  scratch_free(&sc);
  return NULL;
}

int orc_quantize(int fmt, const float *w, int64_t rows, int64_t cols, int64_t rows_per_expert,
                 const int64_t *row_ids, int64_t n_rows, const float *grid, const float *imp,
                 const uint8_t *choices, uint8_t *out, int threads) {
  if (fmt < 0 || fmt > 4 || cols % 256 != 0 || rows_per_expert <= 0) return -1;
  int64_t n = row_ids ? n_rows : rows;
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if (threads > n) threads = n > 0 ? (int)n : 1;
  orc_job jobs[256];
  pthread_t th[256];
  for (int i = 0; i < threads; ++i) {
    orc_job *J = &jobs[i];
    J->fmt = fmt; J->w = w; J->rows = rows; J->cols = cols; J->rpe = rows_per_expert;
    J->row_ids = row_ids; J->grid = grid; J->imp = imp; J->choices = choices; J->out = out;
    J->r0 = n * i / threads; J->r1 = n * (i + 1) / threads; J->st = 0;
    pthread_create(&th[i], NULL, quantize_rows, J);
  }
  int st = 0;
  for (int i = 0; i < threads; ++i) { pthread_join(th[i], NULL); st |= jobs[i].st; }
  return st;
}

int orc_dequantize(int fmt, const uint8_t *packed, int64_t rows, int64_t cols, const float *grid,
                   float *y) {
  if (fmt < 0 || fmt > 4 || cols % 256 != 0) return -1;
  int64_t nb = cols / 256;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < nb; ++b)
      orc_decode_block(fmt, packed + (r * nb + b) * GEOM[fmt].block_bytes, grid, y + r * cols + b * 256);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Local-Hessian choice search  ([3158] "local_hessian for GGML IQ": encode    */
/* each block under every choice; give each choice unit its best choice under */
/* its own diagonal Hessian block; revisit the units twice, each taking the   */
/* choice that most lowers the block's error dw H dw^T with the others held;  */
/* Hessian blocks damped by perc_damp, as GPTQ damps).                        */
/*                                                                           */
/* Readings: R16 the damped block is H + lambda I with lambda =              */
/* perc_damp * (sum_j H_jj / 256) (the sum in fp64, ascending j, the mean     */
/* rounded to fp32); R17 dw = w - w^ with w^ the decoder's values; the unit   */
/* error is e = sum_i dw_i (sum_j H_ij dw_j), inner and outer sums fmaf       */
/* chains in ascending index; R18 in the two passes unit u takes the first    */
/* choice minimising f = fmaf(2, dw_u . r_u, e_u) where r_u = sum over the    */
/* other units v of H_uv dw_v at the current picks, gathered unit by unit:    */
/* each unit's contribution is an fmaf chain over its columns (ascending,     */
/* from zero) and the contributions are added in ascending unit order; a pick */
/* takes effect at once (units visited in ascending order).  R21 a block no   */
/* calibration token reached (its Hessian diagonal, each column's sum of      */
/* squares, all zero) keeps the encoder's own choices ([3158] Testing: a      */
/* never-reached weight is encoded plainly).                                  */
/* ------------------------------------------------------------------------- */
static float hd(const float *H, float lam, int i, int j) {
  float v = H[i * 256 + j];
  return i == j ? v + lam : v;
}

float orc_damping(const float *H, float perc_damp) {
  double acc = 0.0;
  for (int j = 0; j < 256; ++j) acc += (double)H[j * 256 + j];
  float mean = (float)(acc / 256.0);
  return perc_damp * mean;
}

/* unit error e = dw_u Hd_uu dw_u^T over columns [c0, c0 + n) */
static float unit_error(const float *H, float lam, const float *dw, int c0, int n) {
  float e = 0.0f;
  for (int i = c0; i < c0 + n; ++i) {
    float y = 0.0f;
    for (int j = c0; j < c0 + n; ++j) y = fmaf(hd(H, lam, i, j), dw[j], y);
    e = fmaf(dw[i], y, e);
  }
  return e;
}

/* choices for one block.  x: 256 weights; a: 256 importance; H: 256x256. */
static int choice_search_block(int fmt, const float *x, const float *a, const float *grid, const float *H,
                               float perc_damp, uint8_t *choices, orc_scratch *sc) {
  const orc_geom *G = &GEOM[fmt];
  const int NC = G->nchoices, U = G->units, UV = 8 * G->gpu;
  float *dwc = (float *)malloc(sizeof(float) * 256 * (size_t)NC);  /* dw under each choice */
  uint8_t blk[128], ch[16];
  float yhat[256];
  int st = 0;
  for (int c = 0; c < NC; ++c) {
    for (int u = 0; u < U; ++u) ch[u] = (uint8_t)c;
    st |= encode_block(fmt, x, a, grid, G->grid_n, ch, -1, blk, sc, NULL);
    orc_decode_block(fmt, blk, grid, yhat);
    for (int j = 0; j < 256; ++j) dwc[c * 256 + j] = x[j] - yhat[j];
  }
  /* R21 ([3158] Testing: a never-reached weight is encoded plainly): a block
   * no calibration token reached -- every column's sum of squares, the
   * Hessian's diagonal, is zero -- keeps the encoder's own choices. */
  int reached = 0;
  for (int j = 0; j < 256; ++j)
    if (H[j * 256 + j] != 0.0f) reached = 1;
  if (!reached) {
    st |= encode_block(fmt, x, a, grid, G->grid_n, NULL, -1, blk, sc, choices);
    free(dwc);
    return st;
  }
  const float lam = orc_damping(H, perc_damp);
  int pick[16];
  float dwcur[256];
  for (int u = 0; u < U; ++u) { /* own block */
    float best = 0.0f;
    pick[u] = 0;
    for (int c = 0; c < NC; ++c) {
      float e = unit_error(H, lam, dwc + c * 256, u * UV, UV);
      if (c == 0 || e < best) { best = e; pick[u] = c; }
    }
    for (int j = u * UV; j < (u + 1) * UV; ++j) dwcur[j] = dwc[pick[u] * 256 + j];
  }
  for (int pass = 0; pass < 2; ++pass) {
    for (int u = 0; u < U; ++u) {
      float r[32];
      for (int i = 0; i < UV; ++i) {
        float acc = 0.0f;
        for (int v = 0; v < U; ++v) {
          if (v == u) continue;
          float part = 0.0f;  /* H_uv dw_v, row i */
          for (int j = v * UV; j < (v + 1) * UV; ++j) part = fmaf(hd(H, lam, u * UV + i, j), dwcur[j], part);
          acc = acc + part;
        }
        r[i] = acc;
      }
      float best = 0.0f;
      int bc = 0;
      for (int c = 0; c < NC; ++c) {
        const float *dw = dwc + c * 256;
        float e = unit_error(H, lam, dw, u * UV, UV);
        float dot = 0.0f;
        for (int i = 0; i < UV; ++i) dot = fmaf(dw[u * UV + i], r[i], dot);
        float f = fmaf(2.0f, dot, e);
        if (c == 0 || f < best) { best = f; bc = c; }
      }
      pick[u] = bc;
      for (int j = u * UV; j < (u + 1) * UV; ++j) dwcur[j] = dwc[bc * 256 + j];
    }
  }
  for (int u = 0; u < U; ++u) choices[u] = (uint8_t)pick[u];
  free(dwc);
  return st;
}

typedef struct {
  int fmt;
  const float *w, *grid, *imp, *hess;
  int64_t rows, cols, rpe;
  const int64_t *row_ids;
  float perc_damp;
  uint8_t *out;
  int64_t r0, r1;
  int st;
} orc_cs_job;

static void *choice_rows(void *p) {
  orc_cs_job *J = (orc_cs_job *)p;
  const orc_geom *G = &GEOM[J->fmt];
  int64_t nb = J->cols / 256;
  orc_scratch sc;
  scratch_init(&sc, G->grid_n);
  float ones[256];
  for (int j = 0; j < 256; ++j) ones[j] = 1.0f;
  for (int64_t i = J->r0; i < J->r1; ++i) {
    int64_t r = J->row_ids ? J->row_ids[i] : i;
    int64_t e = r / J->rpe;
    for (int64_t b = 0; b < nb; ++b) {
      const float *x = J->w + r * J->cols + b * 256;
      const float *a = J->imp ? J->imp + e * J->cols + b * 256 : ones;
      const float *H = J->hess + (e * nb + b) * 65536;
      J->st |= choice_search_block(J->fmt, x, a, J->grid, H, J->perc_damp, J->out + (i * nb + b) * G->units, &sc);
    }
  }
  scratch_free(&sc);
  return NULL;
}

/* choices [n_rows, cols/256, units]; hess [E, cols/256, 256, 256] (row r uses
 * expert r / rows_per_expert); importance as orc_quantize. */
int orc_choice_search(int fmt, const float *w, int64_t rows, int64_t cols, int64_t rows_per_expert,
                      const int64_t *row_ids, int64_t n_rows, const float *grid, const float *imp,
                      const float *hess, float perc_damp, uint8_t *out, int threads) {
  if (fmt < 0 || fmt > 4 || cols % 256 != 0 || rows_per_expert <= 0) return -1;
  int64_t n = row_ids ? n_rows : rows;
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if (threads > n) threads = n > 0 ? (int)n : 1;
  orc_cs_job jobs[256];
  pthread_t th[256];
  for (int i = 0; i < threads; ++i) {
    orc_cs_job *J = &jobs[i];
    J->fmt = fmt; J->w = w; J->grid = grid; J->imp = imp; J->hess = hess;
    J->rows = rows; J->cols = cols; J->rpe = rows_per_expert; J->row_ids = row_ids;
    J->perc_damp = perc_damp; J->out = out;
    J->r0 = n * i / threads; J->r1 = n * (i + 1) / threads; J->st = 0;
    pthread_create(&th[i], NULL, choice_rows, J);
  }
  int st = 0;
  for (int i = 0; i < threads; ++i) { pthread_join(th[i], NULL); st |= jobs[i].st; }
  return st;
}
