/*
 * CPU oracle for causal, packed-document attention on token-block MXFP8 operands
 * (the FLAMIA method: "FLAMIA: FLAsh MIcroscaling Attention for Fast and Causally
 * Safe Training on Blackwell", as reviewed on jaehun.me and summarised on agihunt.info).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call this file: only the
 * tests, the smoke check and the CPU-baseline leg of the benchmark load it.  It shares
 * no code, header, table or constant with the HIP library.
 *
 * Style: plain scalar loops in double precision.  Values are rounded only where the
 * method itself rounds or stores a narrower type:
 *   - operand codes (E4M3, round-to-nearest-even) and block exponents (E8M0),
 *   - the probability and dS operands of the products (E4M3 + E8M0),
 *   - the FP16 dQ accumulator,
 *   - the stored outputs: O, dQ, dK, dV in BF16, LSE and D in FP32.
 * Everything else (scores, softmax, dot products) is computed in double.
 *
 * Where the pages leave a step open, the reading taken is stated next to the code
 * (the same readings are listed in the design notes of the repository).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define E4M3_MAX 448.0
#define BLK 32        /* tokens per scale block (jaehun.me §3.1, MXFP8 path) */
#define KV_TILE 128   /* key tile: running-max update and dQ partial-sum granularity */

/* ------------------------------------------------------------------------------------
 * Number formats
 * ---------------------------------------------------------------------------------- */

/* OCP E4M3 ("FN" variant): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; largest
 * finite value 448 (jaehun.me §2); 0x7F / 0xFF are NaN; no infinity.  Normal values
 * (1 + m/8) * 2^(e-7) for e = 1..15, subnormals (m/8) * 2^-6. */
double orc_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

/* Round a double to the nearest E4M3 value, ties to even.  The sign is kept for results
 * that round to zero.  Magnitudes that round past 448 give NaN (no saturation); the
 * round-up exponent rule below guarantees this never happens for quantised operands. */
uint8_t orc_e4m3_rne(double y) {
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  double a = fabs(y), m;
  int e, E;
  if (isnan(a)) return (uint8_t)(sign | 0x7F);
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: quantum 2^-9 */
    m = nearbyint(ldexp(a, 9));
    return (uint8_t)(sign | (uint8_t)m); /* m == 8 encodes the smallest normal, 2^-6 */
  }
  frexp(a, &e);
  E = e - 1; /* a = 1.f * 2^E, E >= -6 */
  m = nearbyint(ldexp(a, 3 - E)); /* 8 <= m <= 16 */
  if (m == 16.0) { m = 8.0; E += 1; }
  if (E > 8 || (E == 8 && m > 14.0)) return (uint8_t)(sign | 0x7F);
  return (uint8_t)(sign | ((E + 7) << 3) | ((int)m - 8));
}

/* Round-up E8M0 exponent (jaehun.me §3.2; agihunt.info): the smallest integer s such
 * that amax <= 448 * 2^s, so no element of the block exceeds the largest code after
 * scaling.  Clamped to the E8M0 range [-127, 127]; an all-zero block gets -127.
 * Returns 128 (byte 0xFF, the E8M0 NaN) for a NaN or infinite amax. */
int orc_e8m0_roundup(double amax) {
  int e, s;
  if (isnan(amax) || isinf(amax)) return 128;
  if (amax == 0.0) return -127;
  frexp(amax, &e);
  s = e - 9;
  while (amax > ldexp(E4M3_MAX, s)) s++;
  while (amax <= ldexp(E4M3_MAX, s - 1)) s--;
  if (s < -127) s = -127;
  if (s > 127) s = 127;
  return s;
}

/* The OCP reference conversion's exponent (jaehun.me §2): floor(log2 amax) - e_max with
 * e_max = 8 for E4M3.  Kept only as the leaking foil of the worked example; elements
 * above 448 after scaling are clipped to 448. */
int orc_e8m0_floor(double amax) {
  int e, s;
  if (isnan(amax) || isinf(amax)) return 128;
  if (amax == 0.0) return -127;
  frexp(amax, &e); /* amax = f * 2^e, f in [0.5, 1): floor(log2 amax) = e - 1 */
  s = (e - 1) - 8;
  if (s < -127) s = -127;
  if (s > 127) s = 127;
  return s;
}

/* BF16: 8-bit significand, 8-bit exponent; round to nearest even directly from double
 * (a detour through float could round twice). */
uint16_t orc_bf16_rne(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v), m, r;
  int e, q;
  float f;
  uint32_t u;
  if (isnan(v)) return 0x7FC0;
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80);
  frexp(a, &e);
  q = (e - 1 < -126) ? -133 : (e - 1) - 7; /* quantum: 2^-133 below the normal range */
  m = nearbyint(ldexp(a, -q));
  r = ldexp(m, q);
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
  f = (float)r; /* exact */
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

double orc_bf16_decode(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* IEEE binary16, round to nearest even directly from double; overflow gives infinity. */
uint16_t orc_f16_rne(double v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v), m, r;
  int e, q, E;
  if (isnan(v)) return 0x7E00;
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7C00);
  frexp(a, &e);
  q = (e - 1 < -14) ? -24 : (e - 1) - 10;
  m = nearbyint(ldexp(a, -q));
  r = ldexp(m, q);
  if (r >= 65536.0) return (uint16_t)(sign | 0x7C00);
  if (r < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)m); /* subnormal (m == 1024 is 2^-14) */
  frexp(r, &e);
  E = e - 1;
  return (uint16_t)(sign | ((E + 15) << 10) | ((uint16_t)(ldexp(r, 10 - E) - 1024.0)));
}

double orc_f16_decode(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 31) return m ? NAN : (s ? -INFINITY : INFINITY);
  v = (e == 0) ? ldexp((double)m, -24) : ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

/* ------------------------------------------------------------------------------------
 * Token-block quantiser (jaehun.me §3.1, §3.2, §3.4 "Packed documents"; agihunt.info)
 *
 * x: BF16 bit patterns [T][H][d] (contiguous).  For every document k = [cu[k], cu[k+1])
 * and every block b of 32 consecutive tokens counted from the document start (the last
 * block may be shorter), and every head h: amax over the block's tokens and all d
 * channels -> exponent s -> scale byte s + 127 written for each token of the block in
 * scales[h][t] (dense table, one entry per token); codes = E4M3_RNE(x * 2^-s).
 * Tokens outside every document get code 0 and scale byte 0.
 * floor_rule = 1 selects the leaking floor exponent (with clipping) as a test foil.
 * ---------------------------------------------------------------------------------- */
/* The block rule on decoded values v [T][H][d] (double), with blocks of `blk` tokens. */
static void quantize_values(const double* v, int T, int H, int d, const int32_t* cu, int n_docs,
                            uint8_t* codes, uint8_t* scales, int floor_rule, int blk) {
  int k, h, t, c;
  memset(codes, 0, (size_t)T * H * d);
  memset(scales, 0, (size_t)H * T);
  for (k = 0; k < n_docs; ++k) {
    int t_begin = cu[k], t_end = cu[k + 1];
    int t0;
    for (t0 = t_begin; t0 < t_end; t0 += blk) {
      int t1 = t0 + blk < t_end ? t0 + blk : t_end;
      for (h = 0; h < H; ++h) {
        double amax = 0.0;
        int s;
        for (t = t0; t < t1; ++t)
          for (c = 0; c < d; ++c) {
            double a = fabs(v[((size_t)t * H + h) * d + c]);
            if (a > amax || isnan(a)) amax = a;
          }
        s = floor_rule ? orc_e8m0_floor(amax) : orc_e8m0_roundup(amax);
        for (t = t0; t < t1; ++t) {
          scales[(size_t)h * T + t] = (uint8_t)(s + 127);
          for (c = 0; c < d; ++c) {
            double y = ldexp(v[((size_t)t * H + h) * d + c], -s);
            if (floor_rule) {
              if (y > E4M3_MAX) y = E4M3_MAX;
              if (y < -E4M3_MAX) y = -E4M3_MAX;
            }
            codes[((size_t)t * H + h) * d + c] = (s == 128) ? 0x7F : orc_e4m3_rne(y);
          }
        }
      }
    }
  }
}

void orc_quantize(const uint16_t* x, int T, int H, int d, const int32_t* cu, int n_docs,
                  uint8_t* codes, uint8_t* scales, int floor_rule) {
  size_t n = (size_t)T * H * d, i;
  double* v = (double*)malloc((n ? n : 1) * sizeof(double));
  for (i = 0; i < n; ++i) v[i] = orc_bf16_decode(x[i]);
  quantize_values(v, T, H, d, cu, n_docs, codes, scales, floor_rule, BLK);
  free(v);
}

/* Per-token operand scales (jaehun.me §3.2: the precision option that closes the leakage inside
 * a block): the same rule with blocks of one token, so a token's codes and exponent depend on
 * that token alone. */
void orc_quantize_per_token(const uint16_t* x, int T, int H, int d, const int32_t* cu, int n_docs,
                            uint8_t* codes, uint8_t* scales) {
  size_t n = (size_t)T * H * d, i;
  double* v = (double*)malloc((n ? n : 1) * sizeof(double));
  for (i = 0; i < n; ++i) v[i] = orc_bf16_decode(x[i]);
  quantize_values(v, T, H, d, cu, n_docs, codes, scales, 0, 1);
  free(v);
}

/* ------------------------------------------------------------------------------------
 * 4-bit scores (jaehun.me §3.1 "Mixed NVFP4/FP8 path": Q and K stored in a 4-bit format for
 * the score product and its backward recomputation only, one scale per group of head-dimension
 * elements within each token; every other product stays 8-bit).  The pages' format is NVFP4
 * (16-element groups, FP8 scales), an NVIDIA format; the reading taken here is its microscaling
 * analogue, MXFP4: E2M1 codes (OCP: 1 sign, 2 exponent bits with bias 1, 1 mantissa bit;
 * values 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinity or NaN) with one E8M0 exponent per 32
 * consecutive head-dimension elements of one token.  A token's codes and exponents depend on
 * that token alone, so this copy cannot leak across tokens (jaehun.me §3.2).  The exponent is
 * rounded up as for E4M3 (smallest s with amax <= 6 2^s), so no element saturates.
 * ---------------------------------------------------------------------------------- */
#define E2M1_MAX 6.0

void orc_hadamard(float* x, long n_rows, int d);

double orc_e2m1_decode(uint8_t c) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double v = mag[c & 7];
  return (c & 8) ? -v : v;
}

/* Nearest E2M1 value, ties to the even code (mantissa bit 0); the sign is kept for results
 * that round to zero; magnitudes beyond 6 saturate to 6 (the round-up exponent never lets one
 * occur). */
uint8_t orc_e2m1_rne(double y) {
  uint8_t sign = signbit(y) ? 8 : 0, best = 0;
  double a = fabs(y), best_err = INFINITY;
  int c;
  if (a >= E2M1_MAX) return (uint8_t)(sign | 7);
  for (c = 0; c < 8; ++c) {
    double err = fabs(a - orc_e2m1_decode((uint8_t)c));
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best_err = err;
      best = (uint8_t)c;
    }
  }
  return (uint8_t)(sign | best);
}

/* Smallest integer s with amax <= 6 * 2^s, clamped to [-127, 127]; amax = 0 gives -127. */
int orc_e8m0_roundup4(double amax) {
  int e, s;
  if (amax == 0.0) return -127;
  frexp(amax, &e);
  s = e - 3;
  while (amax > ldexp(E2M1_MAX, s)) s++;
  while (amax <= ldexp(E2M1_MAX, s - 1)) s--;
  if (s < -127) s = -127;
  if (s > 127) s = 127;
  return s;
}

/* The 4-bit copy of a tensor.  x: BF16 bit patterns [T][H][d]; for every token of a document
 * and every head, each group of 32 consecutive channels gets exponent s (byte s + 127 at
 * scales[h][t][group], d / 32 bytes per (head, token)) and codes E2M1_RNE(x 2^-s), two per byte,
 * the even channel in the low nibble: codes[t][h][c / 2].  hadamard = 1 rotates each row first,
 * exactly as orc_quantize_hadamard.  Tokens outside every document: codes 0, scale bytes 0. */
void orc_quantize_mx4(const uint16_t* x, int T, int H, int d, const int32_t* cu, int n_docs, int hadamard,
                      uint8_t* codes, uint8_t* scales) {
  size_t n = (size_t)T * H * d, i;
  const int ng = d / 32;
  float* f = (float*)malloc((n ? n : 1) * sizeof(float));
  int k, t, h, gi, c;
  for (i = 0; i < n; ++i) f[i] = (float)orc_bf16_decode(x[i]);
  if (hadamard) orc_hadamard(f, (long)T * H, d);
  memset(codes, 0, n / 2);
  memset(scales, 0, (size_t)H * T * ng);
  for (k = 0; k < n_docs; ++k)
    for (t = cu[k]; t < cu[k + 1]; ++t)
      for (h = 0; h < H; ++h)
        for (gi = 0; gi < ng; ++gi) {
          const float* xs = f + ((size_t)t * H + h) * d + 32 * gi;
          double amax = 0.0;
          int s;
          for (c = 0; c < 32; ++c)
            if (fabs((double)xs[c]) > amax) amax = fabs((double)xs[c]);
          s = orc_e8m0_roundup4(amax);
          scales[((size_t)h * T + t) * ng + gi] = (uint8_t)(s + 127);
          for (c = 0; c < 32; ++c) {
            uint8_t code = orc_e2m1_rne(ldexp((double)xs[c], -s));
            codes[(((size_t)t * H + h) * d + 32 * gi + c) / 2] |= (uint8_t)(code << (4 * (c & 1)));
          }
        }
  free(f);
}

/* Decoded copy of a 4-bit tensor, [T][H][d] in double. */
static double* deq4_all(const uint8_t* codes, const uint8_t* scales, int T, int H, int d) {
  size_t n = (size_t)T * H * d, z;
  const int ng = d / 32;
  double* out = (double*)malloc(sizeof(double) * (n ? n : 1));
  for (z = 0; z < n; ++z) {
    int t = (int)(z / ((size_t)H * d)), h = (int)((z / d) % H), c = (int)(z % d);
    uint8_t code = (uint8_t)((codes[z / 2] >> (4 * (z & 1))) & 15);
    out[z] = ldexp(orc_e2m1_decode(code), (int)scales[((size_t)h * T + t) * ng + c / 32] - 127);
  }
  return out;
}

/* ------------------------------------------------------------------------------------
 * Hadamard rotation of the head dimension (jaehun.me §3.4 "Hadamard rotation", "Quantization
 * fusion"): each row x of d values becomes x H / sqrt(d), H the d x d Sylvester Hadamard
 * matrix (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]), which is symmetric and, normalised,
 * its own inverse.  The pages fix neither the precision nor the order of the arithmetic; the
 * reading taken: FP32 throughout (the inputs are BF16, exact in FP32), the butterflies of the
 * fast transform for strides 1, 2, 4, ..., d/2 in that order, each pair (a, b) at distance
 * `stride` (lower index a) becoming (a + b, a - b) rounded to FP32, then every value multiplied
 * by the FP32 value nearest 1 / sqrt(d) and rounded to FP32.  Each stage's pairs are
 * independent, so the order within a stage does not matter.  Codes are decided on these FP32
 * values, so both sides take that decision in the same precision.
 * ---------------------------------------------------------------------------------- */
void orc_hadamard(float* x, long n_rows, int d) {
  const float c = (float)(1.0 / sqrt((double)d));
  long r;
  for (r = 0; r < n_rows; ++r) {
    float* row = x + (size_t)r * d;
    int stride, i, j;
    for (stride = 1; stride < d; stride *= 2)
      for (i = 0; i < d; i += 2 * stride)
        for (j = i; j < i + stride; ++j) {
          volatile float a = row[j], b = row[j + stride];
          volatile float sum = a + b, diff = a - b;
          row[j] = sum;
          row[j + stride] = diff;
        }
    for (i = 0; i < d; ++i) {
      volatile float y = row[i] * c;
      row[i] = y;
    }
  }
}

/* Quantiser with the rotation: each (token, head) row rotated in FP32, then the block rule
 * on the rotated values. */
void orc_quantize_hadamard(const uint16_t* x, int T, int H, int d, const int32_t* cu, int n_docs,
                           uint8_t* codes, uint8_t* scales) {
  size_t n = (size_t)T * H * d, i;
  float* f = (float*)malloc((n ? n : 1) * sizeof(float));
  double* v = (double*)malloc((n ? n : 1) * sizeof(double));
  for (i = 0; i < n; ++i) f[i] = (float)orc_bf16_decode(x[i]);
  orc_hadamard(f, (long)T * H, d);
  for (i = 0; i < n; ++i) v[i] = (double)f[i];
  quantize_values(v, T, H, d, cu, n_docs, codes, scales, 0, BLK);
  free(f);
  free(v);
}

/* Gradients of rotated operands back to the inputs' basis: dX = dX_rot H / sqrt(d) (the
 * transform is its own inverse), applied to the BF16 gradient rows the backward stores:
 * FP32 rotation as above, then BF16 round-to-nearest-even. */
void orc_unrotate_bf16(const uint16_t* in, uint16_t* out, long n_rows, int d) {
  size_t n = (size_t)n_rows * d, i;
  float* f = (float*)malloc((n ? n : 1) * sizeof(float));
  for (i = 0; i < n; ++i) f[i] = (float)orc_bf16_decode(in[i]);
  orc_hadamard(f, n_rows, d);
  for (i = 0; i < n; ++i) out[i] = orc_bf16_rne((double)f[i]);
  free(f);
}

/* Decoded copy of a whole quantised tensor, [T][H][d] in double (elementwise). */
static double* deq_all(const uint8_t* codes, const uint8_t* scales, int T, int H, int d) {
  size_t n = (size_t)T * H * d, z;
  double* out = (double*)malloc(sizeof(double) * (n ? n : 1));
  for (z = 0; z < n; ++z) {
    int t = (int)(z / ((size_t)H * d)), h = (int)((z / d) % H);
    out[z] = ldexp(orc_e4m3_decode(codes[z]), (int)scales[(size_t)h * T + t] - 127);
  }
  return out;
}

/* Document index of every token (-1 for tokens outside every document). */
static int* doc_map(const int32_t* cu, int n_docs, int T) {
  int* m = (int*)malloc(sizeof(int) * (T ? T : 1));
  int t, k;
  for (t = 0; t < T; ++t) m[t] = -1;
  for (k = 0; k < n_docs; ++k)
    for (t = cu[k]; t < cu[k + 1]; ++t) m[t] = k;
  return m;
}

/* ------------------------------------------------------------------------------------
 * Work lists (jaehun.me §3.4 "Work scheduling"; agihunt.info)
 *
 * kind 0 (forward): one item per 256 consecutive queries of a document, counted from
 *   the document start; cost = number of 128-key blocks the item visits, which for a
 *   causal item b is ceil(min(256(b+1), L) / 128).
 * kind 1 (backward): one item per 128-key tile kappa of a document; cost = number of
 *   128-query tiles at or after the key tile, ceil((L - 128 kappa) / 128).
 * Items are enumerated document by document, block by block, then sorted by descending
 * cost; among items of equal cost, those of documents longer than ORC_SMALL_DOC tokens come
 * first and those of shorter documents (always a single item of cost 1) last, each kept in
 * enumeration order (the pages fix no order among equal costs; this one puts the short
 * documents, which a pass of their own can take, at the end of the list).  `worker` tags the
 * items in alternating (serpentine) directions across n_workers.  Output: 4 ints per item
 * {doc, blk, cost, worker}.  Returns the item count, or -1 if cap is too small.
 * ---------------------------------------------------------------------------------- */
/* Schedule of a list (jaehun.me §3.4 "Work scheduling"): non-causal calls take their units
 * dynamically when the longest document is at least 4 times the average document length, the
 * average taken over the call's n_docs documents (empty ones included); longest * n_docs >=
 * 4 * (total length) in integers.  Causal lists: 0 here (the forward walks them statically; the
 * backward takes its units dynamically whatever the flag).  Returns 1 for dynamic, else 0. */
int orc_schedule_dynamic(const int32_t* cu, int n_docs, int kind) {
  long long longest = 0, total = 0;
  int k;
  if (kind < 2 || n_docs <= 0) return 0;
  for (k = 0; k < n_docs; ++k) {
    const long long L = (long long)cu[k + 1] - cu[k];
    if (L > longest) longest = L;
    total += L;
  }
  return total > 0 && longest * n_docs >= 4 * total;
}

#define ORC_SMALL_DOC 8

/* Number of documents of 1 .. ORC_SMALL_DOC tokens: the items at the end of every list. */
int orc_small_docs(const int32_t* cu, int n_docs) {
  int k, n = 0;
  for (k = 0; k < n_docs; ++k) {
    const int L = cu[k + 1] - cu[k];
    if (L >= 1 && L <= ORC_SMALL_DOC) n++;
  }
  return n;
}

/* items while sorting: {doc, blk, cost, enumeration index, small document (0 or 1)} */
static int cmp_items(const void* a, const void* b) {
  const int32_t* x = (const int32_t*)a;
  const int32_t* y = (const int32_t*)b;
  if (x[2] != y[2]) return x[2] > y[2] ? -1 : 1; /* cost descending */
  if (x[4] != y[4]) return x[4] < y[4] ? -1 : 1; /* longer documents first */
  return x[3] < y[3] ? -1 : (x[3] > y[3]); /* then enumeration order */
}

int orc_worklist(const int32_t* cu, int n_docs, int kind, int n_workers, int32_t* out, int cap) {
  int k, n = 0, i;
  int32_t* tmp;
  for (k = 0; k < n_docs; ++k) {
    int L = cu[k + 1] - cu[k];
    n += (kind % 2 == 0) ? (L + 255) / 256 : (L + 127) / 128;
  }
  if (n > cap) return -1;
  tmp = (int32_t*)malloc(sizeof(int32_t) * 5 * (n > 0 ? n : 1));
  n = 0;
  for (k = 0; k < n_docs; ++k) {
    int L = cu[k + 1] - cu[k], b;
    int nb = (kind % 2 == 0) ? (L + 255) / 256 : (L + 127) / 128;
    for (b = 0; b < nb; ++b) {
      int cost;
      if (kind >= 2) {
        cost = (L + 127) / 128; /* non-causal: every item visits / serves all key or query tiles */
      } else if (kind == 0) {
        int hi = 256 * (b + 1) < L ? 256 * (b + 1) : L;
        cost = (hi + 127) / 128;
      } else {
        cost = (L - 128 * b + 127) / 128;
      }
      tmp[5 * n + 0] = k;
      tmp[5 * n + 1] = b;
      tmp[5 * n + 2] = cost;
      tmp[5 * n + 3] = n; /* enumeration index, for the stable tie-break */
      tmp[5 * n + 4] = L <= ORC_SMALL_DOC;
      n++;
    }
  }
  qsort(tmp, (size_t)n, sizeof(int32_t) * 5, cmp_items);
  for (i = 0; i < n; ++i) {
    int r = i / n_workers, w = i % n_workers;
    out[4 * i + 0] = tmp[5 * i + 0];
    out[4 * i + 1] = tmp[5 * i + 1];
    out[4 * i + 2] = tmp[5 * i + 2];
    out[4 * i + 3] = (r % 2 == 0) ? w : n_workers - 1 - w;
  }
  free(tmp);
  return n;
}

/* ------------------------------------------------------------------------------------
 * Intermediate dumps (test infrastructure): the forward and backward below can copy the
 * per-pair values they form into caller arrays laid out [heads][rows][keys] over a window of
 * query heads, absolute rows and absolute keys, so that the tests can compare decisions one by
 * one and replay the products from given decisions (orc_fwd_replay, orc_bwd_replay).  Only
 * visible pairs (same document, key <= row) are written.  NULL arrays are skipped.
 * ---------------------------------------------------------------------------------- */
typedef struct {
  int row_lo, row_hi, key_lo, key_hi, head_lo, head_hi;
  double* fwd_s;   /* forward: score accumulator sum_c deq(Q_ic) deq(K_jc) */
  double* fwd_m;   /* forward: running maximum (score units) the pair's probability used */
  uint8_t* fwd_p;  /* forward: E4M3 code of 2^p_shift 2^(t - m) */
  double* bwd_dp;  /* backward: D_i - dP_ij */
  uint8_t* bwd_p;  /* backward: Phat code and block exponent byte */
  uint8_t* bwd_ps;
  uint8_t* bwd_ds; /* backward: dShat code and block exponent byte */
  uint8_t* bwd_dss;
  uint8_t* fwd_ps; /* forward, 4-bit scores: exponent byte of the probability code's 32-key group */
} orc_window;

static long long win_index(const orc_window* w, int h, int row, int key) {
  if (!w || h < w->head_lo || h >= w->head_hi || row < w->row_lo || row >= w->row_hi || key < w->key_lo ||
      key >= w->key_hi)
    return -1;
  return ((long long)(h - w->head_lo) * (w->row_hi - w->row_lo) + (row - w->row_lo)) * (w->key_hi - w->key_lo) +
         (key - w->key_lo);
}

/* ------------------------------------------------------------------------------------
 * Forward (jaehun.me §1.2 and §3.1; online softmax of the FlashAttention family)
 *
 * Scores in the base-2 domain: t_ij = softmax_scale * log2(e) * sum_c deq(Q_ic) deq(K_jc)
 * (row and column scale factors sit outside the code dot product, jaehun.me §3.1).
 * For each query row i of a document (offset r), key tiles kappa = floor(r/128) down to 0
 * are visited (tiles counted from the document start; the diagonal tile first).  Per tile:
 *   m' = max(m, max_j t_ij);  alpha = 2^(m - m');  p_j = 2^(t_ij - m');  l = alpha l + sum p_j;
 *   Phat_j = E4M3_RNE(2^p_shift p_j);  acc = alpha acc + 2^-p_shift sum_j Phat_j deq(V_j).
 * O_i = BF16(acc / l), LSE_i = FP32(m + log2 l).  Rows outside every document: O = 0,
 * LSE = +inf.  exact_p = 1 skips the Phat rounding (used by the exact-arithmetic pins).
 * o64 (optional) receives acc / l in double.  GQA: query head h reads KV head
 * h / (Hq / Hkv).  sel_docs / sel_kv (optional, one byte per document / KV head): rows of
 * unselected documents or heads are skipped and their outputs left as they were (lets the
 * tests sample large calls).
 * tail_rows > 0 (a work restriction for sampling long documents, no change to what is
 * computed): only the last tail_rows rows of each document are computed; the outputs of the
 * other rows are left as they were.  win (optional): intermediate dumps, see orc_window.
 * ---------------------------------------------------------------------------------- */
/* Precision option (jaehun.me §3.2: per-token operand scales; the V scale folded into the
 * probability operand of P V, since a per-token scale cannot be applied to one 32-key block of
 * the product).  Reading taken: the probability operand of row i in a key tile is
 * E4M3(2^(P_SHIFT + e(V_j) - v_i) p_ij) with operand scale 2^(v_i - P_SHIFT), v_i the largest
 * V exponent among the keys row i has visited so far (this tile included; the first tile is the
 * diagonal one, so only keys j <= i count), at least -119 so the scale stays an E8M0 byte.
 * Every factor depends on row i and its visible keys alone. */
static int fold_ref(const uint8_t* sv_doc, int j0, int j1, int ref) {
  int j;
  if (ref < -119) ref = -119;
  for (j = j0; j < j1; ++j)
    if ((int)sv_doc[j] - 127 > ref) ref = (int)sv_doc[j] - 127;
  return ref;
}

void orc_fwd(const uint8_t* q, const uint8_t* sq, const uint8_t* k, const uint8_t* sk,
             const uint8_t* v, const uint8_t* sv, int T, int Hq, int Hkv, int d,
             double softmax_scale, const int32_t* cu, int n_docs, int p_shift, int exact_p,
             uint16_t* o, float* lse, double* o64, const uint8_t* sel_docs, const uint8_t* sel_kv,
             int tail_rows, const orc_window* win, int causal, int precise,
             const uint8_t* q4, const uint8_t* sq4, const uint8_t* k4, const uint8_t* sk4) {
  const int group = Hq / Hkv;
  const double c_scale = softmax_scale * 1.4426950408889634074; /* log2(e) */
  /* 4-bit scores (q4 given): the score product takes the 4-bit copies of Q and K */
  const int qk4 = q4 != NULL;
  double* Qd = qk4 ? deq4_all(q4, sq4, T, Hq, d) : deq_all(q, sq, T, Hq, d);
  double* Kd = qk4 ? deq4_all(k4, sk4, T, Hkv, d) : deq_all(k, sk, T, Hkv, d);
  double* Vd = deq_all(v, sv, T, Hkv, d);
  int* dm = doc_map(cu, n_docs, T);
  long long task, n_tasks = (long long)T * Hq;
#pragma omp parallel for schedule(dynamic, 64)
  for (task = 0; task < n_tasks; ++task) {
    int row = (int)(task / Hq), hh = (int)(task % Hq), g = hh / group;
    int doc = dm[row], kappa, j, cc;
    double m = -INFINITY, l = 0.0;
    double acc[256];
    double t_tile[KV_TILE], dot_tile[KV_TILE];
    int vref = -1000; /* precise: running maximum of the visible keys' V exponents */
    const double* qi = Qd + ((size_t)row * Hq + hh) * d;
    if (doc < 0) {
      lse[(size_t)hh * T + row] = INFINITY;
      for (cc = 0; cc < d; ++cc) {
        o[((size_t)row * Hq + hh) * d + cc] = 0;
        if (o64) o64[((size_t)row * Hq + hh) * d + cc] = 0.0;
      }
      continue;
    }
    if ((sel_docs && !sel_docs[doc]) || (sel_kv && !sel_kv[g])) continue;
    if (tail_rows > 0 && row < cu[doc + 1] - tail_rows) continue;
    for (cc = 0; cc < d; ++cc) acc[cc] = 0.0;
    {
      int start = cu[doc], r = row - start, L = cu[doc + 1] - start;
      for (kappa = (causal ? r : L - 1) / KV_TILE; kappa >= 0; --kappa) {
        int j0 = kappa * KV_TILE, j1 = (kappa + 1) * KV_TILE;
        double mt = -INFINITY, m_new, alpha, sum = 0.0;
        if (causal && j1 > r + 1) j1 = r + 1; /* causal: keys j <= i only */
        if (j1 > L) j1 = L;
        for (j = j0; j < j1; ++j) {
          const double* kj = Kd + ((size_t)(start + j) * Hkv + g) * d;
          double dot = 0.0;
          for (cc = 0; cc < d; ++cc) dot += qi[cc] * kj[cc];
          dot_tile[j - j0] = dot;
          t_tile[j - j0] = dot * c_scale;
          if (t_tile[j - j0] > mt) mt = t_tile[j - j0];
        }
        m_new = m > mt ? m : mt;
        alpha = (m == -INFINITY) ? 0.0 : exp2(m - m_new);
        for (cc = 0; cc < d; ++cc) acc[cc] *= alpha;
        if (precise) vref = fold_ref(sv + (size_t)g * T + start, j0, j1, vref);
        /* 4-bit scores: the probability operand is quantised in the log domain (jaehun.me §3.4
         * "Softmax throughput"): one exponent per 32-key group of the tile (keys counted from the
         * document start), the round-up exponent of the group's largest probability, found from
         * the group's largest score before any exponential (max_j 2^x_j = 2^max_j x_j); its
         * codes are E4M3(p 2^-e) with operand scale 2^e.  Reading taken: the group holds the
         * row's visible keys of those 32. */
        int e_grp[KV_TILE / 32];
        if (qk4)
          for (j = 0; j < KV_TILE / 32; ++j) {
            int jj, g0 = j0 + 32 * j, g1 = g0 + 32 < j1 ? g0 + 32 : j1;
            double gmax = -INFINITY;
            for (jj = g0; jj < g1; ++jj)
              if (t_tile[jj - j0] > gmax) gmax = t_tile[jj - j0];
            e_grp[j] = g1 > g0 ? orc_e8m0_roundup(exp2(gmax - m_new)) : -127;
          }
        for (j = j0; j < j1; ++j) {
          const double* vj = Vd + ((size_t)(start + j) * Hkv + g) * d;
          double p = exp2(t_tile[j - j0] - m_new);
          /* precise: V's exponent folded into the probability operand (relative to vref) */
          const int fold = precise ? (int)sv[(size_t)g * T + start + j] - 127 - vref : 0;
          /* the operand's exponent: -p_shift - fold, or the 4-bit path's group exponent */
          const int pe = qk4 ? e_grp[(j - j0) / 32] : -p_shift - fold;
          const uint8_t code = orc_e4m3_rne(ldexp(p, -pe));
          double ph = exact_p ? p : ldexp(orc_e4m3_decode(code), pe);
          long long wi = win_index(win, hh, row, start + j);
          if (wi >= 0) {
            if (win->fwd_s) win->fwd_s[wi] = dot_tile[j - j0];
            if (win->fwd_m) win->fwd_m[wi] = m_new;
            if (win->fwd_p) win->fwd_p[wi] = code;
            if (qk4 && win->fwd_ps) win->fwd_ps[wi] = (uint8_t)(pe + 127);
          }
          sum += p;
          for (cc = 0; cc < d; ++cc) acc[cc] += ph * vj[cc];
        }
        l = alpha * l + sum;
        m = m_new;
      }
      for (cc = 0; cc < d; ++cc) {
        o[((size_t)row * Hq + hh) * d + cc] = orc_bf16_rne(acc[cc] / l);
        if (o64) o64[((size_t)row * Hq + hh) * d + cc] = acc[cc] / l;
      }
      lse[(size_t)hh * T + row] = (float)(m + log2(l));
    }
  }
  free(Qd); free(Kd); free(Vd); free(dm);
}

/* ------------------------------------------------------------------------------------
 * dO quantiser and D (jaehun.me §3.3): dO is quantised by the same token-block rule as
 * the inputs, and D_i = sum_c deq(dO_ic) * O_ic uses that same quantised dO (the one the
 * backward's dP product reads) and the stored BF16 output O.  D is stored in FP32;
 * rows outside every document get D = 0.
 * ---------------------------------------------------------------------------------- */
void orc_quantize_do_ex(const uint16_t* dO, const uint16_t* O, int T, int H, int d, const int32_t* cu,
                        int n_docs, uint8_t* codes, uint8_t* scales, float* D, int per_token) {
  int i, h, c;
  int* dm;
  double* dOd;
  if (per_token) orc_quantize_per_token(dO, T, H, d, cu, n_docs, codes, scales);
  else orc_quantize(dO, T, H, d, cu, n_docs, codes, scales, 0);
  dm = doc_map(cu, n_docs, T);
  dOd = deq_all(codes, scales, T, H, d);
  for (i = 0; i < T; ++i)
    for (h = 0; h < H; ++h) {
      double s = 0.0;
      if (dm[i] >= 0)
        for (c = 0; c < d; ++c)
          s += dOd[((size_t)i * H + h) * d + c] * orc_bf16_decode(O[((size_t)i * H + h) * d + c]);
      D[(size_t)h * T + i] = (float)s;
    }
  free(dm);
  free(dOd);
}

void orc_quantize_do(const uint16_t* dO, const uint16_t* O, int T, int H, int d,
                     const int32_t* cu, int n_docs, uint8_t* codes, uint8_t* scales, float* D) {
  orc_quantize_do_ex(dO, O, T, H, d, cu, n_docs, codes, scales, D, 0);
}

/* ------------------------------------------------------------------------------------
 * dQ prescale exponent pi (jaehun.me §3.2 "Accumulator leakage", §3.4 "Backward pass")
 *
 * dQ partial sums are accumulated in FP16 after multiplication by 2^pi.  The pages give
 * only the ingredients (dO, V and K magnitudes; sequence-wide by default, visible keys
 * only with the causal option).  Reading: with C_d the smallest integer such that
 * 2 d 448^3 <= 2^C_d, any partial sum of row i is at most 2^(C_d + E_i) with
 * E_i = e(dO_i) + max e(V) + max e(K) over the relevant keys, so pi_i = 15 - C_d - E_i
 * keeps every partial and the running sum below 2^15 < 65504.
 *   default (causal_dq = 0): maxima over every token of the call, per query head;
 *                            e(dO) also the maximum over the call;
 *   causal  (causal_dq = 1): e(dO_i) of the row's own block, maxima of e(V), e(K) over the
 *                            blocks of the row's document up to and including the
 *                            row's own block.
 * pi is clamped to [-64, 64].  Output pi[h][t]; rows outside documents get 0.
 * ---------------------------------------------------------------------------------- */
static int cd_const(int d) {
  double bound = 2.0 * d * E4M3_MAX * E4M3_MAX * E4M3_MAX;
  int C = 0;
  while (ldexp(1.0, C) < bound) C++;
  return C;
}

void orc_dq_exponents(const uint8_t* sk, const uint8_t* sv, const uint8_t* sdo, int T, int Hq, int Hkv,
                      int d, const int32_t* cu, int n_docs, int causal_dq, int16_t* pi) {
  const int group = Hq / Hkv, C = cd_const(d);
  int h, kk, t;
  memset(pi, 0, sizeof(int16_t) * (size_t)Hq * T);
  for (h = 0; h < Hq; ++h) {
    int g = h / group;
    int max_do = -1000, max_v = -1000, max_k = -1000;
    for (kk = 0; kk < n_docs; ++kk)
      for (t = cu[kk]; t < cu[kk + 1]; ++t) {
        int edo = (int)sdo[(size_t)h * T + t] - 127, ev = (int)sv[(size_t)g * T + t] - 127,
            ek = (int)sk[(size_t)g * T + t] - 127;
        if (edo > max_do) max_do = edo;
        if (ev > max_v) max_v = ev;
        if (ek > max_k) max_k = ek;
      }
    for (kk = 0; kk < n_docs; ++kk)
      for (t = cu[kk]; t < cu[kk + 1]; ++t) {
        int E, p;
        if (!causal_dq) {
          E = max_do + max_v + max_k;
        } else {
          /* causal_dq = 1: maxima up to the row's block end; 2 (per-token scales): up to the row */
          int r = t - cu[kk];
          int block_end = causal_dq == 2 ? t + 1 : cu[kk] + (r / BLK + 1) * BLK;
          int pv = -1000, pk = -1000, u;
          if (block_end > cu[kk + 1]) block_end = cu[kk + 1];
          for (u = cu[kk]; u < block_end; ++u) {
            int ev = (int)sv[(size_t)g * T + u] - 127, ek = (int)sk[(size_t)g * T + u] - 127;
            if (ev > pv) pv = ev;
            if (ek > pk) pk = ek;
          }
          E = ((int)sdo[(size_t)h * T + t] - 127) + pv + pk;
        }
        p = 15 - C - E;
        if (p < -64) p = -64;
        if (p > 64) p = 64;
        pi[(size_t)h * T + t] = (int16_t)p;
      }
  }
}

/* ------------------------------------------------------------------------------------
 * Backward (jaehun.me §1.2, §3.1, §3.3; agihunt.info)
 *
 * For visible pairs (j <= i, same document):
 *   t_ij as in the forward;  P_ij = 2^(t_ij - LSE_i) with the stored FP32 LSE;
 *   dP_ij = sum_c deq(dO_ic) deq(V_jc);  dS_ij = P_ij (dP_ij - D_i) with the stored FP32 D.
 * Operands of the gradient products: P and dS are each quantised to E4M3 with one
 * round-up E8M0 exponent per 32x32 block (query block x key block, both counted from the
 * document start; invisible entries count as zero in the block maximum).
 *   dV_j = sum_{h in group} sum_i deq(Phat_ij) deq(dO_i)
 *   dK_j = softmax_scale sum_{h in group} sum_i deq(dShat_ij) deq(Q_i)
 *   dQ_i: for key tiles kappa ascending, part = sum_{j in kappa} deq(dShat_ij) deq(K_j),
 *         acc16 = FP16(acc16 + FP16(part 2^pi_i));  dQ_i = BF16(softmax_scale acc16 2^-pi_i).
 * exact bits: 1 = no Phat rounding, 2 = no dShat rounding, 4 = FP64 instead of the FP16
 * accumulator (with pi still applied and removed).  Outputs are BF16; d?64 (optional)
 * receive the values before the final BF16 rounding.  dbg_* (optional, single-document
 * calls only) receive the P and dS block exponent bytes [Hq][nb][nb] and codes
 * [Hq][L][L] (0 for invisible entries).  sel_docs / sel_kv as in the forward: unselected
 * (document, KV head) pairs are skipped and their gradient rows stay zero; pi is always
 * computed for the whole call.
 * tail_blocks > 0 (a work restriction for sampling long documents, no change to what is
 * computed): only the last tail_blocks 32-query blocks of each document are visited.  dQ of
 * those rows is then complete (every key block up to theirs is visited), and so are dK and dV
 * of the keys in those blocks (only queries at or after a key see it); the gradients of earlier
 * keys hold partial sums and must not be read.
 * ---------------------------------------------------------------------------------- */
typedef struct {
  uint8_t* p_scale;
  uint8_t* ds_scale;
  uint8_t* p_code;
  uint8_t* ds_code;
} orc_bwd_debug;

void orc_bwd(const uint8_t* q, const uint8_t* sq, const uint8_t* k, const uint8_t* sk,
             const uint8_t* v, const uint8_t* sv, const uint8_t* dO, const uint8_t* sdo,
             const float* lse, const float* D, int T, int Hq, int Hkv, int d,
             double softmax_scale, const int32_t* cu, int n_docs, int causal_dq, int exact,
             uint16_t* dq, uint16_t* dk, uint16_t* dv, int16_t* pi_out,
             double* dq64, double* dk64, double* dv64, const orc_bwd_debug* dbg,
             const uint8_t* sel_docs, const uint8_t* sel_kv, int tail_blocks, const orc_window* win,
             int causal, int precise,
             const uint8_t* q4, const uint8_t* sq4, const uint8_t* k4, const uint8_t* sk4) {
  const int group = Hq / Hkv;
  const double c_scale = softmax_scale * 1.4426950408889634074;
  int16_t* pi = (int16_t*)malloc(sizeof(int16_t) * (size_t)Hq * T + 2);
  long long task, n_tasks = (long long)n_docs * Hkv;
  size_t n_q = (size_t)T * Hq * d, n_kv = (size_t)T * Hkv * d, z;
  double* Qd = deq_all(q, sq, T, Hq, d);
  double* Kd = deq_all(k, sk, T, Hkv, d);
  double* Vd = deq_all(v, sv, T, Hkv, d);
  double* dOd = deq_all(dO, sdo, T, Hq, d);
  /* 4-bit scores: the recomputed score takes the forward's 4-bit copies; dK and dQ keep the
   * 8-bit ones */
  double* Qs = q4 ? deq4_all(q4, sq4, T, Hq, d) : Qd;
  double* Ks = q4 ? deq4_all(k4, sk4, T, Hkv, d) : Kd;
  orc_dq_exponents(sk, sv, sdo, T, Hq, Hkv, d, cu, n_docs, precise ? 2 : causal_dq, pi);
  if (pi_out) memcpy(pi_out, pi, sizeof(int16_t) * (size_t)Hq * T);
  for (z = 0; z < n_q; ++z) { dq[z] = 0; if (dq64) dq64[z] = 0.0; }
  for (z = 0; z < n_kv; ++z) {
    dk[z] = 0; dv[z] = 0;
    if (dk64) dk64[z] = 0.0;
    if (dv64) dv64[z] = 0.0;
  }

#pragma omp parallel for schedule(dynamic, 1)
  for (task = 0; task < n_tasks; ++task) {
    int doc = (int)(task / Hkv), g = (int)(task % Hkv);
    int start = cu[doc], L = cu[doc + 1] - start;
    int nb = (L + BLK - 1) / BLK, hq, bq, bk, ii, jj, cc;
    double* dk_acc;
    double* dv_acc;
    double P[BLK][BLK], dS[BLK][BLK], dPv[BLK][BLK], dSq[BLK][BLK];
    uint8_t Pc[BLK][BLK], dSc[BLK][BLK];
    double part[BLK * 256];
    double acc16[BLK * 256];
    if (L <= 0) continue;
    if ((sel_docs && !sel_docs[doc]) || (sel_kv && !sel_kv[g])) continue;
    dk_acc = (double*)calloc((size_t)L * d, sizeof(double));
    dv_acc = (double*)calloc((size_t)L * d, sizeof(double));
    for (hq = g * group; hq < (g + 1) * group; ++hq) {
      for (bq = (tail_blocks > 0 && nb > tail_blocks) ? nb - tail_blocks : 0; bq < nb; ++bq) {
        int i0 = bq * BLK, i1 = i0 + BLK < L ? i0 + BLK : L;
        int kappa, kappa_last = (causal ? i1 - 1 : L - 1) / KV_TILE;
        for (z = 0; z < (size_t)BLK * d; ++z) acc16[z] = 0.0;
        for (kappa = 0; kappa <= kappa_last; ++kappa) {
          for (z = 0; z < (size_t)BLK * d; ++z) part[z] = 0.0;
          for (bk = kappa * (KV_TILE / BLK); bk < (kappa + 1) * (KV_TILE / BLK) && bk < nb && (!causal || bk <= bq);
               ++bk) {
            int j0 = bk * BLK, j1 = j0 + BLK < L ? j0 + BLK : L;
            double pmax = 0.0, dsmax = 0.0;
            int sp, sds;
            /* P, dP, dS on the 32x32 block */
            for (ii = i0; ii < i1; ++ii)
              for (jj = j0; jj < j1; ++jj) {
                double dot = 0.0, dp = 0.0, p;
                if (causal && jj > ii) { P[ii - i0][jj - j0] = 0.0; dS[ii - i0][jj - j0] = 0.0; continue; }
                const double* qi = Qs + ((size_t)(start + ii) * Hq + hq) * d;
                const double* doi = dOd + ((size_t)(start + ii) * Hq + hq) * d;
                const double* kj = Ks + ((size_t)(start + jj) * Hkv + g) * d;
                const double* vj = Vd + ((size_t)(start + jj) * Hkv + g) * d;
                for (cc = 0; cc < d; ++cc) {
                  dot += qi[cc] * kj[cc];
                  dp += doi[cc] * vj[cc];
                }
                p = exp2(dot * c_scale - (double)lse[(size_t)hq * T + start + ii]);
                dPv[ii - i0][jj - j0] = dp;
                dS[ii - i0][jj - j0] = p * (dp - (double)D[(size_t)hq * T + start + ii]);
                if (precise) {
                  /* per-token scales: each gradient product's other operand loses its exponent,
                   * which moves into P or dS here: dO's into P (for dV), Q's into dS (for dK),
                   * K's into the dS of dQ (the K fold) */
                  const int edo = (int)sdo[(size_t)hq * T + start + ii] - 127;
                  const int eq = (int)sq[(size_t)hq * T + start + ii] - 127;
                  const int ek = (int)sk[(size_t)g * T + start + jj] - 127;
                  dSq[ii - i0][jj - j0] = ldexp(dS[ii - i0][jj - j0], ek);
                  p = ldexp(p, edo);
                  dS[ii - i0][jj - j0] = ldexp(dS[ii - i0][jj - j0], eq);
                }
                P[ii - i0][jj - j0] = p;
                if (fabs(p) > pmax) pmax = fabs(p);
                if (fabs(dS[ii - i0][jj - j0]) > dsmax) dsmax = fabs(dS[ii - i0][jj - j0]);
              }
            /* block quantisation of the two product operands */
            sp = orc_e8m0_roundup(pmax);
            sds = orc_e8m0_roundup(dsmax);
            if (precise) {
              /* the dS operand of dQ: one exponent per (query row, 32-key block), so no other row's
               * values enter a row's rounding (query-row-wise dS exponents) */
              for (ii = i0; ii < i1; ++ii) {
                double rmax = 0.0;
                int sr;
                for (jj = j0; jj < j1 && (!causal || jj <= ii); ++jj)
                  if (fabs(dSq[ii - i0][jj - j0]) > rmax) rmax = fabs(dSq[ii - i0][jj - j0]);
                sr = orc_e8m0_roundup(rmax);
                for (jj = j0; jj < j1; ++jj) {
                  if (causal && jj > ii) { dSq[ii - i0][jj - j0] = 0.0; continue; }
                  if (!(exact & 2)) dSq[ii - i0][jj - j0] = ldexp(orc_e4m3_decode(orc_e4m3_rne(ldexp(dSq[ii - i0][jj - j0], -sr))), sr);
                }
              }
            }
            for (ii = i0; ii < i1; ++ii)
              for (jj = j0; jj < j1; ++jj) {
                if (causal && jj > ii) { Pc[ii - i0][jj - j0] = 0; dSc[ii - i0][jj - j0] = 0; continue; }
                Pc[ii - i0][jj - j0] = orc_e4m3_rne(ldexp(P[ii - i0][jj - j0], -sp));
                dSc[ii - i0][jj - j0] = orc_e4m3_rne(ldexp(dS[ii - i0][jj - j0], -sds));
                if (!(exact & 1)) P[ii - i0][jj - j0] = ldexp(orc_e4m3_decode(Pc[ii - i0][jj - j0]), sp);
                if (!(exact & 2)) dS[ii - i0][jj - j0] = ldexp(orc_e4m3_decode(dSc[ii - i0][jj - j0]), sds);
              }
            if (win)
              for (ii = i0; ii < i1; ++ii)
                for (jj = j0; jj < j1 && (!causal || jj <= ii); ++jj) {
                  long long wi = win_index(win, hq, start + ii, start + jj);
                  if (wi < 0) continue;
                  if (win->bwd_dp) win->bwd_dp[wi] = (double)D[(size_t)hq * T + start + ii] - dPv[ii - i0][jj - j0];
                  if (win->bwd_p) { win->bwd_p[wi] = Pc[ii - i0][jj - j0]; win->bwd_ps[wi] = (uint8_t)(sp + 127); }
                  if (win->bwd_ds) { win->bwd_ds[wi] = dSc[ii - i0][jj - j0]; win->bwd_dss[wi] = (uint8_t)(sds + 127); }
                }
            if (dbg && n_docs == 1) {
              size_t bi = ((size_t)hq * nb + bq) * nb + bk;
              if (dbg->p_scale) dbg->p_scale[bi] = (uint8_t)(sp + 127);
              if (dbg->ds_scale) dbg->ds_scale[bi] = (uint8_t)(sds + 127);
              for (ii = i0; ii < i1; ++ii)
                for (jj = j0; jj < j1; ++jj) {
                  size_t ci = ((size_t)hq * L + ii) * L + jj;
                  if (dbg->p_code) dbg->p_code[ci] = Pc[ii - i0][jj - j0];
                  if (dbg->ds_code) dbg->ds_code[ci] = dSc[ii - i0][jj - j0];
                }
            }
            /* the three gradient products of this block (precise: the folded exponents are taken
             * back out of the operand that carries them, so deq() of the other operand applies) */
            for (ii = i0; ii < i1; ++ii)
              for (jj = j0; jj < j1 && (!causal || jj <= ii); ++jj) {
                double ph = P[ii - i0][jj - j0], dsh = dS[ii - i0][jj - j0], dsq = dsh;
                const double* qi = Qd + ((size_t)(start + ii) * Hq + hq) * d;
                const double* doi = dOd + ((size_t)(start + ii) * Hq + hq) * d;
                const double* kj = Kd + ((size_t)(start + jj) * Hkv + g) * d;
                if (precise) {
                  ph = ldexp(ph, 127 - (int)sdo[(size_t)hq * T + start + ii]);
                  dsh = ldexp(dsh, 127 - (int)sq[(size_t)hq * T + start + ii]);
                  dsq = ldexp(dSq[ii - i0][jj - j0], 127 - (int)sk[(size_t)g * T + start + jj]);
                }
                for (cc = 0; cc < d; ++cc) {
                  dv_acc[(size_t)jj * d + cc] += ph * doi[cc];
                  dk_acc[(size_t)jj * d + cc] += dsh * qi[cc];
                  part[(size_t)(ii - i0) * d + cc] += dsq * kj[cc];
                }
              }
          }
          /* FP16 accumulation of this key tile's partial sums, in ascending tile order */
          for (ii = i0; ii < i1; ++ii) {
            int p = pi[(size_t)hq * T + start + ii];
            for (cc = 0; cc < d; ++cc) {
              double x = ldexp(part[(size_t)(ii - i0) * d + cc], p);
              double* a = &acc16[(size_t)(ii - i0) * d + cc];
              if (exact & 4) *a += x;
              else *a = orc_f16_decode(orc_f16_rne(*a + orc_f16_decode(orc_f16_rne(x))));
            }
          }
        }
        for (ii = i0; ii < i1; ++ii) {
          int p = pi[(size_t)hq * T + start + ii];
          for (cc = 0; cc < d; ++cc) {
            double val = softmax_scale * ldexp(acc16[(size_t)(ii - i0) * d + cc], -p);
            dq[((size_t)(start + ii) * Hq + hq) * d + cc] = orc_bf16_rne(val);
            if (dq64) dq64[((size_t)(start + ii) * Hq + hq) * d + cc] = val;
          }
        }
      }
    }
    for (jj = 0; jj < L; ++jj)
      for (cc = 0; cc < d; ++cc) {
        double kval = softmax_scale * dk_acc[(size_t)jj * d + cc], vval = dv_acc[(size_t)jj * d + cc];
        dk[((size_t)(start + jj) * Hkv + g) * d + cc] = orc_bf16_rne(kval);
        dv[((size_t)(start + jj) * Hkv + g) * d + cc] = orc_bf16_rne(vval);
        if (dk64) dk64[((size_t)(start + jj) * Hkv + g) * d + cc] = kval;
        if (dv64) dv64[((size_t)(start + jj) * Hkv + g) * d + cc] = vval;
      }
    free(dk_acc);
    free(dv_acc);
  }
  free(pi);
  if (Qs != Qd) free(Qs);
  if (Ks != Kd) free(Ks);
  free(Qd); free(Kd); free(Vd); free(dOd);
}

/* ------------------------------------------------------------------------------------
 * Replays (test infrastructure): the method's products computed from GIVEN per-pair
 * decisions instead of the oracle's own, in the same order and arithmetic as orc_fwd and
 * orc_bwd.  Fed the oracle's own dumps (orc_window) they reproduce its outputs bit for bit;
 * fed the GPU's decisions, each checked separately against the method's definition, they
 * give what the GPU's products should be up to the FP8 instruction's accumulation and the
 * final rounding.  The decision arrays are laid out [heads][rows][keys] over `win`.
 *
 * Forward replay (jaehun.me §1.2, §3.1): for every (query head, row) of the window whose
 * document's keys up to the row lie in the key window, key tiles from the diagonal tile down
 * to tile 0; per tile the running maximum m is read from M (at the tile's first key),
 * alpha = 2^(m_prev - m) (0 at the first tile), acc = alpha acc + sum_j 2^-p_shift deq(P_ij) V_j,
 * l = alpha l + sum_j 2^(c S_ij - m).  o64 [nh][nr][d] = acc / l and lse64 [nh][nr] = m + log2 l,
 * NaN for rows not replayed.  c_scale = softmax_scale log2(e) as the caller gives it.
 * ---------------------------------------------------------------------------------- */
void orc_fwd_replay(const uint8_t* v, const uint8_t* sv, int T, int Hq, int Hkv, int d, double c_scale,
                    const int32_t* cu, int n_docs, int p_shift, const orc_window* win, const double* S,
                    const double* M, const uint8_t* P, double* o64, double* lse64, int causal, int precise,
                    const uint8_t* PS) {
  const int group = Hq / Hkv;
  const int nh = win->head_hi - win->head_lo, nr = win->row_hi - win->row_lo;
  double* Vd = deq_all(v, sv, T, Hkv, d);
  int* dm = doc_map(cu, n_docs, T);
  long long task;
#pragma omp parallel for schedule(dynamic, 16)
  for (task = 0; task < (long long)nh * nr; ++task) {
    int hh = win->head_lo + (int)(task / nr), row = win->row_lo + (int)(task % nr), g = hh / group;
    int doc = (row >= 0 && row < T) ? dm[row] : -1, kappa, j, cc;
    double acc[256], m = -INFINITY, l = 0.0;
    int vref = -1000;
    double* o = o64 + (size_t)task * d;
    lse64[task] = NAN;
    for (cc = 0; cc < d; ++cc) o[cc] = NAN;
    if (doc < 0 || cu[doc] < win->key_lo || (causal ? row : cu[doc + 1] - 1) >= win->key_hi) continue;
    for (cc = 0; cc < d; ++cc) acc[cc] = 0.0;
    {
      int start = cu[doc], r = row - start, L = cu[doc + 1] - start;
      for (kappa = (causal ? r : L - 1) / KV_TILE; kappa >= 0; --kappa) {
        int j0 = kappa * KV_TILE, j1 = (kappa + 1) * KV_TILE;
        double m_new, alpha, sum = 0.0;
        if (causal && j1 > r + 1) j1 = r + 1;
        if (j1 > L) j1 = L;
        m_new = M[win_index(win, hh, row, start + j0)];
        alpha = (m == -INFINITY) ? 0.0 : exp2(m - m_new);
        for (cc = 0; cc < d; ++cc) acc[cc] *= alpha;
        if (precise) vref = fold_ref(sv + (size_t)g * T + start, j0, j1, vref);
        for (j = j0; j < j1; ++j) {
          long long wi = win_index(win, hh, row, start + j);
          const double* vj = Vd + ((size_t)(start + j) * Hkv + g) * d;
          const int fold = precise ? (int)sv[(size_t)g * T + start + j] - 127 - vref : 0;
          /* PS (4-bit scores): the code's group exponent byte */
          double ph = ldexp(orc_e4m3_decode(P[wi]), PS ? (int)PS[wi] - 127 : -p_shift - fold);
          sum += exp2(S[wi] * c_scale - m_new);
          for (cc = 0; cc < d; ++cc) acc[cc] += ph * vj[cc];
        }
        l = alpha * l + sum;
        m = m_new;
      }
      for (cc = 0; cc < d; ++cc) o[cc] = acc[cc] / l;
      lse64[task] = m + log2(l);
    }
  }
  free(Vd); free(dm);
}

/* Backward replay (jaehun.me §1.2, §3.1, §3.2): dQ of every (query head, row) of the window,
 * and dK, dV of every key in [row_lo, row_hi) for the KV heads whose whole query-head group lies
 * in the head window, from the given Phat / dShat codes and block exponent bytes (PS, DSS hold
 * exponent + 127 per pair):
 *   dV_j = sum_{h in group} sum_i 2^ps deq(P_ij) deq(dO_i),
 *   dK_j = softmax_scale sum_{h in group} sum_i 2^dss deq(DS_ij) deq(Q_i),
 *   dQ_i: 128-key tiles ascending, part = sum_j 2^dss deq(DS_ij) deq(K_j),
 *         acc16 = f16(acc16 + f16(2^pi part)), dQ = softmax_scale 2^-pi acc16.
 * Each document is replayed from the 32-query block that contains the window's first row (the
 * window must start on a block of the document, or before it); all visible pairs from there to
 * the document end must be in the dump, keys from the document start.  Order of every sum as in
 * orc_bwd.  dq64 [nh][nr][d]; dk64, dv64 [Hkv][nr][d] (key rows of the row window); NaN where
 * not computed. */
void orc_bwd_replay(const uint8_t* q, const uint8_t* sq, const uint8_t* k, const uint8_t* sk, const uint8_t* dO,
                    const uint8_t* sdo, int T, int Hq, int Hkv, int d, double softmax_scale, const int32_t* cu,
                    int n_docs, const int16_t* pi, const orc_window* win, const uint8_t* P, const uint8_t* PS,
                    const uint8_t* DS, const uint8_t* DSS, double* dq64, double* dk64, double* dv64, int causal) {
  const int group = Hq / Hkv;
  const int nr = win->row_hi - win->row_lo;
  long long task, n_tasks = (long long)n_docs * Hkv;
  size_t z;
  double* Qd = deq_all(q, sq, T, Hq, d);
  double* Kd = deq_all(k, sk, T, Hkv, d);
  double* dOd = deq_all(dO, sdo, T, Hq, d);
  for (z = 0; z < (size_t)(win->head_hi - win->head_lo) * nr * d; ++z) dq64[z] = NAN;
  for (z = 0; z < (size_t)Hkv * nr * d; ++z) { dk64[z] = NAN; dv64[z] = NAN; }
#pragma omp parallel for schedule(dynamic, 1)
  for (task = 0; task < n_tasks; ++task) {
    int doc = (int)(task / Hkv), g = (int)(task % Hkv);
    int start = cu[doc], L = cu[doc + 1] - start, hq, bq, bk, ii, jj, cc, bq0, kv_ok;
    int nb = (L + BLK - 1) / BLK;
    double *dk_acc, *dv_acc, part[BLK * 256], acc16[BLK * 256];
    if (L <= 0 || cu[doc + 1] <= win->row_lo || start >= win->row_hi) continue;
    bq0 = win->row_lo > start ? (win->row_lo - start) / BLK : 0;
    /* dK, dV of a key need every row that sees it: all of them here only when the window's rows
       start at the document start or, causally, at or before the key */
    kv_ok = g * group >= win->head_lo && (g + 1) * group <= win->head_hi && (causal || bq0 == 0);
    dk_acc = (double*)calloc((size_t)L * d, sizeof(double));
    dv_acc = (double*)calloc((size_t)L * d, sizeof(double));
    for (hq = g * group; hq < (g + 1) * group; ++hq) {
      int in_heads = hq >= win->head_lo && hq < win->head_hi;
      if (!in_heads) continue;
      for (bq = bq0; bq < nb; ++bq) {
        int i0 = bq * BLK, i1 = i0 + BLK < L ? i0 + BLK : L;
        int kappa, kappa_last = (causal ? i1 - 1 : L - 1) / KV_TILE;
        for (z = 0; z < (size_t)BLK * d; ++z) acc16[z] = 0.0;
        for (kappa = 0; kappa <= kappa_last; ++kappa) {
          for (z = 0; z < (size_t)BLK * d; ++z) part[z] = 0.0;
          for (bk = kappa * (KV_TILE / BLK); bk < (kappa + 1) * (KV_TILE / BLK) && bk < nb && (!causal || bk <= bq);
               ++bk) {
            int j0 = bk * BLK, j1 = j0 + BLK < L ? j0 + BLK : L;
            for (ii = i0; ii < i1; ++ii)
              for (jj = j0; jj < j1 && (!causal || jj <= ii); ++jj) {
                long long wi = win_index(win, hq, start + ii, start + jj);
                double ph = ldexp(orc_e4m3_decode(P[wi]), (int)PS[wi] - 127);
                double dsh = ldexp(orc_e4m3_decode(DS[wi]), (int)DSS[wi] - 127);
                const double* qi = Qd + ((size_t)(start + ii) * Hq + hq) * d;
                const double* doi = dOd + ((size_t)(start + ii) * Hq + hq) * d;
                const double* kj = Kd + ((size_t)(start + jj) * Hkv + g) * d;
                for (cc = 0; cc < d; ++cc) {
                  dv_acc[(size_t)jj * d + cc] += ph * doi[cc];
                  dk_acc[(size_t)jj * d + cc] += dsh * qi[cc];
                  part[(size_t)(ii - i0) * d + cc] += dsh * kj[cc];
                }
              }
          }
          for (ii = i0; ii < i1; ++ii) {
            int p = pi[(size_t)hq * T + start + ii];
            for (cc = 0; cc < d; ++cc) {
              double x = ldexp(part[(size_t)(ii - i0) * d + cc], p);
              double* a = &acc16[(size_t)(ii - i0) * d + cc];
              *a = orc_f16_decode(orc_f16_rne(*a + orc_f16_decode(orc_f16_rne(x))));
            }
          }
        }
        for (ii = i0; ii < i1; ++ii) {
          int p = pi[(size_t)hq * T + start + ii], row = start + ii;
          if (row < win->row_lo || row >= win->row_hi) continue;
          for (cc = 0; cc < d; ++cc)
            dq64[((size_t)(hq - win->head_lo) * nr + (row - win->row_lo)) * d + cc] =
                softmax_scale * ldexp(acc16[(size_t)(ii - i0) * d + cc], -p);
        }
      }
    }
    if (kv_ok)
      for (jj = 0; jj < L; ++jj) {
        int key = start + jj;
        if (key < win->row_lo || key >= win->row_hi || jj < bq0 * BLK) continue;
        for (cc = 0; cc < d; ++cc) {
          dk64[((size_t)g * nr + (key - win->row_lo)) * d + cc] = softmax_scale * dk_acc[(size_t)jj * d + cc];
          dv64[((size_t)g * nr + (key - win->row_lo)) * d + cc] = dv_acc[(size_t)jj * d + cc];
        }
      }
    free(dk_acc);
    free(dv_acc);
  }
  free(Qd); free(Kd); free(dOd);
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Array forms of the codecs (elementwise), for the tests. */
void orc_e4m3_rne_array(const double* y, uint8_t* out, long n) { long i; for (i = 0; i < n; ++i) out[i] = orc_e4m3_rne(y[i]); }
void orc_e4m3_decode_array(const uint8_t* c, double* out, long n) { long i; for (i = 0; i < n; ++i) out[i] = orc_e4m3_decode(c[i]); }
void orc_bf16_rne_array(const double* y, uint16_t* out, long n) { long i; for (i = 0; i < n; ++i) out[i] = orc_bf16_rne(y[i]); }
void orc_f16_rne_array(const double* y, uint16_t* out, long n) { long i; for (i = 0; i < n; ++i) out[i] = orc_f16_rne(y[i]); }
void orc_e8m0_roundup_array(const double* a, int32_t* out, long n) { long i; for (i = 0; i < n; ++i) out[i] = orc_e8m0_roundup(a[i]); }
