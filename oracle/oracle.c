/*
 * oracle.c -- plain CPU oracle (TEST INFRASTRUCTURE ONLY; see oracle.h).
 *
 * Written for clarity, not speed: every weight is rebuilt element by element
 * from its block bytes and every dot product is a plain fp64 loop.  The only
 * concession to run time is an OpenMP loop over independent output rows.
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* sizes                                                                     */
/* ------------------------------------------------------------------------ */

int or_block_elems(int fmt) {
  switch (fmt) {
    case OR_Q4_0: case OR_Q8_0: case OR_MXFP4: case OR_Q8_1: case OR_Q4_1: case OR_Q5_0: case OR_Q5_1:
      return 32;
    case OR_Q4_K: case OR_Q5_K: case OR_Q6_K: case OR_Q8_K: case OR_Q2_K: case OR_Q3_K: return 256;
    default: return 0;
  }
}

int or_block_bytes(int fmt) {
  switch (fmt) {
    case OR_Q4_0: return 18;    /* fp16 d, 16 bytes of nibbles */
    case OR_Q8_0: return 34;    /* fp16 d, 32 int8 */
    case OR_Q4_K: return 144;   /* fp16 d, fp16 dmin, 12 scale bytes, 128 nibble bytes */
    case OR_Q5_K: return 176;   /* as Q4_K plus 32 bytes of fifth bits */
    case OR_Q6_K: return 210;   /* 128 low-nibble bytes, 64 high-bit bytes, 16 int8 scales, fp16 d */
    case OR_MXFP4: return 17;   /* E8M0 exponent byte, 16 bytes of E2M1 codes */
    case OR_Q8_1: return 36;    /* fp16 d, fp16 s, 32 int8 */
    case OR_Q8_K: return 292;   /* fp32 d, 256 int8, 16 int16 group sums */
    case OR_Q2_K: return 84;    /* 16 scale/min bytes, 64 bytes of 2-bit codes, fp16 d, fp16 dmin */
    case OR_Q3_K: return 110;
    case OR_Q4_1: return 20;    /* fp16 d, fp16 m, 16 bytes of nibbles */
    case OR_Q5_0: return 22;    /* fp16 d, 4 bytes of fifth bits, 16 bytes of nibbles */
    case OR_Q5_1: return 24;    /* fp16 d, fp16 m, 4 bytes of fifth bits, 16 bytes of nibbles */   /* 32 high-bit bytes, 64 bytes of 2-bit codes, 12 scale bytes, fp16 d */
    default: return 0;
  }
}

int or_sub_elems(int wfmt) { return wfmt == OR_Q6_K || wfmt == OR_Q2_K || wfmt == OR_Q3_K ? 16 : 32; }

int or_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void or_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* binary16                                                                  */
/* ------------------------------------------------------------------------ */

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)(v & 0xFF); p[1] = (uint8_t)(v >> 8); }

float or_f16_to_f32(uint16_t h) {
  /* value = (-1)^s * 2^(E-15) * 1.m  (normal) or 2^-14 * 0.m (subnormal) */
  int s = (h >> 15) & 1;
  int E = (h >> 10) & 0x1F;
  int m = h & 0x3FF;
  double v;
  if (E == 0x1F) {
    if (m) return NAN;
    v = INFINITY;
  } else if (E == 0) {
    v = ldexp((double)m, -24);
  } else {
    v = ldexp((double)(m | 0x400), E - 25);
  }
  return (float)(s ? -v : v); /* exact: fp16 values are exact in fp32 */
}

uint16_t or_f32_to_f16(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  uint16_t sign = (uint16_t)((x >> 16) & 0x8000);
  uint32_t exp = (x >> 23) & 0xFF;
  uint32_t man = x & 0x7FFFFF;
  if (exp == 0xFF) /* inf stays inf; NaN stays a (quiet) NaN */
    return (uint16_t)(sign | 0x7C00 | (man ? (0x200 | (man >> 13)) : 0));
  if (exp == 0) /* zero or fp32 subnormal: |f| < 2^-126, far below half of 2^-24 */
    return sign;
  int E = (int)exp - 127;                 /* f = sig * 2^(E-23), sig has 24 bits */
  uint32_t sig = man | 0x800000;
  /* bits dropped: 13 for a normal fp16 result; more once E < -14 (subnormal,
     whose unit is 2^-24) */
  int shift = (E >= -14) ? 13 : 13 + (-14 - E);
  if (shift > 24) return sign;            /* |f| < 2^-25 rounds to zero */
  uint32_t q = sig >> shift;
  uint32_t rem = sig & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q++;   /* ties to even */
  /* normal: exponent field E+15 plus (q - 2^10); writing it as (E+14)<<10 + q lets a
     rounding carry (q == 2^11) step the exponent.  subnormal: q is the field; q == 2^10
     becomes the smallest normal. */
  uint32_t bits = (E >= -14) ? (((uint32_t)(E + 14) << 10) + q) : q;
  if (bits >= 0x7C00) bits = 0x7C00;      /* overflow to infinity */
  return (uint16_t)(sign | bits);
}

void or_f32_to_f16_range(uint32_t first, uint32_t count, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)count; i++) {
    uint32_t b = first + (uint32_t)i;
    float f;
    memcpy(&f, &b, 4);
    out[i] = or_f32_to_f16(f);
  }
}

static double f16d(const uint8_t* p) { return (double)or_f16_to_f32(rd16(p)); }

/* ------------------------------------------------------------------------ */
/* per-element weight codes                                                  */
/* Each format writes w_e = scale_j * code_e - min_j, with j the sub-block of */
/* element e.  The keep-quant method multiplies integer codes, so the oracle */
/* keeps code, scale and min apart.                                          */
/* ------------------------------------------------------------------------ */

/* Q4_0: element e<16 is the low nibble of qs[e], e>=16 the high nibble of qs[e-16];
   w = d * (n - 8). */
static int code_q4_0(const uint8_t* b, int e) {
  const uint8_t* qs = b + 2;
  int n = e < 16 ? (qs[e] & 15) : (qs[e - 16] >> 4);
  return n - 8;
}

/* Q8_0: w = d * qs[e]. */
static int code_q8_0(const uint8_t* b, int e) { return (int)(int8_t)b[2 + e]; }

/* K-quant 6-bit scale / min of sub-block j (0..7) from the 12 packed bytes:
   sub-blocks 0-3 keep their low six bits in bytes j (scale) and j+4 (min);
   sub-blocks 4-7 take four bits from byte j+4 (low nibble: scale, high: min)
   and their top two bits from the spare top bits of bytes j-4 (scale) and j (min). */
static void kq_scale_min(const uint8_t* sc12, int j, int* sc, int* m) {
  if (j < 4) {
    *sc = sc12[j] & 63;
    *m = sc12[j + 4] & 63;
  } else {
    *sc = (sc12[j + 4] & 15) | ((sc12[j - 4] >> 6) << 4);
    *m = (sc12[j + 4] >> 4) | ((sc12[j] >> 6) << 4);
  }
}

/* Q4_K: element e = 64c + 32h + l (c<4, h<2, l<32) sits in qs[32c + l],
   low nibble for h=0, high nibble for h=1; sub-block j = e/32.
   w = (d*sc_j) * n - (dmin*m_j). */
static int code_q4_k(const uint8_t* b, int e) {
  const uint8_t* qs = b + 16;
  int c = e / 64, h = (e / 32) & 1, l = e & 31;
  uint8_t v = qs[32 * c + l];
  return h ? (v >> 4) : (v & 15);
}

/* Q5_K: as Q4_K, plus the fifth bit: bit (2c+h) of qh[l]. */
static int code_q5_k(const uint8_t* b, int e) {
  const uint8_t* qh = b + 16;
  const uint8_t* qs = b + 48;
  int c = e / 64, h = (e / 32) & 1, l = e & 31;
  uint8_t v = qs[32 * c + l];
  int n = h ? (v >> 4) : (v & 15);
  return n + 16 * ((qh[l] >> (2 * c + h)) & 1);
}

/* Q6_K: element e = 128g + 32r + l (g<2, r<4, l<32).  Low four bits: for r<2 the low
   nibble of ql[64g + 32r + l], for r>=2 the high nibble of ql[64g + 32(r-2) + l].
   Top two bits: bits 2r..2r+1 of qh[32g + l].  w = (d * sc[e/16]) * (q6 - 32). */
static int code_q6_k(const uint8_t* b, int e) {
  const uint8_t* ql = b;
  const uint8_t* qh = b + 128;
  int g = e / 128, r = (e / 32) & 3, l = e & 31;
  int lo = r < 2 ? (ql[64 * g + 32 * r + l] & 15) : (ql[64 * g + 32 * (r - 2) + l] >> 4);
  int hi = (qh[32 * g + l] >> (2 * r)) & 3;
  return (lo | (hi << 4)) - 32;
}

/* MXFP4: 4-bit E2M1 code per element (nibble order as Q4_0).  The code's value
   (sign bit 3, exponent bits 2..1, mantissa bit 0) doubled, so it is an integer:
   magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 -> 0, 1, 2, 3, 4, 6, 8, 12.
   w = doubled * 2^(e8 - 128) = E2M1 * 2^(e8 - 127). */
static int e2m1_doubled(int code) {
  int mag = code & 7;
  int ex = mag >> 1, mb = mag & 1;
  /* ex == 0: subnormal 0.5*mb -> doubled mb; else (1 + mb/2) * 2^(ex-1) -> doubled (2+mb) << (ex-1) */
  int v = ex == 0 ? mb : ((2 + mb) << (ex - 1));
  return (code & 8) ? -v : v;
}
static int code_mxfp4(const uint8_t* b, int e) {
  const uint8_t* qs = b + 1;
  int c = e < 16 ? (qs[e] & 15) : (qs[e - 16] >> 4);
  return e2m1_doubled(c);
}

/* Q2_K and Q3_K share one code order: element e = 128g + 32r + l (g<2, r<4, l<32)
   takes bits 2r..2r+1 of byte 32g + l of the 64 code bytes; its sub-block is e/16.
   Q2_K: scales[16] @0 (low nibble scale, high nibble min), codes @16, d @80,
   dmin @82;  w = (d * sc_j) * q - dmin * m_j with q in 0..3. */
static int code_q2_k(const uint8_t* b, int e) {
  int g = e / 128, r = (e / 32) & 3, l = e & 31;
  return (b[16 + 32 * g + l] >> (2 * r)) & 3;
}

/* Q3_K: hmask[32] @0, codes @32, scales[12] @96, d @108.  The third bit of element
   e is bit (4g + r) of hmask[l]; q = low two bits + 4 * third bit - 4, in -4..3. */
static int code_q3_k(const uint8_t* b, int e) {
  int g = e / 128, r = (e / 32) & 3, l = e & 31;
  int lo = (b[32 + 32 * g + l] >> (2 * r)) & 3;
  int hi = (b[l] >> (4 * g + r)) & 1;
  return lo + 4 * hi - 4;
}

/* Q3_K signed 6-bit scale of sub-block j (0..15), stored plus 32: the low four bits
   are the low nibble of byte j for j<8 and the high nibble of byte j-8 for j>=8; the
   top two bits are bits 2(j/4)..2(j/4)+1 of byte 8 + j%4. */
static int q3k_scale(const uint8_t* sc12, int j) {
  int lo = j < 8 ? (sc12[j] & 15) : (sc12[j - 8] >> 4);
  int hi = (sc12[8 + (j & 3)] >> (2 * (j >> 2))) & 3;
  return (lo | (hi << 4)) - 32;
}

/* Q4_1: d @0, m @2, nibbles @4 in Q4_0's order; w = d * n + m. */
static int code_q4_1(const uint8_t* b, int e) {
  const uint8_t* qs = b + 4;
  return e < 16 ? (qs[e] & 15) : (qs[e - 16] >> 4);
}

/* Q5_0 / Q5_1: nibbles in Q4_0's order plus a fifth bit, bit e of the little-endian
   32-bit qh.  Q5_0: d @0, qh @2, nibbles @6, w = d * (q - 16).  Q5_1: d @0, m @2,
   qh @4, nibbles @8, w = d * q + m. */
static int code_q5(const uint8_t* b, int e, int qh_off) {
  const uint8_t* qh = b + qh_off;
  const uint8_t* qs = b + qh_off + 4;
  int n = e < 16 ? (qs[e] & 15) : (qs[e - 16] >> 4);
  int fifth = (qh[e / 8] >> (e % 8)) & 1;
  return n + 16 * fifth;
}

/* integer code of weight element e */
static int wcode(int fmt, const uint8_t* b, int e) {
  switch (fmt) {
    case OR_Q4_0: return code_q4_0(b, e);
    case OR_Q8_0: return code_q8_0(b, e);
    case OR_Q4_K: return code_q4_k(b, e);
    case OR_Q5_K: return code_q5_k(b, e);
    case OR_Q6_K: return code_q6_k(b, e);
    case OR_MXFP4: return code_mxfp4(b, e);
    case OR_Q2_K: return code_q2_k(b, e);
    case OR_Q3_K: return code_q3_k(b, e);
    case OR_Q4_1: return code_q4_1(b, e);
    case OR_Q5_0: return code_q5(b, e, 2) - 16;
    case OR_Q5_1: return code_q5(b, e, 4);
    default: return 0;
  }
}

/* 2^(e8-128) for an E8M0 byte (e8 = 255 is NaN in the MX format) */
static double e8m0_half(int e8) { return e8 == 255 ? NAN : ldexp(1.0, e8 - 128); }

/* scale and min (fp64, exact) of the sub-block holding weight element e */
static void wscale(int fmt, const uint8_t* b, int e, double* scale, double* mn) {
  *mn = 0.0;
  switch (fmt) {
    case OR_Q4_0:
    case OR_Q8_0: *scale = f16d(b); break;
    case OR_Q4_K:
    case OR_Q5_K: {
      int sc, m;
      kq_scale_min(b + 4, e / 32, &sc, &m);
      *scale = f16d(b) * sc;
      *mn = f16d(b + 2) * m;
      break;
    }
    case OR_Q6_K: *scale = f16d(b + 208) * (double)(int8_t)b[192 + e / 16]; break;
    case OR_MXFP4: *scale = e8m0_half(b[0]); break;
    case OR_Q2_K:
      *scale = f16d(b + 80) * (b[e / 16] & 15);
      *mn = f16d(b + 82) * (b[e / 16] >> 4);
      break;
    case OR_Q3_K: *scale = f16d(b + 108) * q3k_scale(b + 96, e / 16); break;
    case OR_Q5_0: *scale = f16d(b); break;
    case OR_Q4_1:
    case OR_Q5_1:   /* the offset m is added: w = scale * code - (-m) */
      *scale = f16d(b);
      *mn = -f16d(b + 2);
      break;
    default: *scale = 0.0;
  }
}

/* activation blocks: int8 code and fp64 scale of element e.  Q8_1 and Q8_K keep
   their codes from byte 4 on, Q8_0 (fp16 d, no sum field) from byte 2. */
static int acode(int afmt, const uint8_t* b, int e) {
  return (int)(int8_t)b[(afmt == OR_Q8_0 ? 2 : 4) + e];
}
static double ascale(int afmt, const uint8_t* b) {
  if (afmt == OR_Q8_1 || afmt == OR_Q8_0) return f16d(b);
  float d;
  memcpy(&d, b, 4);
  return (double)d;
}

double or_elem(int fmt, const uint8_t* b, int e) {
  if (fmt == OR_Q8_1 || fmt == OR_Q8_K) return ascale(fmt, b) * acode(fmt, b, e);
  double scale, mn;
  wscale(fmt, b, e, &scale, &mn);
  /* scale*code and mn are exact in fp64 and so is their difference for the
     value ranges the formats produce */
  return scale * wcode(fmt, b, e) - mn;
}

static int is_weight(int f) { return (f >= OR_Q4_0 && f <= OR_MXFP4) || (f >= OR_Q2_K && f <= OR_Q5_1); }
/* Q8_0 is both: a weight format and, in the same layout, an activation format */
static int is_act(int f) { return f == OR_Q8_1 || f == OR_Q8_K || f == OR_Q8_0; }

void or_dequant_f32(int fmt, const uint8_t* blocks, int64_t rows, int64_t k, float* out) {
  int be = or_block_elems(fmt), bb = or_block_bytes(fmt);
  int64_t nb = k / be;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; r++)
    for (int64_t i = 0; i < k; i++) {
      const uint8_t* b = blocks + (r * nb + i / be) * bb;
      /* rounding the exact value once gives the fp32 dequantized weight */
      out[r * k + i] = (float)or_elem(fmt, b, (int)(i % be));
    }
}

/* ------------------------------------------------------------------------ */
/* activation quantizers                                                     */
/* ------------------------------------------------------------------------ */

/* Q8_1 of one 32-block: d = fp16(amax/127); q = clamp(round(x/d)) against the
   stored (fp16) scale; s = fp16(d * sum q).  Rounds half away from zero. */
static void quant_q8_1_block(const float* x, uint8_t* out) {
  float amax = 0.0f;
  for (int i = 0; i < 32; i++) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  uint16_t dh = or_f32_to_f16(amax / 127.0f);
  float d = or_f16_to_f32(dh);
  int sum = 0;
  for (int i = 0; i < 32; i++) {
    int q = 0;
    if (d != 0.0f) {
      float v = roundf(x[i] / d);
      q = v > 127.0f ? 127 : (v < -127.0f ? -127 : (int)v);
    }
    out[4 + i] = (uint8_t)(int8_t)q;
    sum += q;
  }
  if (d == 0.0f) dh = 0;
  wr16(out, dh);
  wr16(out + 2, or_f32_to_f16(d * (float)sum));
}

/* Q8_0 of one 32-block: the Q8_1 scale and codes, d = fp16(amax/127) and q =
   clamp(round(x/d)) against the stored d, in a block without the sum field (d at
   byte 0, codes from byte 2). */
static void quant_q8_0_block(const float* x, uint8_t* out) {
  float amax = 0.0f;
  for (int i = 0; i < 32; i++) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  uint16_t dh = or_f32_to_f16(amax / 127.0f);
  float d = or_f16_to_f32(dh);
  for (int i = 0; i < 32; i++) {
    int q = 0;
    if (d != 0.0f) {
      float v = roundf(x[i] / d);
      q = v > 127.0f ? 127 : (v < -127.0f ? -127 : (int)v);
    }
    out[2 + i] = (uint8_t)(int8_t)q;
  }
  if (d == 0.0f) dh = 0;
  wr16(out, dh);
}

/* Q8_K of one 256-block: d = amax/127 in fp32 (kept, positive);
   q = clamp(round(x/d)); bsums[g] = sum of q over elements 16g..16g+15. */
static void quant_q8_k_block(const float* x, uint8_t* out) {
  float amax = 0.0f;
  for (int i = 0; i < 256; i++) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float d = amax / 127.0f;
  int8_t q[256];
  for (int i = 0; i < 256; i++) {
    int v = 0;
    if (d != 0.0f) {
      float r = roundf(x[i] / d);
      v = r > 127.0f ? 127 : (r < -127.0f ? -127 : (int)r);
    }
    q[i] = (int8_t)v;
  }
  memcpy(out, &d, 4);
  memcpy(out + 4, q, 256);
  for (int g = 0; g < 16; g++) {
    int s = 0;
    for (int i = 0; i < 16; i++) s += q[16 * g + i];
    int16_t s16 = (int16_t)s;
    memcpy(out + 260 + 2 * g, &s16, 2);
  }
}

void or_quantize(int afmt, const float* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* out) {
  int be = or_block_elems(afmt), bb = or_block_bytes(afmt);
  int64_t nb = k / be;
  for (int64_t r = 0; r < rows; r++)
    for (int64_t i = 0; i < nb; i++) {
      const float* xb = x + r * ldx + i * be;
      uint8_t* ob = out + (r * nb + i) * bb;
      if (afmt == OR_Q8_1) quant_q8_1_block(xb, ob);
      else if (afmt == OR_Q8_0) quant_q8_0_block(xb, ob);
      else quant_q8_k_block(xb, ob);
    }
}

/* ------------------------------------------------------------------------ */
/* integer block dots                                                        */
/* ------------------------------------------------------------------------ */

int or_block_dots(int wfmt, const uint8_t* W, int64_t n, int64_t k,
                  int afmt, const uint8_t* xq, int64_t t, int32_t* partials) {
  if (!is_weight(wfmt) || !is_act(afmt)) return -1;
  int wbe = or_block_elems(wfmt), wbb = or_block_bytes(wfmt);
  int abe = or_block_elems(afmt), abb = or_block_bytes(afmt);
  if (k % wbe || k % abe) return -1;
  int sub = or_sub_elems(wfmt);
  int64_t nsub = k / sub, wnb = k / wbe, anb = k / abe;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; r++)
    for (int64_t tt = 0; tt < t; tt++)
      for (int64_t s = 0; s < nsub; s++) {
        int64_t acc = 0;
        for (int64_t i = s * sub; i < (s + 1) * sub; i++) {
          const uint8_t* wb = W + (r * wnb + i / wbe) * wbb;
          const uint8_t* ab = xq + (tt * anb + i / abe) * abb;
          acc += (int64_t)wcode(wfmt, wb, (int)(i % wbe)) * acode(afmt, ab, (int)(i % abe));
        }
        partials[(tt * n + r) * nsub + s] = (int32_t)acc;
      }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* plain-definition matvec                                                   */
/* ------------------------------------------------------------------------ */

static void dequant_row_f64(int fmt, const uint8_t* row_blocks, int64_t k, double* out) {
  int be = or_block_elems(fmt), bb = or_block_bytes(fmt);
  for (int64_t i = 0; i < k; i++) out[i] = or_elem(fmt, row_blocks + (i / be) * bb, (int)(i % be));
}

static int pair_ok(int wfmt, int afmt, int64_t k) {
  if (!is_weight(wfmt) || !is_act(afmt)) return 0;
  return k % or_block_elems(wfmt) == 0 && k % or_block_elems(afmt) == 0;
}

static double dot64(const double* a, const double* b, int64_t k) {
  double s = 0.0;
  for (int64_t i = 0; i < k; i++) s += a[i] * b[i];
  return s;
}

int or_matvec(int wfmt, const uint8_t* W, int64_t n, int64_t k,
              int afmt, const uint8_t* xq, int64_t t, float* y, int64_t ldy) {
  if (!pair_ok(wfmt, afmt, k)) return -1;
  int64_t wrow = k / or_block_elems(wfmt) * or_block_bytes(wfmt);
  int64_t arow = k / or_block_elems(afmt) * or_block_bytes(afmt);
  double* xa = (double*)malloc(sizeof(double) * (size_t)(t * k + 1));
  for (int64_t tt = 0; tt < t; tt++) dequant_row_f64(afmt, xq + tt * arow, k, xa + tt * k);
#pragma omp parallel
  {
    double* wr = (double*)malloc(sizeof(double) * (size_t)(k + 1));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < n; r++) {
      dequant_row_f64(wfmt, W + r * wrow, k, wr);
      for (int64_t tt = 0; tt < t; tt++) y[tt * ldy + r] = (float)dot64(wr, xa + tt * k, k);
    }
    free(wr);
  }
  free(xa);
  return 0;
}

/* keep-quant: per weight sub-block j, y += d_x * (scale_j * I_j - min_j * B_j) with
   I_j the integer dot of weight codes and activation codes and B_j the sum of the
   activation codes (sub-blocks never straddle an activation block). */
int or_matvec_keepquant(int wfmt, const uint8_t* W, int64_t n, int64_t k,
                        int afmt, const uint8_t* xq, int64_t t, double* y) {
  if (!pair_ok(wfmt, afmt, k)) return -1;
  int wbe = or_block_elems(wfmt), wbb = or_block_bytes(wfmt);
  int abe = or_block_elems(afmt), abb = or_block_bytes(afmt);
  int sub = or_sub_elems(wfmt);
  int64_t wnb = k / wbe, anb = k / abe;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; r++)
    for (int64_t tt = 0; tt < t; tt++) {
      double acc = 0.0;
      for (int64_t s0 = 0; s0 < k; s0 += sub) {
        const uint8_t* wb = W + (r * wnb + s0 / wbe) * wbb;
        const uint8_t* ab = xq + (tt * anb + s0 / abe) * abb;
        int64_t I = 0, B = 0;
        for (int64_t i = s0; i < s0 + sub; i++) {
          int q = acode(afmt, ab, (int)(i % abe));
          I += (int64_t)wcode(wfmt, wb, (int)(i % wbe)) * q;
          B += q;
        }
        double scale, mn;
        wscale(wfmt, wb, (int)(s0 % wbe), &scale, &mn);
        acc += ascale(afmt, ab) * (scale * (double)I - mn * (double)B);
      }
      y[tt * n + r] = acc;
    }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* routing and sort                                                          */
/* ------------------------------------------------------------------------ */

int or_route(const float* logits, int64_t t, int64_t n_expert, int topk,
             int32_t* ids, float* w) {
  if (topk < 1 || topk > n_expert) return -1;
  char* taken = (char*)malloc((size_t)n_expert);
  for (int64_t tt = 0; tt < t; tt++) {
    const float* l = logits + tt * n_expert;
    memset(taken, 0, (size_t)n_expert);
    for (int k = 0; k < topk; k++) {
      int64_t best = -1;
      for (int64_t e = 0; e < n_expert; e++)
        if (!taken[e] && (best < 0 || l[e] > l[best])) best = e; /* strict >: lower index wins ties */
      taken[best] = 1;
      ids[tt * topk + k] = (int32_t)best;
    }
    double lmax = l[ids[tt * topk]];
    double den = 0.0;
    for (int k = 0; k < topk; k++) den += exp((double)l[ids[tt * topk + k]] - lmax);
    for (int k = 0; k < topk; k++)
      w[tt * topk + k] = (float)(exp((double)l[ids[tt * topk + k]] - lmax) / den);
  }
  free(taken);
  return 0;
}

int or_sort_pairs(const int32_t* ids, int64_t t, int topk, int64_t n_expert,
                  int32_t* counts, int32_t* offsets, int32_t* pairs) {
  int64_t np = t * topk, pos = 0;
  for (int64_t e = 0; e < n_expert; e++) {
    offsets[e] = (int32_t)pos;
    int32_t c = 0;
    for (int64_t p = 0; p < np; p++)
      if (ids[p] == e) { pairs[pos++] = (int32_t)p; c++; }
    counts[e] = c;
  }
  offsets[n_expert] = (int32_t)pos;
  return pos == np ? 0 : -1; /* an id outside [0, E) leaves pairs unsorted */
}

/* ------------------------------------------------------------------------ */
/* routed MoE stages and grouped GEMM                                        */
/* ------------------------------------------------------------------------ */

int or_moe_gate_up(int wfmt, const uint8_t* w_gate, const uint8_t* w_up,
                   int64_t n_expert, int64_t hidden, int64_t inter,
                   int afmt, const uint8_t* xq, int64_t t,
                   const int32_t* ids, int topk, float* g, float* u, float* h) {
  if (!pair_ok(wfmt, afmt, hidden)) return -1;
  int64_t wrow = hidden / or_block_elems(wfmt) * or_block_bytes(wfmt);
  int64_t arow = hidden / or_block_elems(afmt) * or_block_bytes(afmt);
  int64_t np = t * topk;
  for (int64_t p = 0; p < np; p++)
    if (ids[p] < 0 || ids[p] >= n_expert) return -1;
  double* xa = (double*)malloc(sizeof(double) * (size_t)(t * hidden + 1));
  for (int64_t tt = 0; tt < t; tt++) dequant_row_f64(afmt, xq + tt * arow, hidden, xa + tt * hidden);
#pragma omp parallel
  {
    double* wg = (double*)malloc(sizeof(double) * (size_t)hidden);
    double* wu = (double*)malloc(sizeof(double) * (size_t)hidden);
#pragma omp for schedule(static)
    for (int64_t idx = 0; idx < np * inter; idx++) {
      int64_t p = idx / inter, r = idx % inter;
      int64_t e = ids[p];
      const double* x = xa + (p / topk) * hidden;
      dequant_row_f64(wfmt, w_gate + (e * inter + r) * wrow, hidden, wg);
      dequant_row_f64(wfmt, w_up + (e * inter + r) * wrow, hidden, wu);
      double gv = dot64(wg, x, hidden), uv = dot64(wu, x, hidden);
      /* SwiGLU, gate first: silu(g) * u with silu(g) = g / (1 + e^-g) */
      double hv = gv / (1.0 + exp(-gv)) * uv;
      if (g) g[p * inter + r] = (float)gv;
      if (u) u[p * inter + r] = (float)uv;
      if (h) h[p * inter + r] = (float)hv;
    }
    free(wg);
    free(wu);
  }
  free(xa);
  return 0;
}

int or_moe_down(int wfmt, const uint8_t* w_down, int64_t n_expert, int64_t hidden,
                int64_t inter, int afmt, const uint8_t* hq, int64_t t,
                const int32_t* ids, int topk, float* d) {
  if (!pair_ok(wfmt, afmt, inter)) return -1;
  int64_t wrow = inter / or_block_elems(wfmt) * or_block_bytes(wfmt);
  int64_t arow = inter / or_block_elems(afmt) * or_block_bytes(afmt);
  int64_t np = t * topk;
  for (int64_t p = 0; p < np; p++)
    if (ids[p] < 0 || ids[p] >= n_expert) return -1;
  double* ha = (double*)malloc(sizeof(double) * (size_t)(np * inter + 1));
  for (int64_t p = 0; p < np; p++) dequant_row_f64(afmt, hq + p * arow, inter, ha + p * inter);
#pragma omp parallel
  {
    double* wd = (double*)malloc(sizeof(double) * (size_t)inter);
#pragma omp for schedule(static)
    for (int64_t idx = 0; idx < np * hidden; idx++) {
      int64_t p = idx / hidden, r = idx % hidden;
      dequant_row_f64(wfmt, w_down + ((int64_t)ids[p] * hidden + r) * wrow, inter, wd);
      d[p * hidden + r] = (float)dot64(wd, ha + p * inter, inter);
    }
    free(wd);
  }
  free(ha);
  return 0;
}

void or_moe_combine(const float* d, const float* w, int64_t t, int topk,
                    int64_t hidden, float* y) {
  for (int64_t tt = 0; tt < t; tt++)
    for (int64_t c = 0; c < hidden; c++) {
      double s = 0.0;
      for (int k = 0; k < topk; k++)
        s += (double)w[tt * topk + k] * (double)d[(tt * topk + k) * hidden + c];
      y[tt * hidden + c] = (float)s;
    }
}

int or_grouped(int wfmt, const uint8_t* W, int64_t n_expert, int64_t n, int64_t k,
               int afmt, const uint8_t* xq, int x_per_pair,
               const int32_t* ids, int64_t t, int topk, float* y) {
  if (!pair_ok(wfmt, afmt, k)) return -1;
  int64_t wrow = k / or_block_elems(wfmt) * or_block_bytes(wfmt);
  int64_t arow = k / or_block_elems(afmt) * or_block_bytes(afmt);
  int64_t np = t * topk, nx = x_per_pair ? np : t;
  for (int64_t p = 0; p < np; p++)
    if (ids[p] < 0 || ids[p] >= n_expert) return -1;
  double* xa = (double*)malloc(sizeof(double) * (size_t)(nx * k + 1));
  for (int64_t i = 0; i < nx; i++) dequant_row_f64(afmt, xq + i * arow, k, xa + i * k);
#pragma omp parallel
  {
    double* wr = (double*)malloc(sizeof(double) * (size_t)k);
#pragma omp for schedule(static)
    for (int64_t idx = 0; idx < np * n; idx++) {
      int64_t p = idx / n, r = idx % n;
      const double* x = xa + (x_per_pair ? p : p / topk) * k;
      dequant_row_f64(wfmt, W + ((int64_t)ids[p] * n + r) * wrow, k, wr);
      y[p * n + r] = (float)dot64(wr, x, k);
    }
    free(wr);
  }
  free(xa);
  return 0;
}
