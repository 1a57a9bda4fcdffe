/*
 * CPU oracle for the grouped routed-expert MoE decode step -- TEST INFRASTRUCTURE ONLY.
 * See oracle.h for the page citations. Every function is the plain definition, one value at a
 * time, in the order the definition states it; nothing is blocked, fused or reordered.
 * Parity pins: tests/test_oracle_*.py (golden hand-derived blocks, numpy float16 conversion,
 * dense float64 matmul equivalence, numpy lexsort/bincount, closed forms, brute force).
 */
#include "oracle.h"
#include <math.h>
#include <string.h>
#include <stdlib.h>

/* ---------------------------------------------------------------- binary16 ---------------- */

float orc_h2f(uint16_t h) {
  unsigned sign = h >> 15, ex = (h >> 10) & 31u, man = h & 1023u;
  double v;
  if (ex == 0) v = ldexp((double)man, -24);                    /* zero / subnormal */
  else if (ex == 31) v = man ? (double)NAN : (double)INFINITY;
  else v = ldexp((double)(man | 1024u), (int)ex - 25);         /* 1.man * 2^(ex-15) */
  return (float)(sign ? -v : v);
}

uint16_t orc_f2h(float f) {
  uint32_t bits;
  memcpy(&bits, &f, 4);
  uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
  if (isnan(f)) return (uint16_t)(sign | 0x7E00u);
  if (isinf(f)) return (uint16_t)(sign | 0x7C00u);
  double a = fabs((double)f);
  if (a == 0.0) return sign;
  int ex;
  frexp(a, &ex);                 /* a in [2^(ex-1), 2^ex) */
  int e = ex - 1;
  if (e < -14) e = -14;          /* below the normal range the quantum stays 2^-24 */
  double quantum = ldexp(1.0, e - 10);
  double r = nearbyint(a / quantum); /* exact quotient, then round half to even */
  uint32_t m = (uint32_t)r;      /* 0 .. 2048 */
  if (m >= 1024u) {
    if (m == 2048u) { m = 1024u; e += 1; }
    int ef = e + 15;
    if (ef >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | ((uint32_t)ef << 10) | (m - 1024u));
  }
  return (uint16_t)(sign | m);   /* subnormal (or zero after rounding) */
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t* p, uint16_t v) { p[0] = (uint8_t)(v & 0xFF); p[1] = (uint8_t)(v >> 8); }

/* ---------------------------------------------------------------- formats ----------------- */

int orc_block_bytes(int fmt) {
  switch (fmt) {
    case ORC_Q8_0: return 34;
    case ORC_NL4: return 18;
    case ORC_CB2: return 70;
    case ORC_CB3: return 110;
    case ORC_Q5_1: return 24;
    case ORC_NL4X: return 136;
    default: return 0;
  }
}

int orc_block_weights(int fmt) {
  switch (fmt) {
    case ORC_Q8_0: case ORC_NL4: case ORC_Q5_1: return 32;
    case ORC_CB2: case ORC_CB3: case ORC_NL4X: return 256;
    default: return 0;
  }
}

/* 4-bit sub-scale s of 32-weight sub-block `sub` (0..7) of a 256-weight super-block; the
 * multiplier applied to the super-block scale is the odd number 2s+1. */
static int sub_scale(const uint8_t* nibbles, int sub) {
  return (nibbles[sub / 2] >> (4 * (sub % 2))) & 15;
}

/* Decode weights [32*sb32, 32*sb32+32) of a row: integer codes, the sub-block's scale and its
 * additive offset (weight = scale * code + offset; the offset is 0 except for Q5_1). */
static void decode_sub32(int fmt, const uint8_t* row, int sb32, const int8_t* nl4_table,
                         const uint8_t* cb2_grid, const uint8_t* cb3_grid, int32_t code[32],
                         double* scale, double* offset) {
  *offset = 0.0;
  if (fmt == ORC_Q5_1) {
    const uint8_t* blk = row + 24 * sb32;
    *scale = (double)orc_h2f(rd16(blk));
    *offset = (double)orc_h2f(rd16(blk + 2));
    uint32_t qh = (uint32_t)blk[4] | ((uint32_t)blk[5] << 8) | ((uint32_t)blk[6] << 16) |
                  ((uint32_t)blk[7] << 24);
    for (int i = 0; i < 16; ++i) {
      code[i] = (blk[8 + i] & 15) | (int)(((qh >> i) & 1u) << 4);              /* weight i */
      code[i + 16] = (blk[8 + i] >> 4) | (int)(((qh >> (i + 16)) & 1u) << 4);  /* weight i+16 */
    }
  } else if (fmt == ORC_NL4X) {
    const uint8_t* blk = row + 136 * (sb32 / 8);
    int sub = sb32 % 8;
    /* 6-bit sub-block scale: low 4 bits from the nibble bytes at [4:8] (sub-block 2j in the low
     * nibble of byte 4 + j, 2j+1 in the high one), high 2 bits from the 16-bit word at [2:4]
     * (bits 2 sub, 2 sub + 1); the sub-block's scale is D * (l - 32) */
    int lo = (blk[4 + sub / 2] >> (4 * (sub % 2))) & 15;
    int hi = (rd16(blk + 2) >> (2 * sub)) & 3;
    int l = lo | (hi << 4);
    *scale = (double)orc_h2f(rd16(blk)) * (double)(l - 32);
    const uint8_t* q = blk + 8 + 16 * sub;
    for (int i = 0; i < 16; ++i) {
      code[i] = nl4_table[q[i] & 15];        /* low nibble: weight i of the sub-block */
      code[i + 16] = nl4_table[q[i] >> 4];   /* high nibble: weight i + 16 */
    }
  } else if (fmt == ORC_Q8_0) {
    const uint8_t* blk = row + 34 * sb32;
    *scale = (double)orc_h2f(rd16(blk));
    for (int j = 0; j < 32; ++j) code[j] = (int8_t)blk[2 + j];
  } else if (fmt == ORC_NL4) {
    const uint8_t* blk = row + 18 * sb32;
    *scale = (double)orc_h2f(rd16(blk));
    for (int i = 0; i < 16; ++i) {
      code[i] = nl4_table[blk[2 + i] & 15];       /* low nibble: weight i */
      code[i + 16] = nl4_table[blk[2 + i] >> 4];  /* high nibble: weight i+16 */
    }
  } else if (fmt == ORC_CB2) {
    const uint8_t* blk = row + 70 * (sb32 / 8);
    int sub = sb32 % 8;
    double D = (double)orc_h2f(rd16(blk));
    *scale = D * (double)(2 * sub_scale(blk + 66, sub) + 1);
    for (int w = 0; w < 32; ++w) {
      int i = 32 * sub + w;                 /* weight index inside the super-block */
      int g = i / 8, j = i % 8;             /* 8-weight group and position in it */
      int mag = cb2_grid[8 * blk[2 + g] + j];
      int neg = (blk[34 + g] >> j) & 1;
      code[w] = neg ? -mag : mag;
    }
  } else { /* ORC_CB3 */
    const uint8_t* blk = row + 110 * (sb32 / 8);
    int sub = sb32 % 8;
    double D = (double)orc_h2f(rd16(blk));
    *scale = D * (double)(2 * sub_scale(blk + 106, sub) + 1);
    for (int w = 0; w < 32; ++w) {
      int i = 32 * sub + w;
      int g = i / 4, j = i % 4;             /* 4-weight group: 9-bit grid index */
      int idx = blk[2 + g] | (((blk[66 + g / 8] >> (g % 8)) & 1) << 8);
      int mag = cb3_grid[4 * idx + j];
      int neg = (blk[74 + i / 8] >> (i % 8)) & 1;
      code[w] = neg ? -mag : mag;
    }
  }
}

static int shape_ok(int fmt, int ncols) {
  int bw = orc_block_weights(fmt);
  return bw > 0 && ncols > 0 && ncols % bw == 0;
}

int orc_decode_row(int fmt, const uint8_t* row, int ncols, const int8_t* nl4_table,
                   const uint8_t* cb2_grid, const uint8_t* cb3_grid, int32_t* codes, double* scales,
                   double* offsets) {
  if (!shape_ok(fmt, ncols)) return -1;
  for (int b = 0; b < ncols / 32; ++b) {
    double off;
    decode_sub32(fmt, row, b, nl4_table, cb2_grid, cb3_grid, codes + 32 * b, scales + b, &off);
    if (offsets) offsets[b] = off;
  }
  return 0;
}

/* ---------------------------------------------------------------- quantizers -------------- */

void orc_quantize_q8_1(const float* x, int n, uint8_t* out) {
  for (int b = 0; b < n / 32; ++b) {
    const float* xb = x + 32 * b;
    uint8_t* ob = out + 36 * b;
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
      float a = fabsf(xb[i]);
      if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    int isum = 0;
    for (int i = 0; i < 32; ++i) {
      int q = 0;
      if (amax != 0.0f) {
        float r = roundf(xb[i] / d);   /* half away from zero */
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q = (int)r;
      }
      ob[4 + i] = (uint8_t)(int8_t)q;
      isum += q;
    }
    uint16_t d16 = orc_f2h(d);
    float s = orc_h2f(d16) * (float)isum;
    wr16(ob, d16);
    wr16(ob + 2, orc_f2h(s));
  }
}

void orc_quantize_q8_0(const float* x, int n, uint8_t* out) {
  for (int b = 0; b < n / 32; ++b) {
    const float* xb = x + 32 * b;
    uint8_t* ob = out + 34 * b;
    float amax = 0.0f;
    for (int i = 0; i < 32; ++i) {
      float a = fabsf(xb[i]);
      if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    for (int i = 0; i < 32; ++i) {
      int q = 0;
      if (amax != 0.0f) {
        float r = roundf(xb[i] / d);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q = (int)r;
      }
      ob[2 + i] = (uint8_t)(int8_t)q;
    }
    wr16(ob, orc_f2h(d));
  }
}

/* ---------------------------------------------------------------- block dot --------------- */

int orc_matvec(int fmt, const uint8_t* mat, int rows, int ncols, const uint8_t* xq,
               const int8_t* nl4_table, const uint8_t* cb2_grid, const uint8_t* cb3_grid,
               double* out, double* S) {
  if (!shape_ok(fmt, ncols) || rows < 0) return -1;
  size_t row_bytes = (size_t)(ncols / orc_block_weights(fmt)) * (size_t)orc_block_bytes(fmt);
  int32_t code[32];
  for (int r = 0; r < rows; ++r) {
    const uint8_t* row = mat + (size_t)r * row_bytes;
    double acc = 0.0, sabs = 0.0;
    for (int b = 0; b < ncols / 32; ++b) {
      double scale, offset;
      decode_sub32(fmt, row, b, nl4_table, cb2_grid, cb3_grid, code, &scale, &offset);
      const uint8_t* xb = xq + 36 * b;
      double dx = (double)orc_h2f(rd16(xb));
      long isum = 0;
      for (int j = 0; j < 32; ++j) isum += (long)code[j] * (long)(int8_t)xb[4 + j];
      double c = scale * dx * (double)isum;
      /* an offset weight adds offset * sum of the block's activations, taken from the q8_1 sum
       * field s = fp16(f(d) * sum q) */
      double co = offset * (double)orc_h2f(rd16(xb + 2));
      acc += c + co;
      sabs += fabs(c) + fabs(co);
    }
    out[r] = acc;
    if (S) S[r] = sabs;
  }
  return 0;
}

/* ---------------------------------------------------------------- SwiGLU ------------------ */

void orc_swiglu(const float* g, const float* u, int n, float* h) {
  for (int i = 0; i < n; ++i) {
    /* float32 throughout, one rounding per operation in this order (no contraction: the file is
     * built with -ffp-contract=off); expf is libm's single-precision exponential */
    float e = expf(-g[i]);
    float den = 1.0f + e;
    float silu = g[i] / den;
    h[i] = silu * u[i];
  }
}

/* ---------------------------------------------------------------- routing ----------------- */

void orc_route_topk(const float* logits, int T, int E, int k, int32_t* ids, double* w) {
  double* p = (double*)malloc(sizeof(double) * (size_t)(E > 0 ? E : 1));
  char* taken = (char*)malloc((size_t)(E > 0 ? E : 1));
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    /* softmax over the whole row */
    double m = -INFINITY;
    for (int e = 0; e < E; ++e) if ((double)l[e] > m) m = (double)l[e];
    double z = 0.0;
    for (int e = 0; e < E; ++e) { p[e] = exp((double)l[e] - m); z += p[e]; }
    for (int e = 0; e < E; ++e) p[e] /= z;
    /* top-k: softmax is monotone in the logit, so rank by (logit desc, id asc) */
    memset(taken, 0, (size_t)E);
    double sel = 0.0;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;  /* strict: equal logits keep the lower id */
      }
      taken[best] = 1;
      ids[t * k + j] = best;
      sel += p[best];
    }
    /* renormalise over the k selected */
    for (int j = 0; j < k; ++j) w[t * k + j] = p[ids[t * k + j]] / sel;
  }
  free(p);
  free(taken);
}

int orc_build_plan(const int32_t* ids, const float* w, const int32_t* dst_of_token, int T, int k,
                   int E, int entry_base, int32_t* grp_expert, int32_t* grp_start, int32_t* ent_src,
                   int32_t* ent_dst, float* ent_w) {
  for (int i = 0; i < T * k; ++i)
    if (ids[i] < 0 || ids[i] >= E) return -1;
  int* cnt = (int*)calloc((size_t)E, sizeof(int));
  int* fill = (int*)calloc((size_t)E, sizeof(int));
  for (int i = 0; i < T * k; ++i) cnt[ids[i]]++;
  int ng = 0, pos = 0;
  for (int e = 0; e < E; ++e) {       /* groups ascending by expert id */
    if (cnt[e] == 0) continue;
    grp_expert[ng] = e;
    grp_start[ng] = entry_base + pos;
    fill[e] = pos;
    pos += cnt[e];
    ++ng;
  }
  grp_start[ng] = entry_base + pos;
  for (int t = 0; t < T; ++t) {       /* tokens ascending inside each group */
    for (int j = 0; j < k; ++j) {
      int e = ids[t * k + j];
      int p = fill[e]++;
      ent_src[p] = t;
      ent_dst[p] = dst_of_token ? dst_of_token[t] : t;
      ent_w[p] = w ? w[t * k + j] : 0.0f;
    }
  }
  free(cnt);
  free(fill);
  return ng;
}
