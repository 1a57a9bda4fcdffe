// Device building blocks for the grouped routed-expert decode kernels (gfx950, wave64).
//
// * binary16 helpers and the q8_1 block quantizer (bit-exact IEEE float32: d = amax / 127,
//   q = x / d rounded half away from zero, clamped to +-127; s = fp16(f(d16) * sum q)). The
//   36-byte q8_1 block is the activation format of "#2058 Verify window: the routed experts'
//   gate/up with the group's q8_1 rows in shared memory", section "Why"; the rounding rule is the
//   library's reading of a quantizer the pages leave unstated.
// * SwiGLU rounded op by op in float32 ("#363 experts: smaller and fewer launches for the verify
//   window's PCIe call", "What changes": the product is rounded on its own before the q8_1 sums).
// * Weight decoders that read a weight unit (32 weights) out of a byte image staged in LDS, at any
//   byte alignment, and return eight dwords of int8 codes plus the unit's float scale.
// * Fixed-order cross-lane sums (DPP), so every kernel variant reduces a row in the same order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_LDS __attribute__((address_space(3)))

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace moe {

constexpr int kThreads = 256;          // the small kernels (quantize, SwiGLU, repack, scatter): 4 waves of 64
constexpr int kMaxSlots = 4;           // entries staged at once (a group's rows of the window)

enum Fmt : int { Q8_0 = 1, NL4 = 2, CB2 = 3, CB3 = 4, Q5_1 = 5, NL4X = 6 };

// ------------------------------------------------------------------ binary16 ----------------

__device__ __forceinline__ float h2f(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ uint32_t f2h(float f) {   // round to nearest even, subnormals kept
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// ------------------------------------------------------------------ q8_1 ---------------------

// A block's scale d = amax / 127 and what quant_code needs besides it: rd = rcp(d), and whether
// d is in the range where x rd is accurate (2^-100 <= d <= 2^100; false for 0, inf and NaN).
struct QScale {
  float d, rd;
  bool ok;
};
__device__ __forceinline__ QScale q_scale(float amax) {
  QScale s;
  s.d = amax / 127.0f;
  s.rd = __builtin_amdgcn_rcpf(s.d);
  s.ok = s.d >= 0x1p-100f && s.d <= 0x1p100f;
  return s;
}

// The code of a quotient y: rounded to the nearest integer, halves away from zero, clamped to +-127.
__device__ __forceinline__ int code_of(float y) {
  const float t = __builtin_truncf(y);
  float r = __builtin_fabsf(y - t) >= 0.5f ? t + __builtin_copysignf(1.0f, y) : t;   // y - t is exact
  r = r > 127.0f ? 127.0f : r;
  r = r < -127.0f ? -127.0f : r;
  return (int)r;
}

// The codes of x0..x3 in a block of scale s (|x| <= amax), packed little-endian: code_of(x / d)
// with x / d the correctly rounded float32 quotient, as the definition has it, but without a
// division in the common case. y = x rd is within 2^-15 of x / d (rcp is good to 1 ulp, the product
// to half an ulp, and |x / d| < 128) and the rounded quotient within 2^-18 of x / d. While y is more
// than 2^-14 from every half-integer, both lie strictly between the same two, so the code is
// trunc(y + copysign(1/2, y)) (that sum is off by at most 2^-17, and no clamp is needed below
// 127.5). A lane with some y + copysign(1/2, y) within 2^-13 of an integer (rare), and every lane
// of a block whose scale is out of range, redoes its four with the division.
__device__ __forceinline__ uint32_t quant_pack4(const float (&x)[4], const QScale& s) {
  uint32_t packed = 0;
  float gap = 1.0f;   // the least distance of a z from an integer (a NaN z gives code 0 either way)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float y = x[j] * s.rd;
    const float z = y + __builtin_copysignf(0.5f, y);
    gap = __builtin_fminf(gap, __builtin_fabsf(z - __builtin_rintf(z)));
    packed |= ((uint32_t)(int)z & 0xFFu) << (8 * j);
  }
  if (!s.ok || gap <= 0x1p-13f) {
    packed = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) packed |= ((uint32_t)code_of(x[j] / s.d) & 0xFFu) << (8 * j);
  }
  return packed;
}
// One code, as quant_pack4.
__device__ __forceinline__ int quant_code(float x, const QScale& s) {
  const float y = x * s.rd;
  const float z = y + __builtin_copysignf(0.5f, y);
  return (!s.ok || !(__builtin_fabsf(z - __builtin_rintf(z)) > 0x1p-13f)) ? code_of(x / s.d) : (int)z;
}

// s16 = fp16(f(d16) * isum). The product is exact in float32 (11 x 12 bits), so rounding it once
// to fp16 is the whole story except for the sign of a zero product: IEEE gives -0 when d16 is
// +0 and isum < 0. That case is set explicitly, whatever instruction the compiler picks for the
// multiply + convert.
__device__ __forceinline__ uint32_t sum_field(uint32_t d16, int isum) {
  uint32_t s = f2h(h2f(d16) * (float)isum);
  if (d16 == 0 && isum < 0) s = 0x8000u;
  return s;
}

// One 32-value block: q[0..7] = the 32 int8 codes packed little-endian, d = f(d16) as float,
// d16 / s16 = the stored fp16 fields.
struct QBlock {
  uint32_t q[8];
  float d;
  uint32_t d16, s16;
};

__device__ __forceinline__ QBlock quant_block(const float v[32]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float a = __builtin_fabsf(v[i]);
    amax = a > amax ? a : amax;
  }
  const QScale qs = q_scale(amax);
  const float d = qs.d;
  QBlock b;
  int isum = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const float x4[4] = {v[4 * w], v[4 * w + 1], v[4 * w + 2], v[4 * w + 3]};
    const uint32_t packed = amax != 0.0f ? quant_pack4(x4, qs) : 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) isum += (int)(int8_t)(packed >> (8 * j));
    b.q[w] = packed;
  }
  b.d16 = f2h(d);
  b.d = h2f(b.d16);
  b.s16 = sum_field(b.d16, isum);
  return b;
}

// h = silu(g) * u with every operation a float32 rounding, in this order.
__device__ __forceinline__ float swiglu(float g, float u) {
  float den = 1.0f + expf(-g);
  float s = g / den;
  return s * u;
}

// ------------------------------------------------------------------ cross-lane sums ---------

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, false));
}

// Sum over aligned groups of L lanes (L a power of two, 1..64); every lane of a group ends with
// the same value (each step adds two equal partial sums in either order, which is exact-
// commutative), so the result is a fixed function of the L inputs.
__device__ __forceinline__ float group_sum(float v, int L) {
  if (L >= 2) v = v + dpp<0xB1>(v);    // quad_perm [1,0,3,2]  (xor 1)
  if (L >= 4) v = v + dpp<0x4E>(v);    // quad_perm [2,3,0,1]  (xor 2)
  if (L >= 8) v = v + dpp<0x141>(v);   // row_half_mirror      (quad <-> quad)
  if (L >= 16) v = v + dpp<0x140>(v);  // row_mirror           (half-row <-> half-row)
  if (L >= 32) v = v + __shfl_xor(v, 16);
  if (L >= 64) v = v + __shfl_xor(v, 32);
  return v;
}

// Max and integer sum over aligned groups of 32 lanes. Within a row of 16 lanes the partners come
// from DPP moves (pairs, then pairs of pairs, then the mirrored half-row and row), which pair every
// lane with every other lane of its row once; only the step across rows goes through a lane
// shuffle. Both results do not depend on the order of the steps.
__device__ __forceinline__ float wave_max32(float v) {
  float o = dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v = o > v ? o : v;
  o = dpp<0x4E>(v);          // quad_perm [2,3,0,1]
  v = o > v ? o : v;
  o = dpp<0x141>(v);         // row_half_mirror
  v = o > v ? o : v;
  o = dpp<0x140>(v);         // row_mirror
  v = o > v ? o : v;
  o = __shfl_xor(v, 16);
  return o > v ? o : v;
}
__device__ __forceinline__ int wave_sum32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  return v + __shfl_xor(v, 16);
}

// ------------------------------------------------------------------ LDS byte images ---------

// Little-endian dword starting at any byte offset of an LDS image (reads two aligned dwords; the
// image keeps 16 bytes of slack after its end for this).
__device__ __forceinline__ uint32_t ldw(const MOE_LDS uint32_t* W, uint32_t off) {
  const uint32_t i = off >> 2;
  return __builtin_amdgcn_alignbyte(W[i + 1], W[i], off & 3u);
}

struct Tables {
  uint32_t nl4[4];                       // NL4 table, in VGPRs (tables_init)
  uint32_t k7, k8, k4;                   // byte-lane constants, in VGPRs (tables_init)
  const MOE_LDS uint32_t* cb2;           // 256 x 8 B grid in LDS (2 dwords per row)
  const MOE_LDS uint32_t* cb3;           // 512 x 4 B grid in LDS (1 dword per row)
};

// Put a value in a VGPR the compiler treats as opaque: the lookup below then reads its table and
// masks from VGPRs (one VOP3 may read only one SGPR or literal on this target), with no copies
// rematerialised inside the loops.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(v));
  return r;
}

__device__ __forceinline__ void tables_init(Tables& tb, const uint32_t nl4[4], const MOE_LDS uint32_t* cb2,
                                            const MOE_LDS uint32_t* cb3) {
  tb.nl4[0] = in_vgpr(nl4[0]);
  tb.nl4[1] = in_vgpr(nl4[1]);
  tb.nl4[2] = in_vgpr(nl4[2]);
  tb.nl4[3] = in_vgpr(nl4[3]);
  tb.k7 = in_vgpr(0x07070707u);
  tb.k8 = in_vgpr(0x08080808u);
  tb.k4 = in_vgpr(0x04040404u);
  tb.cb2 = cb2;
  tb.cb3 = cb3;
}

// 16-entry int8 lookup of the four 4-bit codes in bits 0-3 of each byte of c (bits 4-7 ignored)
// with v_perm: entries 0-7 and 8-15 are looked up separately and merged by the code's bit 3
// (selector byte 4 picks byte 0 of 0xFFFFFFFF, selector 12 yields 0x00).
__device__ __forceinline__ uint32_t lut16(uint32_t c, const Tables& tb) {
  const uint32_t s = c & tb.k7;
  const uint32_t lo = __builtin_amdgcn_perm(tb.nl4[1], tb.nl4[0], s);
  const uint32_t hi = __builtin_amdgcn_perm(tb.nl4[3], tb.nl4[2], s);
  const uint32_t m = __builtin_amdgcn_perm(0xFFFFFFFFu, 0u, (c & tb.k8) | tb.k4);
  return (lo & m) | (hi & ~m);
}

// Negate the bytes of `mag` (each 1..15) selected by the low 4 bits of `nib` (bit j -> byte j).
__device__ __forceinline__ uint32_t apply_sign(uint32_t mag, uint32_t nib) {
  const uint32_t t = (nib * 0x00204081u) & 0x01010101u;   // bit j -> bit 0 of byte j
  const uint32_t m = (t << 8) - t;                          // 0xFF in selected bytes
  return (mag ^ m) + t;                                     // ~mag + 1 per selected byte
}


// Where a row's fields sit: for block b of the row (b = u for Q8_0 / NL4, u / 8 for CB2 / CB3) the
// fp16 scale at d_a b + d_b, the codes at c_a b + c_b and (CB2 / CB3) the packed sub-scales at
// x_a b + x_b, byte offsets from the row's start. The row-major layout interleaves them block by
// block; the planar layout (same bytes per row) puts every block's codes first, then the scales.
struct Lay {
  uint32_t d_a, d_b, c_a, c_b, x_a, x_b;
};

__host__ __device__ constexpr int block_bytes(int fmt) {
  return fmt == Q8_0 ? 34 : fmt == NL4 ? 18 : fmt == CB2 ? 70 : fmt == CB3 ? 110 : fmt == Q5_1 ? 24
         : fmt == NL4X ? 136 : 0;
}
__host__ __device__ constexpr int block_weights(int fmt) {
  return (fmt == CB2 || fmt == CB3 || fmt == NL4X) ? 256 : 32;
}
// Header bytes of a block before its codes: the fp16 scale (Q5_1: scale and offset; NL4X: scale,
// then the 16-bit and 32-bit words of its sub-block scales).
__host__ __device__ constexpr int head_bytes(int fmt) { return fmt == Q5_1 ? 4 : fmt == NL4X ? 8 : 2; }
// Code bytes of one block: the block minus its header and (CB2 / CB3) its 4 trailing sub-scale
// bytes.
__host__ __device__ constexpr int code_bytes(int fmt) {
  return block_bytes(fmt) - head_bytes(fmt) - ((fmt == CB2 || fmt == CB3) ? 4 : 0);
}
// The field map of a row of nblk blocks in either layout.
__host__ __device__ inline Lay make_lay(int fmt, int nblk, bool planar) {
  const uint32_t B = (uint32_t)block_bytes(fmt), C = (uint32_t)code_bytes(fmt), n = (uint32_t)nblk;
  const uint32_t H = (uint32_t)head_bytes(fmt);
  if (!planar) return Lay{B, 0u, B, H, B, B - 4u};
  return Lay{B - C, C * n, C, 0u, B - C, C * n + H};
}

// A weight unit (32 weights, u = 32-weight index inside its row) is read from LDS in two steps so
// that the reads of the next unit can be in flight while this one is decoded: unit_load issues the
// aligned dword reads covering the unit's fields, unit_decode turns them into codes. c[k] holds the
// codes of weights 4k..4k+3 of the unit, sc the unit's scale.
template <int FMT>
struct URaw {
  // Q8_0: scale pair, 9 quant dwords; NL4: scale pair, 5 nibble dwords; CB2: D, index, sign and
  // sub-scale pairs; CB3: D, two index pairs, high-bit, sign and sub-scale pairs
  // Q5_1: scale and offset pair, 6 dwords of high bits and nibbles; NL4X: 3 header dwords, 5 of
  // the sub-block's nibbles
  uint32_t v[FMT == Q8_0 ? 11 : FMT == NL4 ? 7 : FMT == CB2 ? 8 : FMT == Q5_1 ? 8 : FMT == NL4X ? 8 : 12];
  uint32_t od, oc, ox;   // byte offsets of the block's scale, codes and (CB2 / CB3) sub-scales
};

template <int FMT>
__device__ __forceinline__ void unit_load(const MOE_LDS uint32_t* W, uint32_t row, int u, const Lay& ly,
                                          URaw<FMT>& r) {
  auto pair = [&](int j, uint32_t off) {
    r.v[2 * j] = W[off >> 2];
    r.v[2 * j + 1] = W[(off >> 2) + 1];
  };
  if constexpr (FMT == Q8_0 || FMT == NL4 || FMT == Q5_1) {
    const uint32_t b = (uint32_t)u;
    r.od = row + ly.d_a * b + ly.d_b;
    r.oc = row + ly.c_a * b + ly.c_b;
    r.ox = 0;
    pair(0, r.od);
    const uint32_t c = r.oc >> 2;
#pragma unroll
    for (int i = 0; i < (FMT == Q8_0 ? 9 : FMT == NL4 ? 5 : 6); ++i) r.v[2 + i] = W[c + i];
  } else if constexpr (FMT == NL4X) {
    const uint32_t b = (uint32_t)u >> 3, su = (uint32_t)u & 7u;
    r.od = row + ly.d_a * b + ly.d_b;
    r.oc = row + ly.c_a * b + ly.c_b + 16u * su;   // this sub-block's 16 nibble bytes
    r.ox = 0;
    const uint32_t h = r.od >> 2;
#pragma unroll
    for (int i = 0; i < 3; ++i) r.v[i] = W[h + i];
    const uint32_t c = r.oc >> 2;
#pragma unroll
    for (int i = 0; i < 5; ++i) r.v[3 + i] = W[c + i];
  } else if constexpr (FMT == CB2) {
    const uint32_t b = (uint32_t)u >> 3, su = (uint32_t)u & 7u;
    r.od = row + ly.d_a * b + ly.d_b;
    r.oc = row + ly.c_a * b + ly.c_b;
    r.ox = row + ly.x_a * b + ly.x_b;
    pair(0, r.od);
    pair(1, r.oc + 4 * su);
    pair(2, r.oc + 32 + 4 * su);
    pair(3, r.ox);
  } else {  // CB3
    const uint32_t b = (uint32_t)u >> 3, su = (uint32_t)u & 7u;
    r.od = row + ly.d_a * b + ly.d_b;
    r.oc = row + ly.c_a * b + ly.c_b;
    r.ox = row + ly.x_a * b + ly.x_b;
    pair(0, r.od);
    pair(1, r.oc + 8 * su);
    pair(2, r.oc + 4 + 8 * su);
    pair(3, r.oc + 64 + su);
    pair(4, r.oc + 72 + 4 * su);
    pair(5, r.ox);
  }
}

// mo: the block's additive offset (Q5_1; 0 for the other formats): weight = sc * code + mo.
template <int FMT>
__device__ __forceinline__ void unit_decode(const URaw<FMT>& r, int u, const Tables& tb, uint32_t c[8], float& sc,
                                            float& mo) {
  // the dword at byte offset off of a pair read from off & ~3
  auto at = [&](int j, uint32_t off) { return __builtin_amdgcn_alignbyte(r.v[2 * j + 1], r.v[2 * j], off & 3u); };
  mo = 0.0f;
  if constexpr (FMT == Q5_1) {
    const uint32_t dm = at(0, r.od);
    sc = h2f(dm & 0xFFFFu);
    mo = h2f(dm >> 16);
    const uint32_t sh = r.oc & 3u;
    const uint32_t qh = __builtin_amdgcn_alignbyte(r.v[3], r.v[2], sh);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t n = __builtin_amdgcn_alignbyte(r.v[4 + k], r.v[3 + k], sh);   // nibbles of weights 4k.., 16+4k..
      const uint32_t hl = (((qh >> (4 * k)) & 15u) * 0x00204081u) & 0x01010101u;       // bit j -> bit 0 of byte j
      const uint32_t hh = (((qh >> (16 + 4 * k)) & 15u) * 0x00204081u) & 0x01010101u;
      c[k] = (n & 0x0F0F0F0Fu) | (hl << 4);              // weights 4k..4k+3
      c[k + 4] = ((n >> 4) & 0x0F0F0F0Fu) | (hh << 4);   // weights 16+4k..16+4k+3
    }
  } else if constexpr (FMT == NL4X) {
    // header: fp16 D, 16-bit word of the sub-scales' high bit pairs, 32-bit word of their low
    // nibbles; sub-block su's 6-bit scale l gives D (l - 32)
    const uint32_t ha = r.od & 3u;
    const uint32_t w0 = __builtin_amdgcn_alignbyte(r.v[1], r.v[0], ha);   // D | high pairs << 16
    const uint32_t w1 = __builtin_amdgcn_alignbyte(r.v[2], r.v[1], ha);   // low nibbles
    const uint32_t su = (uint32_t)u & 7u;
    const int l = (int)(((w1 >> (4u * su)) & 15u) | (((w0 >> (16u + 2u * su)) & 3u) << 4));
    sc = h2f(w0 & 0xFFFFu) * (float)(l - 32);
    const uint32_t sh = r.oc & 3u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t n = __builtin_amdgcn_alignbyte(r.v[4 + k], r.v[3 + k], sh);
      c[k] = lut16(n, tb);            // weights 4k..4k+3 of the sub-block (low nibbles)
      c[k + 4] = lut16(n >> 4, tb);   // weights 16+4k..16+4k+3 (high nibbles)
    }
  } else if constexpr (FMT == Q8_0) {
    sc = h2f(at(0, r.od) & 0xFFFFu);
    const uint32_t sh = r.oc & 3u;
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_alignbyte(r.v[3 + k], r.v[2 + k], sh);
  } else if constexpr (FMT == NL4) {
    sc = h2f(at(0, r.od) & 0xFFFFu);
    const uint32_t sh = r.oc & 3u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t n = __builtin_amdgcn_alignbyte(r.v[3 + k], r.v[2 + k], sh);
      c[k] = lut16(n, tb);            // weights 4k..4k+3 (low nibbles)
      c[k + 4] = lut16(n >> 4, tb);   // weights 16+4k..16+4k+3 (high nibbles)
    }
  } else if constexpr (FMT == CB2) {
    const uint32_t su = (uint32_t)u & 7u;
    const float D = h2f(at(0, r.od) & 0xFFFFu);
    const uint32_t idx4 = at(1, r.oc + 4 * su);
    const uint32_t sg4 = at(2, r.oc + 32 + 4 * su);
    const uint32_t s = (at(3, r.ox) >> (4 * su)) & 15u;
    sc = D * (float)(2 * s + 1);
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const uint32_t idx = (idx4 >> (8 * gq)) & 0xFFu;
      const uint32_t sg = (sg4 >> (8 * gq)) & 0xFFu;
      c[2 * gq] = apply_sign(tb.cb2[2 * idx], sg & 15u);
      c[2 * gq + 1] = apply_sign(tb.cb2[2 * idx + 1], sg >> 4);
    }
  } else {  // CB3
    const uint32_t su = (uint32_t)u & 7u;
    const float D = h2f(at(0, r.od) & 0xFFFFu);
    const uint32_t lo0 = at(1, r.oc + 8 * su);
    const uint32_t lo1 = at(2, r.oc + 4 + 8 * su);
    const uint32_t hib = at(3, r.oc + 64 + su);
    const uint32_t sg4 = at(4, r.oc + 72 + 4 * su);
    const uint32_t s = (at(5, r.ox) >> (4 * su)) & 15u;
    sc = D * (float)(2 * s + 1);
#pragma unroll
    for (int gq = 0; gq < 8; ++gq) {
      const uint32_t lo = ((gq < 4 ? lo0 : lo1) >> (8 * (gq & 3))) & 0xFFu;
      const uint32_t idx = lo | (((hib >> gq) & 1u) << 8);
      c[gq] = apply_sign(tb.cb3[idx], (sg4 >> (4 * gq)) & 15u);
    }
  }
}

}  // namespace moe
