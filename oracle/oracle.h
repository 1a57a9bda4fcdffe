/*
 * CPU oracle for the grouped routed-expert MoE decode step -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow C (C11, libm only, no SIMD, built with -O2 -fno-fast-math -ffp-contract=off).
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load it.
 * It shares no code, header, table or constant with the HIP library.
 *
 * Sources (the web pages this method is described on):
 *  [EXPDEC]  "#2058 Verify window: the routed experts' gate/up with the group's q8_1 rows in
 *            shared memory" -- sections "Why" (36-byte q8_1 blocks, grouping by expert),
 *            "Bit for bit" (entries of a group are independent).
 *  [GROUPED] "#363 experts: smaller and fewer launches for the verify window's PCIe call" --
 *            opening paragraph (cap_groups = window tokens x top-k), "What changes" (a call
 *            covers its own entries grp_start[0]..grp_start[n_groups]; SwiGLU product rounded
 *            on its own before the q8_1 block sums), "Exactness" (entries past 0, scattered
 *            destinations, rows a call must not write).
 *  [NIBBLE]  "#3455 GP100 (sm_60): 4-bit slots ..." -- "Validation" (gate, up, h, hq and the
 *            combined output compared stage by stage).
 * The pages give no byte layout for any weight format; the layouts implemented here are the
 * readings written down in the repository's design notes (header fp16 scale first). Q5_1 (named
 * among the down formats on [GROUPED] "Exactness") is an offset format: its block contribution
 * adds offset * f(s_x), the q8_1 sum field. NL4X (the IQ4_XS class on the same list) scales each
 * 32-weight sub-block by D (l - 32) with a 6-bit l.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>
#include <stddef.h>

enum { ORC_Q8_0 = 1, ORC_NL4 = 2, ORC_CB2 = 3, ORC_CB3 = 4, ORC_Q5_1 = 5, ORC_NL4X = 6 };

/* IEEE binary16 <-> binary32 (round to nearest even, subnormals kept). */
float    orc_h2f(uint16_t h);
uint16_t orc_f2h(float f);

/* Bytes per block and weights per block of a weight format; 0 for an unknown format. */
int orc_block_bytes(int fmt);
int orc_block_weights(int fmt);

/* q8_1 (36 B per 32 values: fp16 d, fp16 s, int8 q[32]) from float32, exactly in float32. */
void orc_quantize_q8_1(const float* x, int n, uint8_t* out);
/* Q8_0 (34 B per 32: fp16 d, int8 q[32]); used only for round-trip invariants. */
void orc_quantize_q8_0(const float* x, int n, uint8_t* out);

/* Decode one row of `ncols` weights: integer code per weight, scale and offset per 32-weight
 * sub-block (weight value = scale[j/32] * code[j] + offset[j/32]; offsets may be NULL, and are 0
 * except for Q5_1). Returns 0, or -1 for a bad format / shape. */
int orc_decode_row(int fmt, const uint8_t* row, int ncols, const int8_t* nl4_table,
                   const uint8_t* cb2_grid, const uint8_t* cb3_grid, int32_t* codes, double* scales,
                   double* offsets);

/* out[r] = sum over 32-blocks b of c_b, c_b = scale_w * f(d_x) * sum_j code_j * q_j
 * + offset_w * f(s_x) (double; the second term only for Q5_1, whose offset multiplies the block's
 * activation sum, read from the q8_1 sum field s), S[r] = sum_b of the terms' absolute values.
 * mat: rows x ncols weights, row-major blocks. xq: ncols/32 q8_1 blocks. */
int orc_matvec(int fmt, const uint8_t* mat, int rows, int ncols, const uint8_t* xq,
               const int8_t* nl4_table, const uint8_t* cb2_grid, const uint8_t* cb3_grid,
               double* out, double* S);

/* h = silu(g) * u, evaluated in float32 one operation at a time: e = expf(-g), den = 1 + e,
 * s = g / den, h = s * u, each result rounded to float32 ([GROUPED] "What changes": the product
 * is rounded on its own before the q8_1 block sums). expf overflows to +inf for g < -88.72, so h
 * is then a signed zero. */
void orc_swiglu(const float* g, const float* u, int n, float* h);

/* Per token: top-k experts by (logit descending, id ascending); weights are the softmax over the
 * whole row restricted to those k and renormalised (double). */
void orc_route_topk(const float* logits, int T, int E, int k, int32_t* ids, double* w);

/* Group the T*k (token, expert) entries by expert: groups ascending by expert id, entries within
 * a group ascending by token. Entry indices are absolute, starting at entry_base.
 * dst_of_token may be NULL (identity). Returns n_groups. Arrays ent_* are indexed by
 * (absolute entry index - entry_base). w may be NULL (weights then 0). */
int orc_build_plan(const int32_t* ids, const float* w, const int32_t* dst_of_token, int T, int k,
                   int E, int entry_base, int32_t* grp_expert, int32_t* grp_start, int32_t* ent_src,
                   int32_t* ent_dst, float* ent_w);

#endif
