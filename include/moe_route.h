/*
 * moe_route.h -- grouped routed-expert MoE decode for one MI355X (gfx950), C ABI.
 *
 * The operation (from the pages this method is described on):
 *   "#363 experts: smaller and fewer launches for the verify window's PCIe call", opening
 *   paragraph: a verify window of T tokens with top-k routing has up to cap_groups = T x k
 *   (expert) groups; the grouped gate/up and down kernels run one group per block row, with
 *   n_groups read on the device. "What changes": group g runs in block row g % gridDim.y and the
 *   results do not depend on the grid; SwiGLU and the q8_1 quantization run in one kernel over the
 *   call's own entries [grp_start[0], grp_start[n_groups]), the SwiGLU product rounded on its own
 *   before the q8_1 block sums. "Exactness": entries may start past index 0, destinations may be
 *   scattered, stale scratch must not matter, rows a call must not write keep their contents.
 *   "#2058 Verify window: the routed experts' gate/up with the group's q8_1 rows in shared
 *   memory", "Why": each expert's weights are decoded once per group and applied to the group's
 *   1-4 entries, whose 36-byte q8_1 activation rows are staged on chip.
 *
 * Conventions for every entry point:
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only enqueues work on it:
 *    no call allocates, frees, synchronises or reads device memory from the host, so every call
 *    can be captured into a HIP graph.
 *  - Pointers are device pointers unless a comment says "host". The caller owns all memory.
 *  - Return value: MOE_OK (0) or a negative moe_status for a problem the host can see (null
 *    pointer, bad shape or format, a HIP launch error). Problems only the device can see (an
 *    expert id, token or destination out of range, n_groups above cap_groups, a bounded wait that
 *    ran out) make the device skip that group or entry and OR a bit into *plan->err
 *    (MOE_ERR_* below); nothing traps. Nothing prints either, unless MOE_ROUTE_VERBOSE is set in
 *    the environment: then each distinct kernel choice of a launch (role, weight format and
 *    layout, kernel instance, grid, LDS, stream shape) is noted once on stderr.
 *  - Results are bit-identical for every grid_limit (0 = automatic) and between
 *    moe_layer_decode and the composed calls quantize -> gate_up -> swiglu -> down_scatter.
 *
 * Weight formats (the pages name the formats but print no layout; these are the layouts this
 * library reads, all little-endian, blocks packed with no padding, fp16 scale first):
 *   Q8_0  34 B / 32 w : [0:2] fp16 d, [2:34] int8 q[32]; w_j = d * q_j.
 *   NL4   18 B / 32 w : [0:2] fp16 d, [2:18] b[16]; code of w_i = T[b[i] & 15], of w_(i+16) =
 *                       T[b[i] >> 4]; T = 16-entry int8 table (nl4_table); w = d * code.
 *   CB2   70 B / 256 w: [0:2] fp16 D, [2:34] idx[32] (8-weight groups), [34:66] sign bytes (bit j
 *                       of byte g set = weight 8g+j negative), [66:70] eight 4-bit sub-scales s_b
 *                       (sub-block b = weights 32b..32b+31, low nibble first); code =
 *                       +-G2[idx][j], G2 = 256 x 8 uint8 grid (cb2_grid); w = D (2 s_b + 1) code.
 *   CB3  110 B / 256 w: [0:2] fp16 D, [2:66] low index bytes (4-weight groups), [66:74] high index
 *                       bits (group g: bit g%8 of byte g/8), [74:106] sign bits (weight i: bit i%8
 *                       of byte i/8), [106:110] sub-scales as CB2; code = +-G3[idx][j], G3 = 512 x 4
 *                       uint8 grid (cb3_grid); w = D (2 s_b + 1) code.
 *   Q5_1  24 B / 32 w : [0:2] fp16 d, [2:4] fp16 m, [4:8] high bits (bit i of the little-endian
 *                       word = bit 4 of code i), [8:24] b[16]; code of w_i = (b[i] & 15) | high
 *                       bit i, of w_(i+16) = (b[i] >> 4) | high bit i+16; w = d * code + m (an
 *                       offset format; down matrices only: fmt_gate_up rejects it).
 *   NL4X 136 B / 256 w: [0:2] fp16 D, [2:4] 16-bit word of the sub-scales' high bits (sub-block b:
 *                       bits 2b, 2b+1), [4:8] their low nibbles (sub-block b: byte 4 + b/2, low
 *                       nibble for even b), [8:136] eight 16-byte nibble groups in the NL4 order
 *                       (sub-block b = weights 32b..32b+31); l_b = low | high << 4 (0..63);
 *                       w = D (l_b - 32) T[nibble] with the NL4 table.
 *   q8_1  36 B / 32 values (activations): [0:2] fp16 d, [2:4] fp16 s, [4:36] int8 q[32], with
 *         amax = max|x|, d = amax / 127 (float32), q = clamp(round-half-away(x / d), +-127)
 *         (0 if amax == 0), d16 = fp16(d), s16 = fp16(f(d16) * sum q), all IEEE float32.
 * A matrix of R rows x C columns is R consecutive rows of C / block_weights blocks.
 * Planar layout (MOE_LAYOUT_PLANAR OR-ed into a moe_layer format field): the same bytes per row,
 * reordered so that the codes of the row's n blocks come first, block after block (Q8_0 32 B,
 * NL4 16 B, CB2 the 64 index and sign bytes, CB3 the 104 low-index, high-bit and sign bytes,
 * Q5_1 the 20 high-bit and nibble bytes, NL4X the 128 nibble bytes, each in its row-major
 * order), then the scales, block after block (Q8_0 / NL4 the fp16 d; Q5_1 d then m; NL4X its 8
 * header bytes; CB2 / CB3 the fp16 D followed by the 4 sub-scale bytes). A row keeps its size and a matrix its rows,
 * so every pointer and size of the row-major layout holds; moe_repack converts either way.
 * Shapes: C must be a multiple of 64 for Q8_0 / NL4 / Q5_1 and of 256 for CB2 / CB3 / NL4X; n_embd and n_ff
 * at most MOE_MAX_DIM.
 * Block contribution: c_b = scale_w * f(d_x) * sum_j code_j q_j (exact int32 sum), plus for Q5_1
 * m * f(s_x): the offset times the block's activation sum, read from the q8_1 sum field (the one
 * consumer of that field); a row's dot product is the sum of its c_b.
 */
#ifndef MOE_ROUTE_H
#define MOE_ROUTE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MAX_DIM 8192          /* max n_embd / n_ff */
#define MOE_MAX_CALL_ENTRIES 64   /* max cap_entries (T x k) of one call */
#define MOE_MAX_GROUPS 64         /* max cap_groups of one call */
#define MOE_MAX_PREFILL_ENTRIES 65535   /* max cap_entries of a prompt-path plan (moe_prefill_*) */
#define MOE_MAX_PREFILL_GROUPS 1024     /* max cap_groups of a prompt-path plan */

typedef enum {
  MOE_FMT_Q8_0 = 1, MOE_FMT_NL4 = 2, MOE_FMT_CB2 = 3, MOE_FMT_CB3 = 4,
  MOE_FMT_Q5_1 = 5,  /* down only */
  MOE_FMT_NL4X = 6
} moe_fmt;
#define MOE_LAYOUT_PLANAR 0x100   /* OR-ed into moe_layer.fmt_gate_up / fmt_down: planar rows */

typedef enum {
  MOE_OK = 0,
  MOE_E_ARG = -1,    /* null pointer or bad scalar argument */
  MOE_E_FMT = -2,    /* unknown weight format */
  MOE_E_SHAPE = -3,  /* dimension not supported (see "Shapes") */
  MOE_E_HIP = -4,    /* a HIP call failed; moe_last_error() has its text */
  MOE_E_WS = -5      /* workspace missing or too small */
} moe_status;

/* Device error bits OR-ed into *plan->err (sticky until the caller clears them). */
#define MOE_ERR_NGROUPS 1u   /* *n_groups < 0 or > cap_groups: the call did nothing */
#define MOE_ERR_ENTRIES 2u   /* grp_start not ascending or more than cap_entries entries */
#define MOE_ERR_EXPERT 4u    /* grp_expert out of [0, n_experts): that group skipped */
#define MOE_ERR_SRC 8u       /* ent_src out of [0, n_tokens): that entry skipped */
#define MOE_ERR_DST 16u      /* ent_dst out of [0, n_rows): that entry skipped */
#define MOE_ERR_ALIGN 32u    /* a weight pointer not 2-byte aligned: that group skipped */
#define MOE_ERR_WAIT 64u     /* moe_layer_step: a workgroup gave up waiting for the others (its
                                down tiles were not written); see moe_layer_step */

/* One MoE layer's experts. Host struct, read during the call only. */
typedef struct moe_layer {
  int32_t n_embd, n_ff, n_experts;
  int32_t fmt_gate_up;           /* format of gate and up (moe_fmt, | MOE_LAYOUT_PLANAR) */
  int32_t fmt_down;              /* format of down (moe_fmt, | MOE_LAYOUT_PLANAR) */
  const void* const* gate;       /* device array [n_experts] of device pointers: n_ff x n_embd */
  const void* const* up;         /* same */
  const void* const* down;       /* device array [n_experts]: n_embd x n_ff */
  const int8_t* nl4_table;       /* 16 B, needed if a format is NL4 or NL4X (else may be NULL) */
  const uint8_t* cb2_grid;       /* 256 x 8 B, needed if a format is CB2 */
  const uint8_t* cb3_grid;       /* 512 x 4 B, needed if a format is CB3 */
} moe_layer;

/* The entries of one call grouped by expert. Host struct holding device pointers. */
typedef struct moe_plan {
  int32_t cap_groups;            /* host: most groups a call may have (grid sizing), >= 1 */
  int32_t cap_entries;           /* host: most entries a call may have, >= 1 */
  int32_t* n_groups;             /* device scalar 0..cap_groups, read on the device */
  int32_t* grp_expert;           /* [cap_groups] expert of each group */
  int32_t* grp_start;            /* [cap_groups + 1] absolute first entry of each group */
  int32_t* ent_src;              /* token row of x / xq of each entry (absolute index) */
  int32_t* ent_dst;              /* output row of Y of each entry */
  float* ent_w;                  /* router weight of each entry */
  uint32_t* err;                 /* device sticky error bits (MOE_ERR_*) */
} moe_plan;

/* One-time weight repack ("#2058 ...", "Risks / limits": the weight-side loads of the blocks were
 * left as the next step; "#3455 [Engine] GP100 (sm_60): 4-bit slots ...", "Problem and result" and
 * "Approach": resident experts are transcoded once at load into a layout the decode kernels read,
 * with the arithmetic order unchanged so the outputs keep their bits, and the original blocks are
 * rebuilt from it and compared byte for byte). Here the layout is the planar one above, of the same
 * size. rows x cols weights of base format fmt (moe_fmt, without the layout flag) at src, row-major
 * when to_planar = 1 (written planar to dst), planar when to_planar = 0 (written row-major);
 * rows may span several matrices of one shape (a pool of experts). src and dst: device, 2-byte
 * aligned, not overlapping, rows x row_bytes each. A planar matrix, named with MOE_LAYOUT_PLANAR in
 * the layer, gives every entry point the same results, bit for bit, as its row-major source.
 * Errors: MOE_E_ARG (null or misaligned pointer, overlap, rows < 0, to_planar not 0 / 1),
 * MOE_E_FMT (unknown format or the layout flag set), MOE_E_SHAPE (cols as under "Shapes"). */
int moe_repack(void* stream, int fmt, const void* src, int64_t rows, int cols, void* dst, int to_planar);

/* ---- Prompt path (many tokens at once): the same layer computation, grouped GEMMs on the matrix
 * cores. "#2058 ...", "Summary", and "#3455 [Engine] GP100 (sm_60): 4-bit slots ...", "Approach":
 * the prompt path is a separate set of kernels (an activation-gathering matrix-multiply path) that
 * the decode changes leave alone. Sequence: moe_quantize_q8_1(x) -> moe_prefill_plan ->
 * moe_prefill_gate_up -> moe_prefill_swiglu_q8_1 -> moe_prefill_down -> moe_prefill_scatter.
 * Plans here may hold up to MOE_MAX_PREFILL_ENTRIES entries and MOE_MAX_PREFILL_GROUPS groups;
 * otherwise the moe_plan rules above hold (entries from grp_start[0], device n_groups, error bits).
 * Results match the oracle within the same tolerance as the decode path; the float summation
 * order differs from the decode kernels', so the two paths are not bit-identical to each other.
 * Row-major weights only (a planar layout flag gives MOE_E_FMT). */

/* The plan of T tokens' top-k choices ids [T][k] (weights w [T][k], may be NULL: weights 0):
 * groups ascending by expert, entries ascending by token from entry_base, as moe_build_plan, for
 * T x k up to MOE_MAX_PREFILL_ENTRIES (one workgroup). ent_of [T][k] (device, may be NULL)
 * receives each choice's entry index (-1 for an id outside [0, E), which is dropped with
 * MOE_ERR_EXPERT). Needs cap_entries >= T k, cap_groups >= min(E, T k), E <= 1024, and entry
 * arrays holding entry_base + T k entries. */
int moe_prefill_plan(void* stream, const int32_t* ids, const float* w, const int32_t* dst_of_token,
                     int T, int k, int E, int entry_base, const moe_plan* P, int32_t* ent_of);
/* g, u [entry][ld] float32 (rows by absolute entry index; n_ff columns written) of every entry
 * of the plan, from q8_1 rows xq [n_tokens][n_embd/32 x 36 B] indexed by ent_src. Per 32-row
 * tile of a matrix and group: weights decoded once per 512-weight chunk into LDS, one
 * v_mfma_i32_16x16x32_i8 per 32-weight block and 16 x 16 (row, entry) tile, the block's integer
 * sums scaled by d_w f(d_x) in float32 and added block after block. */
int moe_prefill_gate_up(void* stream, const moe_layer* L, const moe_plan* P, const void* xq, int n_tokens,
                        float* g, float* u, int ld);
/* SwiGLU + q8_1 of the plan's entries (as moe_swiglu_q8_1, for prompt-path plans). */
int moe_prefill_swiglu_q8_1(void* stream, const moe_plan* P, const float* g, const float* u, int n_ff, int ld,
                            float* h, void* hq);
/* O [entry][ldo] float32 = ent_w[entry] x (down_e . hq[entry]) for every entry of the plan (n_embd
 * columns), hq rows by absolute entry index ([entry][n_ff/32 x 36 B]). Same tiling as gate/up. */
int moe_prefill_down(void* stream, const moe_layer* L, const moe_plan* P, const void* hq, float* O, int ldo);
/* Y[dst(t)] += O[ent_of[t k + j]] for j = 0..k-1 in that order (dst(t) = dst_of_token[t], or t
 * when NULL), one thread per element. Destinations must be distinct rows (a prompt's tokens);
 * a destination outside [0, n_rows) skips its token (MOE_ERR_DST), an ent_of outside the plan's
 * entries skips that term (MOE_ERR_ENTRIES), -1 is a dropped choice. */
int moe_prefill_scatter(void* stream, const moe_plan* P, const int32_t* ent_of, const int32_t* dst_of_token,
                        int T, int k, const float* O, int ldo, int n_embd, float* Y, int n_rows, int ldy);

/* Router ("#363 ...": the window's tokens each pick top-k experts). For each of T tokens:
 * softmax over E float32 logits [T][E], the k largest by (logit descending, expert id
 * ascending), weights renormalised over those k. Outputs ids int32 [T][k] and w float32 [T][k],
 * in rank order. 1 <= k <= min(E, 32), E <= 1024. */
int moe_route_topk(void* stream, const float* logits, int T, int E, int k, int32_t* ids,
                   float* w);

/* Group the T*k entries by expert ("#2058 ...", "Why"): groups ascending by expert id, entries
 * in a group ascending by token; entry indices are absolute, starting at entry_base >= 0.
 * Writes *n_groups, grp_expert, grp_start[0..n_groups], ent_src (= token), ent_dst
 * (= dst_of_token[token], or the token if dst_of_token is NULL), ent_w (= w[token][rank]).
 * Requires T*k <= plan->cap_entries and T*k <= plan->cap_groups (host-checked). Ids out of
 * [0, E) set MOE_ERR_EXPERT and their entries are dropped. One workgroup; tiny. */
int moe_build_plan(void* stream, const int32_t* ids, const float* w, const int32_t* dst_of_token,
                   int T, int k, int E, int entry_base, const moe_plan* plan);

/* q8_1 quantization of `rows` rows of n float32 values (n % 32 == 0) into rows * n/32 blocks of
 * 36 B (layout above), bit-exact IEEE float32 ("#363 ...", "What changes": the quantizer). */
int moe_quantize_q8_1(void* stream, const float* x, int rows, int n, void* q);

/* Grouped gate/up ("#2058 ...", "Why" and "What changed": each expert's gate and up weights are
 * decoded once per group and dotted with the q8_1 rows of the group's 1-4 entries; "#363 ...",
 * "What changes": the call covers its own entries, n_groups read on the device).
 * For each entry a of the call (group g, expert e) and row r < n_ff,
 * g[a][r] = sum_b c_b(gate_e row r, xq row ent_src[a]) and the same for u with up_e.
 * xq: n_tokens rows of n_embd/32 q8_1 blocks. g, u: float32 rows of stride ld >= n_ff, indexed by
 * absolute entry; only the call's entries' rows are written. */
int moe_gate_up(void* stream, const moe_layer* L, const moe_plan* P, const void* xq, int n_tokens,
                float* g, float* u, int ld, int grid_limit);

/* Fused SwiGLU + q8_1 over the call's entries ("#363 ...", "What changes": one kernel over the
 * call's own entries, the SwiGLU product rounded on its own before the q8_1 block sums; "Measured":
 * the fused kernel against the two it replaces): e = expf(-g), h = (g / (1 + e)) * u, each
 * operation a float32 rounding in that order, then hq = q8_1(h). h may be NULL. hq rows: n_ff/32 blocks per absolute entry;
 * h rows: stride ld. Only the call's entries are read or written. */
int moe_swiglu_q8_1(void* stream, const moe_plan* P, const float* g, const float* u, int n_ff,
                    int ld, float* h, void* hq);

/* Grouped down + weighted scatter ("#2058 ...", "Why": the down projection grouped by expert like
 * gate/up, each token's expert outputs weighted by its router weights and added up; "#363 ...",
 * "Exactness": scattered destinations, rows no entry names keep their contents, results
 * independent of the grid): o_a[m] = sum_b c_b(down_e row m, hq row a) for m < n_embd, then
 * Y[ent_dst[a]][m] = Y + sum over the call's entries with that destination, in ascending entry
 * order, of ent_w[a] * o_a[m] (float32, each product and sum rounded). Y: n_rows rows of stride
 * ldy; rows no entry names are neither read nor written. hq: q8_1 rows by absolute entry. */
int moe_down_scatter(void* stream, const moe_layer* L, const moe_plan* P, const void* hq,
                     float* Y, int n_rows, int ldy, int grid_limit);

/* Host: bytes of workspace the single-call paths need for this layer and plan capacity ("#363
 * ...", "Exactness": stale scratch contents must not matter, which this workspace meets; the
 * call's descriptor for the down launch and the q8_1 rows of h). The workspace is 256-byte aligned and
 * needs no clearing: a call reads only bytes it wrote itself. */
size_t moe_workspace_bytes(const moe_layer* L, const moe_plan* P);

/* The whole step for the call's entries in two launches ("#363 ...", opening paragraph and
 * "What changes": fewer launches per call; "#2058 ...", "Why"): q8_1(x rows) -> grouped gate/up ->
 * SwiGLU + q8_1 -> grouped down -> weighted scatter into Y. x: n_tokens float32 rows of n_embd
 * (16-byte aligned). Bit-identical to the composed calls quantize -> gate_up -> swiglu ->
 * down_scatter. Calls that overlap on one workspace race; calls in one stream do not. */
int moe_layer_decode(void* stream, const moe_layer* L, const moe_plan* P, const float* x,
                     int n_tokens, float* Y, int n_rows, int ldy, void* workspace,
                     size_t ws_bytes, int grid_limit);

/* Same step starting from the router logits [T][n_experts] (float32): every gate/up workgroup
 * routes the T tokens (top-k, as moe_route_topk) and groups the entries (as moe_build_plan with
 * entry_base and dst_of_token) itself, and one workgroup writes that plan into P for the down
 * launch and for the caller. Bit-identical to route_topk -> build_plan -> moe_layer_decode.
 * Requires T*k <= cap_entries, T*k <= cap_groups, k <= 32, n_experts <= 1024. */
int moe_layer_decode_routed(void* stream, const moe_layer* L, const moe_plan* P,
                            const float* logits, int T, int k, const int32_t* dst_of_token,
                            int entry_base, const float* x, float* Y, int n_rows, int ldy,
                            void* workspace, size_t ws_bytes, int grid_limit);

/* EXPERIMENTAL, on no default path: slower than the two launches on MI355X (the cross-workgroup
 * wait costs more than the launch it saves) and dependent on every workgroup being resident.
 * The whole step from the router logits in ONE launch (same results, bit for bit, as
 * moe_layer_decode_routed): every workgroup routes and groups, runs its gate/up blocks with SwiGLU
 * and q8_1 ("#363 ...", "What changes"), then, once every workgroup of the launch has finished its
 * blocks, the grouped down projection and the weighted scatter ("#2058 ...", "Why"; "#363 ...",
 * "Exactness"). The workgroups meet through device-scope counts inside the workspace: they must
 * be zero before the first call on a workspace (a zero-filled allocation), and every call leaves
 * them zero. The launch uses at most one workgroup per CU and needs all of them resident at once (the
 * device not shared with other work that holds CUs); a workgroup that has not seen the others
 * within a bounded wait sets MOE_ERR_WAIT and leaves its rows of Y unwritten. Calls that overlap on
 * one workspace race. Limits as moe_layer_gate_up and moe_layer_down together. */
int moe_layer_step(void* stream, const moe_layer* L, const moe_plan* P, const float* logits, int T,
                   int k, const int32_t* dst_of_token, int entry_base, const float* x, float* Y,
                   int n_rows, int ldy, void* workspace, size_t ws_bytes, int grid_limit);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): moe_layer_decode_routed with the workspace taken from
 * a static device array of MOE_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends; nothing is allocated or freed. Same arguments, results and limits
 * as moe_layer_decode_routed (bit-identical), minus the workspace. A layer and plan whose
 * workspace (moe_workspace_bytes) exceeds MOE_NOALLOC_SCRATCH_BYTES gives MOE_E_WS before
 * anything is enqueued. Every call on one GPU uses that GPU's one array: calls that overlap on a
 * GPU (other streams, other threads) race; calls in one stream do not. The first call on a device
 * looks the array's address up (hipGetSymbolAddress) with that device current. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)512 << 10)
int moe_layer_decode_routed_noalloc(void* stream, const moe_layer* L, const moe_plan* P,
                                    const float* logits, int T, int k, const int32_t* dst_of_token,
                                    int entry_base, const float* x, float* Y, int n_rows, int ldy,
                                    int grid_limit);

/* The first of the two launches of moe_layer_decode (logits == NULL: the plan in P as built) or
 * of moe_layer_decode_routed (logits != NULL: route and group here, publish the plan into P;
 * then n_tokens must equal T). Leaves the call's descriptor and the q8_1 rows of h in the
 * workspace (moe_workspace_layout). For callers that put other work between the halves or time
 * them. Limits (else MOE_E_SHAPE): n_tokens * n_embd/32 * 36 B <= 48 KB of staged activations. */
int moe_layer_gate_up(void* stream, const moe_layer* L, const moe_plan* P, const float* logits,
                      int T, int k, const int32_t* dst_of_token, int entry_base, const float* x,
                      int n_tokens, void* workspace, size_t ws_bytes, int grid_limit);

/* The second launch: grouped down over the workspace's q8_1 rows of h + weighted scatter into Y
 * (limit, else MOE_E_SHAPE: cap_entries * n_ff/32 * 36 B <= 64 KB of staged h rows), as
 * moe_down_scatter. n_tokens is the first launch's (that launch marked entries whose token is
 * out of range, and this one skips them). */
int moe_layer_down(void* stream, const moe_layer* L, const moe_plan* P, const void* workspace,
                   size_t ws_bytes, int n_tokens, float* Y, int n_rows, int ldy, int grid_limit);

/* Host: where the last single-call step left the q8_1 rows of h inside the workspace, in split
 * form (row = entry - grp_start[0], n_ff/32 blocks per row, cap_entries rows): off[0] the 16-byte
 * low halves of the blocks' quants (quants 0-15), off[1] the high halves (16-31), off[2] the
 * blocks' scales as float32 (the fp16 d widened exactly). When the down format is Q5_1 the
 * blocks' sum fields (fp16 s widened) follow the scales, 256-byte aligned. */
int moe_workspace_layout(const moe_layer* L, const moe_plan* P, size_t off[3]);

/* The achievable-bandwidth reference the decode launches are measured against (not a step of the
 * method): one launch of `grid` workgroups of 256 threads reads the `bytes` at buf once with
 * 16-byte non-temporal loads, eight in flight per lane, the workgroups striding over the whole
 * buffer. out[b] (grid words, device) receives the XOR of the 32-bit words workgroup b read, so
 * the XOR of out[0..grid) is that of the whole buffer. buf and bytes must be multiples of 16 and
 * 1 <= grid <= 65535, else MOE_E_ARG. */
int moe_stream_read(void* stream, const void* buf, uint64_t bytes, uint32_t* out, int grid);

const char* moe_status_string(int status);   /* host, static string */
const char* moe_last_error(void);            /* host, text of the last MOE_E_HIP on this thread */

#ifdef __cplusplus
}
#endif
#endif
