// Grouped routed-expert MoE decode for MI355X (gfx950): kernels and the C-ABI entry points.
//
// The step ("#363 experts: smaller and fewer launches for the verify window's PCIe call", opening
// paragraph and "What changes"; "#2058 Verify window: the routed experts' gate/up with the group's
// q8_1 rows in shared memory", "Why"): token-expert entries grouped by expert; each expert's
// gate/up weights streamed once per group and dotted with the group's q8_1 activation rows;
// SwiGLU + q8_1 fused; the down projection grouped the same way; its rows scatter-added into the
// destination rows with the router weights.
//
// Design for gfx950 (not the pages' CUDA kernels):
//  * A work item is (group, row tile). Its weight rows are one contiguous byte span per matrix;
//    the span is streamed HBM -> LDS with direct-to-LDS 16-byte loads (global_load_lds_dwordx4,
//    fully coalesced whatever the block size: 18/34/70/110 B blocks do not align to 16 B), and
//    decoded out of LDS at any byte alignment with v_alignbyte.
//  * The group's (<= 4 at a time) q8_1 activation rows sit in LDS split into two 16-byte halves
//    and a float scale per block, so a lane's two ds_read_b128 per block are conflict-free and
//    the rows of a wave read the same words (broadcast).
//  * A row is split over L lanes (a power of two dividing the row's 32-weight units when
//    possible); lane l takes units l, l+L, ...; per unit v_dot4 (int8) per 4 weights, then
//    scale * d_x * isum in float32; the L partial sums are reduced by a fixed DPP tree. The lane
//    map depends only on the shape, so every kernel variant and every grid produces the same bits.
//  * moe_layer_decode is one persistent launch: workgroups take tickets from an atomic counter
//    (gate/up tiles of every group first, then down tiles), so a ticket only waits on lower
//    tickets held by running workgroups and the grid always drains. A gate/up tile covers one
//    32-row h block of gate and up, so SwiGLU + q8_1 of that block run in the same workgroup.
//    A down tile waits (bounded) for its group's h blocks; the last down tile of a row range
//    (atomic arrival counter) adds every entry's weighted rows into Y in ascending entry order:
//    deterministic, no float atomics.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/moe_route.h"
#include "moe_device.hpp"

namespace moe {

constexpr int kMaxRes = 128;        // rows per stage result buffer (per entry slot)
constexpr int kWbufBudget = 32768;  // LDS bytes for staged weight rows
constexpr int kSlack = 48;          // per staged span: 16-byte head misalignment + read slack

// ------------------------------------------------------------------ argument blocks ---------

struct LayerArgs {
  int n_embd, n_ff, n_experts;
  const void* const* gate;
  const void* const* up;
  const void* const* down;
  const int8_t* nl4;
  const uint8_t* cb2;
  const uint8_t* cb3;
};

struct PlanOut {
  int32_t* n_groups;
  int32_t* grp_expert;
  int32_t* grp_start;
  int32_t* ent_src;
  int32_t* ent_dst;
  float* ent_w;
  uint32_t* err;
};

struct PlanArgs {
  int cap_groups, cap_entries;
  const int32_t* n_groups;
  const int32_t* grp_expert;
  const int32_t* grp_start;
  const int32_t* ent_src;
  const int32_t* ent_dst;
  const float* ent_w;
  uint32_t* err;
};

// Row geometry of one matrix kind (gate/up rows have n_embd columns, down rows n_ff).
struct Geom {
  int U;          // 32-weight units per row
  int L;          // lanes per row
  int lgL;        // log2 L
  int upl;        // units per lane, ceil(U / L)
  int rb;         // bytes per row
  int S;          // rows per staged span
  int tile;       // rows per work item (gate/up: 32, down: RD)
  int ntiles;     // work items per group
};

struct Work {
  // workspace pieces (device)
  uint32_t* ctrl;     // [0] ticket, [1] exit count
  uint32_t* hq_cnt;   // [kMaxGroups] finished h blocks per group
  uint32_t* dt_cnt;   // [down tiles] groups finished per down row tile
  float* g;           // [cap_entries][n_ff]
  float* u;
  uint8_t* hq;        // [cap_entries][n_ff/32*36]
  float* o;           // [cap_entries][n_embd]
};

struct Call {
  int ng, e0, e1;
};

// ------------------------------------------------------------------ LDS layout ---------------

struct Smem {
  MOE_LDS uint8_t* wimg;     // staged weight rows
  MOE_LDS u32x4* qlo;        // [kMaxSlots][Umax]
  MOE_LDS u32x4* qhi;
  MOE_LDS float* xd;
  MOE_LDS float* res;        // [kMaxSlots][kMaxRes]
  MOE_LDS float* gu;         // [kMaxSlots][64]: g rows 0..31, u rows 32..63 of a gate/up item
  MOE_LDS uint32_t* grid2;   // 512 dwords
  MOE_LDS uint32_t* grid3;   // 512 dwords
  MOE_LDS int* meta_i;       // [64] dst (or -1 = skip), [64] owner flag
  MOE_LDS float* meta_w;     // [64]
  MOE_LDS int* misc;         // [16] call info / broadcast
  int umax;
};

extern __shared__ __align__(16) uint8_t g_smem[];

__host__ __device__ inline int smem_bytes(int wbuf, int umax) {
  return wbuf + 64 + kMaxSlots * umax * 36 + kMaxSlots * kMaxRes * 4 + kMaxSlots * 64 * 4 + 4096 +
         64 * 12 + 64;
}

__device__ inline Smem smem_layout(int wbuf, int umax) {
  Smem s;
  MOE_LDS uint8_t* p = (MOE_LDS uint8_t*)g_smem;
  s.wimg = p;
  p += wbuf + 64;
  s.qlo = (MOE_LDS u32x4*)p;
  p += kMaxSlots * umax * 16;
  s.qhi = (MOE_LDS u32x4*)p;
  p += kMaxSlots * umax * 16;
  s.xd = (MOE_LDS float*)p;
  p += kMaxSlots * umax * 4;
  s.res = (MOE_LDS float*)p;
  p += kMaxSlots * kMaxRes * 4;
  s.gu = (MOE_LDS float*)p;
  p += kMaxSlots * 64 * 4;
  s.grid2 = (MOE_LDS uint32_t*)p;
  p += 2048;
  s.grid3 = (MOE_LDS uint32_t*)p;
  p += 2048;
  s.meta_i = (MOE_LDS int*)p;
  p += 64 * 8;
  s.meta_w = (MOE_LDS float*)p;
  p += 64 * 4;
  s.misc = (MOE_LDS int*)p;
  s.umax = umax;
  return s;
}

// Values broadcast through LDS are the same in every lane; reading them with readfirstlane puts
// them in scalar registers, so every branch and loop bound built from them is a scalar (whole-
// wave) branch. That keeps each barrier in control flow the compiler sees as uniform.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const uint8_t* uni_ptr(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void set_err(uint32_t* err, uint32_t bit) {
  if (err) atomicOr(err, bit);
}

// Validate the call's group table (thread 0) and broadcast it. Bad tables make the call empty.
__device__ Call read_call(const PlanArgs& P, const Smem& sm) {
  if (threadIdx.x == 0) {
    int ng = *P.n_groups;
    int e0 = 0, e1 = 0;
    if (ng < 0 || ng > P.cap_groups) {
      set_err(P.err, MOE_ERR_NGROUPS);
      ng = 0;
    }
    if (ng > 0) {
      e0 = P.grp_start[0];
      bool ok = e0 >= 0;
      int prev = e0;
      for (int g = 1; g <= ng; ++g) {
        int s = P.grp_start[g];
        ok = ok && s >= prev;
        prev = s;
      }
      e1 = prev;
      if (!ok || e1 - e0 > P.cap_entries) {
        set_err(P.err, MOE_ERR_ENTRIES);
        ng = 0;
        e0 = e1 = 0;
      }
    }
    sm.misc[0] = ng;
    sm.misc[1] = e0;
    sm.misc[2] = e1;
  }
  __syncthreads();
  Call c{uni(sm.misc[0]), uni(sm.misc[1]), uni(sm.misc[2])};
  return c;
}

__device__ void load_tables(const LayerArgs& A, bool need2, bool need3, const Smem& sm,
                            Tables& tb) {
  if (A.nl4) {
    const uint32_t* t = (const uint32_t*)A.nl4;
    tb.nl4[0] = t[0];
    tb.nl4[1] = t[1];
    tb.nl4[2] = t[2];
    tb.nl4[3] = t[3];
  } else {
    tb.nl4[0] = tb.nl4[1] = tb.nl4[2] = tb.nl4[3] = 0;
  }
  if (need2)
    for (int i = threadIdx.x; i < 512; i += kThreads) sm.grid2[i] = ((const uint32_t*)A.cb2)[i];
  if (need3)
    for (int i = threadIdx.x; i < 512; i += kThreads) sm.grid3[i] = ((const uint32_t*)A.cb3)[i];
  tb.cb2 = sm.grid2;
  tb.cb3 = sm.grid3;
}

// ------------------------------------------------------------------ staging -----------------

// Start streaming bytes [src, src + n) into LDS at dst (16-byte aligned): whole aligned 16-byte
// chunks, one 1 KB wave instruction per 64 chunks. Reading the enclosing aligned chunks never
// leaves the pages that hold the span. Returns the LDS offset of src's first byte inside dst.
__device__ __forceinline__ uint32_t stage_span(const uint8_t* src, uint32_t n, MOE_LDS uint8_t* dst) {
  const uintptr_t a = (uintptr_t)src & ~(uintptr_t)15;
  const uint32_t mis = (uint32_t)((uintptr_t)src & 15);
  const uint32_t nch = (mis + n + 15) >> 4;
  const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (uint32_t c0 = wave * 64; c0 < nch; c0 += 256) {
    const uint32_t c = c0 + lane;
    if (c < nch)
      __builtin_amdgcn_global_load_lds((const void*)(a + 16ull * c), (MOE_LDS void*)(dst + 16 * c0),
                                       16, 0, 0);
  }
  return mis;
}

__device__ __forceinline__ void wait_staged() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Activation slots from q8_1 rows in global memory (row pointers per slot; NULL = zeros).
__device__ void stage_q81_rows(const uint8_t* const rows[kMaxSlots], int ne, int U, const Smem& sm) {
  for (int idx = threadIdx.x; idx < ne * U; idx += kThreads) {
    const int e = idx / U, u = idx - e * U;
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = lo;
    float d = 0.0f;
    if (rows[e]) {
      const uint32_t* p = (const uint32_t*)(rows[e] + 36 * u);
      d = h2f(p[0] & 0xFFFFu);
      lo = u32x4{p[1], p[2], p[3], p[4]};
      hi = u32x4{p[5], p[6], p[7], p[8]};
    }
    sm.qlo[e * sm.umax + u] = lo;
    sm.qhi[e * sm.umax + u] = hi;
    sm.xd[e * sm.umax + u] = d;
  }
}

// Activation slots quantized here from float32 rows (same quantizer as moe_quantize_q8_1).
__device__ void stage_f32_rows(const float* const rows[kMaxSlots], int ne, int U, const Smem& sm) {
  for (int idx = threadIdx.x; idx < ne * U; idx += kThreads) {
    const int e = idx / U, u = idx - e * U;
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = lo;
    float d = 0.0f;
    if (rows[e]) {
      const float4* p = (const float4*)(rows[e] + 32 * u);
      float v[32];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 f = p[i];
        v[4 * i] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
      }
      const QBlock b = quant_block(v);
      lo = u32x4{b.q[0], b.q[1], b.q[2], b.q[3]};
      hi = u32x4{b.q[4], b.q[5], b.q[6], b.q[7]};
      d = b.d;
    }
    sm.qlo[e * sm.umax + u] = lo;
    sm.qhi[e * sm.umax + u] = hi;
    sm.xd[e * sm.umax + u] = d;
  }
}

// ------------------------------------------------------------------ row dots ----------------

// Dot every staged row (rows [0, S) at LDS offset off0, rows [S, nrows) at off1) with the ne
// activation slots; res[e * kMaxRes + row] = sum over the row's units of c_b, reduced over L lanes
// in a fixed order.
template <int FMT>
__device__ void dot_rows(const Smem& sm, const Tables& tb, const Geom& G, uint32_t off0,
                         uint32_t off1, int S, int nrows, int ne) {
  const MOE_LDS uint32_t* W = (const MOE_LDS uint32_t*)sm.wimg;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int WR = 64 >> G.lgL;
  const int rr = lane >> G.lgL, li = lane & (G.L - 1);
  for (int base = wave * WR; base < nrows; base += 4 * WR) {
    const int i = base + rr;
    float acc[kMaxSlots] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (i < nrows) {
      const uint32_t row = i < S ? off0 + (uint32_t)(i * G.rb) : off1 + (uint32_t)((i - S) * G.rb);
      for (int k = 0; k < G.upl; ++k) {
        const int u = li + (k << G.lgL);
        if (u < G.U) {
          uint32_t c[8];
          float sc;
          decode_unit<FMT>(W, row, u, tb, c, sc);
#pragma unroll
          for (int e = 0; e < kMaxSlots; ++e) {
            if (e < ne) {
              const u32x4 lo = sm.qlo[e * sm.umax + u];
              const u32x4 hi = sm.qhi[e * sm.umax + u];
              int s = __builtin_amdgcn_sdot4((int)c[0], (int)lo.x, 0, false);
              s = __builtin_amdgcn_sdot4((int)c[1], (int)lo.y, s, false);
              s = __builtin_amdgcn_sdot4((int)c[2], (int)lo.z, s, false);
              s = __builtin_amdgcn_sdot4((int)c[3], (int)lo.w, s, false);
              s = __builtin_amdgcn_sdot4((int)c[4], (int)hi.x, s, false);
              s = __builtin_amdgcn_sdot4((int)c[5], (int)hi.y, s, false);
              s = __builtin_amdgcn_sdot4((int)c[6], (int)hi.z, s, false);
              s = __builtin_amdgcn_sdot4((int)c[7], (int)hi.w, s, false);
              acc[e] = acc[e] + (sc * sm.xd[e * sm.umax + u]) * (float)s;
            }
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < kMaxSlots; ++e)
      if (e < ne) acc[e] = group_sum(acc[e], G.L);
    // every lane of the row holds every sum; lane li stores the entries e = li (mod L)
    if (i < nrows) {
#pragma unroll
      for (int e = 0; e < kMaxSlots; ++e)
        if (e < ne && (e & (G.L - 1)) == li) sm.res[e * kMaxRes + i] = acc[e];
    }
  }
}

// ------------------------------------------------------------------ per-group info ----------

struct GroupInfo {
  int ok;                 // expert valid and pointers aligned
  int a0, a1;             // absolute entry range
  const uint8_t* w0;      // gate (gate/up items) or down
  const uint8_t* w1;      // up
};

__device__ GroupInfo group_info(const LayerArgs& A, const PlanArgs& P, int g, bool down,
                                const Smem& sm) {
  if (threadIdx.x == 0) {
    const int e = P.grp_expert[g];
    int ok = 1;
    const uint8_t* w0 = nullptr;
    const uint8_t* w1 = nullptr;
    if (e < 0 || e >= A.n_experts) {
      set_err(P.err, MOE_ERR_EXPERT);
      ok = 0;
    } else if (down) {
      w0 = (const uint8_t*)A.down[e];
    } else {
      w0 = (const uint8_t*)A.gate[e];
      w1 = (const uint8_t*)A.up[e];
    }
    if (ok && ((((uintptr_t)w0) | ((uintptr_t)w1)) & 1)) {
      set_err(P.err, MOE_ERR_ALIGN);
      ok = 0;
    }
    sm.misc[4] = ok;
    sm.misc[5] = P.grp_start[g];
    sm.misc[6] = P.grp_start[g + 1];
    *(MOE_LDS uint64_t*)(sm.misc + 8) = (uint64_t)(uintptr_t)w0;
    *(MOE_LDS uint64_t*)(sm.misc + 10) = (uint64_t)(uintptr_t)w1;
  }
  __syncthreads();
  GroupInfo gi;
  gi.ok = uni(sm.misc[4]);
  gi.a0 = uni(sm.misc[5]);
  gi.a1 = uni(sm.misc[6]);
  gi.w0 = uni_ptr(*(const MOE_LDS uint64_t*)(sm.misc + 8));
  gi.w1 = uni_ptr(*(const MOE_LDS uint64_t*)(sm.misc + 10));
  __syncthreads();
  return gi;
}

// ------------------------------------------------------------------ SwiGLU + q8_1 -----------

// 32 lanes (an aligned half-wave) turn 32 (g, u) pairs into one q8_1 block of h. Same arithmetic
// as quant_block: amax and the integer sum are order-free, so the bytes match it exactly.
__device__ __forceinline__ void swiglu_q81_lanes(float gv, float uv, int l32, bool live,
                                                 uint8_t* blk, float* hrow) {
  const float h = live ? swiglu(gv, uv) : 0.0f;
  if (live && hrow) hrow[l32] = h;
  const float amax = wave_max32(__builtin_fabsf(h));
  const float d = amax / 127.0f;
  int q = 0;
  if (amax != 0.0f) {
    float r = round_half_away(h / d);
    r = r > 127.0f ? 127.0f : r;
    r = r < -127.0f ? -127.0f : r;
    q = (int)r;
  }
  const int isum = wave_sum32(q);
  if (live) {
    blk[4 + l32] = (uint8_t)(q & 0xFF);
    if (l32 == 0) {
      const uint32_t d16 = f2h(d);
      const uint32_t s16 = sum_field(d16, isum);
      *(uint32_t*)blk = d16 | (s16 << 16);
    }
  }
}

// ------------------------------------------------------------------ gate/up item ------------

// One gate/up item: rows [32 j, 32 j + 32) of gate and up for every entry of group g.
// Composed mode (XF32 == false): activations from q8_1 rows xq, outputs g/u rows (absolute
// entry index, stride ld). Fused mode: activations quantized from x, g/u written to the
// workspace (rows relative to e0) and the h block's q8_1 written to the workspace hq.
template <int FMT, bool FUSED>
__device__ void gate_up_item(const LayerArgs& A, const PlanArgs& P, const Geom& G, const Smem& sm,
                             const Tables& tb, const Call& call, int g, int j, const void* xin,
                             int n_tokens, float* gout, float* uout, int ld, const Work& wk) {
  const GroupInfo gi = group_info(A, P, g, false, sm);
  if (!gi.ok) return;
  const int r_begin = 32 * j;
  for (int c0 = gi.a0; c0 < gi.a1; c0 += kMaxSlots) {
    const int ne = min(kMaxSlots, gi.a1 - c0);
    // entry sources (invalid -> zero activations, nothing written)
    if (threadIdx.x < kMaxSlots) {
      int src = -1;
      if ((int)threadIdx.x < ne) {
        src = P.ent_src[c0 + threadIdx.x];
        if (src < 0 || src >= n_tokens) {
          set_err(P.err, MOE_ERR_SRC);
          src = -1;
        }
      }
      sm.misc[12 + threadIdx.x] = src;
    }
    __syncthreads();
    int srcs[kMaxSlots];
#pragma unroll
    for (int e = 0; e < kMaxSlots; ++e) srcs[e] = uni(sm.misc[12 + e]);
    for (int r0 = r_begin; r0 < r_begin + 32; r0 += G.S) {
      const int S = min(G.S, r_begin + 32 - r0);
      const uint32_t span = (uint32_t)(S * G.rb);
      const uint32_t regB = (span + kSlack + 15) & ~15u;
      const uint32_t off0 = stage_span(gi.w0 + (size_t)r0 * G.rb, span, sm.wimg);
      const uint32_t off1 = regB + stage_span(gi.w1 + (size_t)r0 * G.rb, span, sm.wimg + regB);
      if (r0 == r_begin) {
        if constexpr (FUSED) {
          const float* rows[kMaxSlots];
#pragma unroll
          for (int e = 0; e < kMaxSlots; ++e)
            rows[e] = srcs[e] >= 0 ? (const float*)xin + (size_t)srcs[e] * A.n_embd : nullptr;
          stage_f32_rows(rows, ne, G.U, sm);
        } else {
          const uint8_t* rows[kMaxSlots];
#pragma unroll
          for (int e = 0; e < kMaxSlots; ++e)
            rows[e] = srcs[e] >= 0 ? (const uint8_t*)xin + (size_t)srcs[e] * G.U * 36 : nullptr;
          stage_q81_rows(rows, ne, G.U, sm);
        }
      }
      wait_staged();
      dot_rows<FMT>(sm, tb, G, off0, off1, S, 2 * S, ne);
      __syncthreads();
      // results: rows [0, S) are gate rows r0.., rows [S, 2S) up rows r0..
      for (int idx = threadIdx.x; idx < ne * 2 * S; idx += kThreads) {
        const int e = idx / (2 * S), i = idx - e * 2 * S;
        if (srcs[e] < 0) continue;
        const float v = sm.res[e * kMaxRes + i];
        const int r = r0 + (i < S ? i : i - S);
        if constexpr (FUSED) {
          float* dstp = i < S ? wk.g : wk.u;
          dstp[(size_t)(c0 + e - call.e0) * A.n_ff + r] = v;
          sm.gu[e * 64 + (i < S ? 0 : 32) + r - r_begin] = v;
        } else {
          float* dstp = i < S ? gout : uout;
          dstp[(size_t)(c0 + e) * ld + r] = v;
        }
      }
      __syncthreads();
    }
    if constexpr (FUSED) {
      // SwiGLU + q8_1 of h rows [32 j, 32 j + 32) per entry, from the g/u values kept in LDS
      const int t = threadIdx.x;
      const int e = t >> 5, l32 = t & 31;
      if (e < kMaxSlots) {  // 128 threads: 4 slots x 32 rows
        const bool live = e < ne && srcs[e] >= 0;
        const size_t rrow = (size_t)(c0 + e - call.e0);
        float gv = 0.0f, uv = 0.0f;
        if (live) {
          gv = sm.gu[e * 64 + l32];
          uv = sm.gu[e * 64 + 32 + l32];
        }
        uint8_t* blk = wk.hq + rrow * (size_t)(A.n_ff / 32) * 36 + (size_t)j * 36;
        swiglu_q81_lanes(gv, uv, l32, live, blk, nullptr);
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ down item ---------------

// Entry metadata of the call for the scatter: dst row (-1 = skip) and router weight per entry,
// owner flag = first entry of the call naming its dst. Computed by every workgroup that scatters.
__device__ void entry_meta(const LayerArgs& A, const PlanArgs& P, const Call& call, int n_rows,
                           int n_tokens, const Smem& sm) {
  const int n = call.e1 - call.e0;
  const int i = threadIdx.x;
  if (i < n) {
    const int a = call.e0 + i;
    int g = 0;
    while (g + 1 < call.ng && P.grp_start[g + 1] <= a) ++g;
    const int e = P.grp_expert[g];
    int dst = P.ent_dst[a];
    if (dst < 0 || dst >= n_rows) {
      set_err(P.err, MOE_ERR_DST);
      dst = -1;
    }
    if (e < 0 || e >= A.n_experts) dst = -1;
    if (n_tokens >= 0) {
      const int src = P.ent_src[a];
      if (src < 0 || src >= n_tokens) dst = -1;
    }
    sm.meta_i[i] = dst;
    sm.meta_w[i] = P.ent_w[a];
  }
  __syncthreads();
  if (i < n) {
    const int d = sm.meta_i[i];
    int owner = d >= 0;
    for (int k = 0; k < i && owner; ++k) owner = sm.meta_i[k] != d;
    sm.meta_i[64 + i] = owner;
  }
  __syncthreads();
}

// Y[dst][r] (r in [r0, r0 + nr)) += sum over the call's entries naming dst, ascending, of w * o.
__device__ void scatter_rows(const Call& call, int r0, int nr, const float* o, int n_embd, float* Y,
                             int ldy, const Smem& sm) {
  const int n = call.e1 - call.e0;
  for (int idx = threadIdx.x; idx < n * nr; idx += kThreads) {
    const int i = idx / nr, m = idx - i * nr;
    if (!sm.meta_i[64 + i]) continue;
    const int d = sm.meta_i[i];
    float* y = Y + (size_t)d * ldy + r0 + m;
    float acc = *y;
    for (int k = i; k < n; ++k)
      if (sm.meta_i[k] == d) acc = acc + sm.meta_w[k] * o[(size_t)k * n_embd + r0 + m];
    *y = acc;
  }
}

// One down item: rows [RD t, RD t + RD) of group g's down matrix for all its entries; the rows of o
// (relative entry index) go to the workspace; then the arrival count of row tile t.
template <int FMT>
__device__ void down_item(const LayerArgs& A, const PlanArgs& P, const Geom& G, const Smem& sm,
                          const Tables& tb, const Call& call, int g, int t, const uint8_t* hq,
                          bool hq_abs, const Work& wk, float* Y, int ldy) {
  const GroupInfo gi = group_info(A, P, g, true, sm);
  const int r0 = G.tile * t;
  const int nr = min(G.tile, A.n_embd - r0);
  const int hstride = (A.n_ff / 32) * 36;
  if (gi.ok) {
    for (int c0 = gi.a0; c0 < gi.a1; c0 += kMaxSlots) {
      const int ne = min(kMaxSlots, gi.a1 - c0);
      const uint32_t off0 = stage_span(gi.w0 + (size_t)r0 * G.rb, (uint32_t)(nr * G.rb), sm.wimg);
      const uint8_t* rows[kMaxSlots];
#pragma unroll
      for (int e = 0; e < kMaxSlots; ++e) {
        const int a = c0 + e;
        rows[e] = e < ne ? hq + (size_t)(hq_abs ? a : a - call.e0) * hstride : nullptr;
      }
      stage_q81_rows(rows, ne, G.U, sm);
      wait_staged();
      dot_rows<FMT>(sm, tb, G, off0, off0, nr, nr, ne);
      __syncthreads();
      for (int idx = threadIdx.x; idx < ne * nr; idx += kThreads) {
        const int e = idx / nr, m = idx - e * nr;
        wk.o[(size_t)(c0 + e - call.e0) * A.n_embd + r0 + m] = sm.res[e * kMaxRes + m];
      }
      __syncthreads();
    }
  }
  // arrival: the last group to finish row tile t scatters it
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = atomicAdd(&wk.dt_cnt[t], 1u);
    const int last = old == (uint32_t)(call.ng - 1);
    if (last) atomicExch(&wk.dt_cnt[t], 0u);
    sm.misc[3] = last;
  }
  __syncthreads();
  if (uni(sm.misc[3])) {
    __threadfence();
    scatter_rows(call, r0, nr, wk.o, A.n_embd, Y, ldy, sm);
  }
  __syncthreads();
}

// ------------------------------------------------------------------ kernels -----------------

__global__ __launch_bounds__(kThreads) void k_quantize(const float* __restrict__ x, int rows, int n,
                                                       uint8_t* __restrict__ q) {
  const int nb = n / 32;
  const long total = (long)rows * nb;
  for (long b = (long)blockIdx.x * kThreads + threadIdx.x; b < total; b += (long)gridDim.x * kThreads) {
    const long r = b / nb, k = b - r * nb;
    const float4* p = (const float4*)(x + r * n + 32 * k);
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 f = p[i];
      v[4 * i] = f.x;
      v[4 * i + 1] = f.y;
      v[4 * i + 2] = f.z;
      v[4 * i + 3] = f.w;
    }
    const QBlock qb = quant_block(v);
    uint32_t* o = (uint32_t*)(q + 36 * b);
    o[0] = qb.d16 | (qb.s16 << 16);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[1 + i] = qb.q[i];
  }
}

// One wave per token: top-k by (logit desc, id asc), weights = exp(l - l_max) / sum over the k.
__global__ __launch_bounds__(kThreads) void k_route(const float* __restrict__ logits, int T, int E,
                                                    int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* l = logits + (size_t)t * E;
  constexpr int kPer = 16;  // E <= 1024
  float v[kPer];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? l[e] : 0.0f;
  }
  float top = 0.0f, sum = 0.0f, mine = 0.0f;
  int myid = 0;
  for (int r = 0; r < k; ++r) {
    float bv = 0.0f;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !((taken >> i) & 1u) && (bi == 0x7FFFFFFF || v[i] > bv)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float ov = __shfl_xor(bv, m);
      const int oi = __shfl_xor(bi, m);
      const bool take = oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || ov > bv || (ov == bv && oi < bi));
      if (take) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (r == 0) top = bv;
    const float ex = expf(bv - top);
    sum = sum + ex;
    if (lane == r) {
      mine = ex;
      myid = bi;
    }
  }
  if (lane < k) {
    ids[(size_t)t * k + lane] = myid;
    w[(size_t)t * k + lane] = mine / sum;
  }
}

// Counting sort of n = T*k entries by expert, one workgroup of 64 threads (n <= 64).
__global__ __launch_bounds__(64) void k_plan(const int32_t* __restrict__ ids, const float* __restrict__ w,
                                             const int32_t* __restrict__ dst_of_token, int T, int k,
                                             int E, int entry_base, PlanOut P) {
  __shared__ int s_e[64];
  __shared__ int s_first[64];
  const int n = T * k;
  const int i = threadIdx.x;
  int e = -1;
  if (i < n) {
    e = ids[i];
    if (e < 0 || e >= E) {
      set_err(P.err, MOE_ERR_EXPERT);
      e = -1;
    }
  }
  s_e[i] = e;
  __syncthreads();
  int first = e >= 0;
  for (int q = 0; q < i && first; ++q) first = s_e[q] != e;
  s_first[i] = first;
  __syncthreads();
  int grp = 0, before = 0, pos = 0, nvalid = 0, ngroups = 0;
  for (int m = 0; m < n; ++m) {
    const int em = s_e[m];
    if (em < 0) continue;
    ++nvalid;
    ngroups += s_first[m];
    if (e < 0) continue;
    if (m < i && em == e) ++pos;
    if (em < e) {
      ++before;
      grp += s_first[m];
    }
  }
  if (e >= 0) {
    const int t = i / k;
    const int slot = entry_base + before + pos;
    P.ent_src[slot] = t;
    P.ent_dst[slot] = dst_of_token ? dst_of_token[t] : t;
    P.ent_w[slot] = w[i];
    if (first) {
      P.grp_expert[grp] = e;
      P.grp_start[grp] = entry_base + before;
    }
  }
  if (i == 0) {
    P.grp_start[ngroups] = entry_base + nvalid;
    *P.n_groups = ngroups;
  }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_gate_up(LayerArgs A, PlanArgs P, Geom G, int wbuf,
                                                      int umax, const uint8_t* xq, int n_tokens,
                                                      float* gout, float* uout, int ld) {
  const Smem sm = smem_layout(wbuf, umax);
  Tables tb;
  load_tables(A, FMT == CB2, FMT == CB3, sm, tb);
  const Call call = read_call(P, sm);
  const int items = call.ng * G.ntiles;
  Work wk{};
  for (int it = blockIdx.x; it < items; it += gridDim.x)
    gate_up_item<FMT, false>(A, P, G, sm, tb, call, it / G.ntiles, it % G.ntiles, xq, n_tokens,
                             gout, uout, ld, wk);
}

// Over (entry, h block) of the call: two blocks per wave.
__global__ __launch_bounds__(kThreads) void k_swiglu(PlanArgs P, const float* __restrict__ g,
                                                     const float* __restrict__ u, int n_ff, int ld,
                                                     float* h, uint8_t* hq) {
  __shared__ int s_call[3];
  if (threadIdx.x == 0) {
    int ng = *P.n_groups, e0 = 0, e1 = 0;
    if (ng < 0 || ng > P.cap_groups) {
      set_err(P.err, MOE_ERR_NGROUPS);
      ng = 0;
    }
    if (ng > 0) {
      e0 = P.grp_start[0];
      e1 = P.grp_start[ng];
      if (e0 < 0 || e1 < e0 || e1 - e0 > P.cap_entries) {
        set_err(P.err, MOE_ERR_ENTRIES);
        e0 = e1 = 0;
      }
    }
    s_call[0] = e0;
    s_call[1] = e1;
  }
  __syncthreads();
  const int e0 = s_call[0], e1 = s_call[1];
  const int nb = n_ff / 32;
  const int total = (e1 - e0) * nb;
  const int half = threadIdx.x >> 5, l32 = threadIdx.x & 31;
  // every wave runs the loop the same number of times (shuffles need both halves present)
  for (int base = blockIdx.x * 8; base < total; base += gridDim.x * 8) {
    const int it = base + half;
    const bool live = it < total;
    const int a = live ? e0 + it / nb : e0;
    const int b = live ? it % nb : 0;
    const float gv = live ? g[(size_t)a * ld + 32 * b + l32] : 0.0f;
    const float uv = live ? u[(size_t)a * ld + 32 * b + l32] : 0.0f;
    swiglu_q81_lanes(gv, uv, l32, live, hq + (size_t)a * nb * 36 + (size_t)b * 36,
                     h ? h + (size_t)a * ld + 32 * b : nullptr);
  }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_down(LayerArgs A, PlanArgs P, Geom G, int wbuf, int umax,
                                                   const uint8_t* hq, Work wk, float* Y, int n_rows,
                                                   int ldy) {
  const Smem sm = smem_layout(wbuf, umax);
  Tables tb;
  load_tables(A, FMT == CB2, FMT == CB3, sm, tb);
  const Call call = read_call(P, sm);
  if (call.ng == 0) return;
  entry_meta(A, P, call, n_rows, -1, sm);
  const int items = call.ng * G.ntiles;
  for (int it = blockIdx.x; it < items; it += gridDim.x)
    down_item<FMT>(A, P, G, sm, tb, call, it / G.ntiles, it % G.ntiles, hq, true, wk, Y, ldy);
}

// Bounded wait (thread 0) for *ctr >= need: relaxed polling, then one acquire fence. The wait
// ends after about 50 ms of wall-clock time (100 MHz counter) or 2^20 polls, whichever is first;
// running out sets MOE_ERR_WAIT and lets the workgroup go on, so the grid always drains.
__device__ bool wait_geq(uint32_t* ctr, uint32_t need, uint32_t* err) {
  const uint64_t t0 = wall_clock64();
  for (uint32_t it = 0;; ++it) {
    const uint32_t v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v >= need) {
      __atomic_thread_fence(__ATOMIC_ACQUIRE);
      return true;
    }
    if (it > (1u << 20) || wall_clock64() - t0 > 5000000ull) {
      set_err(err, MOE_ERR_WAIT);
      __atomic_thread_fence(__ATOMIC_ACQUIRE);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

template <int FG, int FD>
__global__ __launch_bounds__(kThreads) void k_layer(LayerArgs A, PlanArgs P, Geom GU, Geom GD,
                                                    int wbuf, int umax, const float* x, int n_tokens,
                                                    Work wk, float* Y, int n_rows, int ldy) {
  const Smem sm = smem_layout(wbuf, umax);
  Tables tb;
  load_tables(A, FG == CB2 || FD == CB2, FG == CB3 || FD == CB3, sm, tb);
  const Call call = read_call(P, sm);
  if (call.ng > 0) entry_meta(A, P, call, n_rows, n_tokens, sm);
  const int n_gu = call.ng * GU.ntiles;
  const int total = n_gu + call.ng * GD.ntiles;
  // Every thread-0-only block below is closed by a barrier before the next one starts: with two
  // such blocks back to back around the loop latch the compiler may merge them into a path that
  // only lane 0 takes, leaving the other lanes looping on a stale ticket.
  for (;;) {
    if (threadIdx.x == 0) sm.misc[7] = (int)atomicAdd(&wk.ctrl[0], 1u);
    __syncthreads();
    const int tk = uni(sm.misc[7]);
    __syncthreads();
    if (tk >= total) break;
    if (tk < n_gu) {
      const int g = tk / GU.ntiles;
      gate_up_item<FG, true>(A, P, GU, sm, tb, call, g, tk % GU.ntiles, x, n_tokens, nullptr,
                             nullptr, 0, wk);
      __threadfence();
      __syncthreads();
      if (threadIdx.x == 0) atomicAdd(&wk.hq_cnt[g], 1u);
      __syncthreads();
    } else {
      const int d = tk - n_gu;
      const int g = d / GD.ntiles;
      if (threadIdx.x == 0) wait_geq(&wk.hq_cnt[g], (uint32_t)GU.ntiles, P.err);
      __syncthreads();
      down_item<FD>(A, P, GD, sm, tb, call, g, d % GD.ntiles, wk.hq, false, wk, Y, ldy);
    }
    __syncthreads();
  }
  // the last workgroup out clears the counters for the next call
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = atomicAdd(&wk.ctrl[1], 1u);
    if (old == gridDim.x - 1) {
      __threadfence();
      for (int g = 0; g < MOE_MAX_GROUPS; ++g) wk.hq_cnt[g] = 0;
      wk.ctrl[0] = 0;
      wk.ctrl[1] = 0;
      __threadfence();
    }
  }
}

__global__ void k_fill_zero(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// ------------------------------------------------------------------ host side ---------------

thread_local std::string t_last_error;

int hip_fail(hipError_t e, const char* what) {
  t_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return MOE_E_HIP;
}

bool fmt_ok(int f) { return f >= Q8_0 && f <= CB3; }

bool cols_ok(int fmt, int n) {
  if (n <= 0 || n > MOE_MAX_DIM) return false;
  return (fmt == CB2 || fmt == CB3) ? n % 256 == 0 : n % 64 == 0;
}

int ilog2(int v) {
  int l = 0;
  while ((1 << (l + 1)) <= v) ++l;
  return l;
}

// Lanes per row: the best lane utilisation for `rows_stage` rows per stage and U units per row
// (ties: fewer lanes, so fewer reduction steps).
int pick_lanes(int U, int rows_stage) {
  int bestL = 1;
  double best = -1.0;
  for (int L = 1; L <= 64; L <<= 1) {
    const int WR = 64 / L;
    const int passes = (rows_stage + 4 * WR - 1) / (4 * WR);
    const int upl = (U + L - 1) / L;
    const double util = (double)rows_stage / (passes * 4.0 * WR) * (double)U / (double)(L * upl);
    if (util > best + 1e-9) {
      best = util;
      bestL = L;
    }
  }
  return bestL;
}

Geom make_geom(int fmt, int ncols, int nrows_total, bool gate_up) {
  Geom G{};
  G.U = ncols / 32;
  G.rb = ncols / block_weights(fmt) * block_bytes(fmt);
  if (gate_up) {
    int S = 32;
    while (S > 1 && 2 * (S * G.rb + kSlack + 16) > kWbufBudget) S >>= 1;
    G.S = S;
    G.tile = 32;
    G.ntiles = nrows_total / 32;
    G.L = pick_lanes(G.U, 2 * S);
  } else {
    int RD = kMaxRes;
    while (RD > 1 && RD * G.rb + kSlack + 16 > kWbufBudget) RD >>= 1;
    G.L = pick_lanes(G.U, RD);
    G.S = RD;
    G.tile = RD;
    G.ntiles = (nrows_total + RD - 1) / RD;
  }
  G.lgL = ilog2(G.L);
  G.upl = (G.U + G.L - 1) / G.L;
  return G;
}

int wbuf_for(const Geom& G, bool gate_up) {
  const int one = G.S * G.rb + kSlack + 16;
  return ((gate_up ? 2 * ((one + 15) & ~15) : one) + 15) & ~15;
}

struct WsLayout {
  size_t ctrl, hq_cnt, dt_cnt, g, u, hq, o, total;
};

size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(const moe_layer* L, const moe_plan* P, const Geom& GD) {
  WsLayout w{};
  size_t p = 0;
  w.ctrl = p;
  p += 256;
  w.hq_cnt = p;
  p += al256(MOE_MAX_GROUPS * 4);
  w.dt_cnt = p;
  p += al256((size_t)GD.ntiles * 4);
  const size_t ce = (size_t)P->cap_entries;
  w.g = p;
  p += al256(ce * L->n_ff * 4);
  w.u = p;
  p += al256(ce * L->n_ff * 4);
  w.hq = p;
  p += al256(ce * (L->n_ff / 32) * 36);
  w.o = p;
  p += al256(ce * L->n_embd * 4);
  w.total = p;
  return w;
}

Work work_ptrs(void* ws, const WsLayout& w) {
  uint8_t* b = (uint8_t*)ws;
  Work k;
  k.ctrl = (uint32_t*)(b + w.ctrl);
  k.hq_cnt = (uint32_t*)(b + w.hq_cnt);
  k.dt_cnt = (uint32_t*)(b + w.dt_cnt);
  k.g = (float*)(b + w.g);
  k.u = (float*)(b + w.u);
  k.hq = b + w.hq;
  k.o = (float*)(b + w.o);
  return k;
}

int check_layer(const moe_layer* L, bool need_down) {
  if (!L || !L->gate || !L->up || (need_down && !L->down)) return MOE_E_ARG;
  if (!fmt_ok(L->fmt_gate_up) || !fmt_ok(L->fmt_down)) return MOE_E_FMT;
  if (L->n_experts <= 0) return MOE_E_ARG;
  if (!cols_ok(L->fmt_gate_up, L->n_embd) || !cols_ok(L->fmt_down, L->n_ff)) return MOE_E_SHAPE;
  const bool nl4 = L->fmt_gate_up == NL4 || L->fmt_down == NL4;
  const bool cb2 = L->fmt_gate_up == CB2 || L->fmt_down == CB2;
  const bool cb3 = L->fmt_gate_up == CB3 || L->fmt_down == CB3;
  if ((nl4 && !L->nl4_table) || (cb2 && !L->cb2_grid) || (cb3 && !L->cb3_grid)) return MOE_E_ARG;
  return MOE_OK;
}

int check_plan(const moe_plan* P) {
  if (!P || !P->n_groups || !P->grp_expert || !P->grp_start || !P->ent_src || !P->ent_dst ||
      !P->ent_w || !P->err)
    return MOE_E_ARG;
  if (P->cap_groups < 1 || P->cap_groups > MOE_MAX_GROUPS || P->cap_entries < 1 ||
      P->cap_entries > MOE_MAX_CALL_ENTRIES)
    return MOE_E_ARG;
  return MOE_OK;
}

LayerArgs layer_args(const moe_layer* L) {
  return LayerArgs{L->n_embd, L->n_ff, L->n_experts, L->gate, L->up, L->down,
                   L->nl4_table, L->cb2_grid, L->cb3_grid};
}

PlanArgs plan_args(const moe_plan* P) {
  return PlanArgs{P->cap_groups, P->cap_entries, P->n_groups, P->grp_expert, P->grp_start,
                  P->ent_src, P->ent_dst, P->ent_w, P->err};
}

int num_cus() {
  static int cus = 0;
  static std::once_flag once;
  std::call_once(once, [] {
    int dev = 0;
    hipDeviceProp_t pr;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&pr, dev) == hipSuccess)
      cus = pr.multiProcessorCount;
    if (cus <= 0) cus = 256;
  });
  return cus;
}

template <class K>
hipError_t allow_smem(K kern, int bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <class K>
int occupancy(K kern, int bytes) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, kThreads, bytes) != hipSuccess || nb < 1)
    nb = 1;
  return nb;
}

}  // namespace moe

using namespace moe;

// ------------------------------------------------------------------ C ABI -------------------

extern "C" {

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_E_ARG: return "bad argument";
    case MOE_E_FMT: return "unknown weight format";
    case MOE_E_SHAPE: return "unsupported shape";
    case MOE_E_HIP: return "HIP error";
    case MOE_E_WS: return "workspace missing or too small";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return t_last_error.c_str(); }

int moe_quantize_q8_1(void* stream, const float* x, int rows, int n, void* q) {
  if (!x || !q || rows < 0 || n <= 0 || n % 32) return MOE_E_ARG;
  if (((uintptr_t)x & 15) || ((uintptr_t)q & 3)) return MOE_E_ARG;
  if (rows == 0) return MOE_OK;
  const long total = (long)rows * (n / 32);
  const int grid = (int)std::min<long>((total + kThreads - 1) / kThreads, 4096);
  hipLaunchKernelGGL(k_quantize, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, x, rows, n,
                     (uint8_t*)q);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_quantize_q8_1");
}

int moe_route_topk(void* stream, const float* logits, int T, int E, int k, int32_t* ids, float* w) {
  if (!logits || !ids || !w || T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > 32)
    return MOE_E_ARG;
  if (T == 0) return MOE_OK;
  hipLaunchKernelGGL(k_route, dim3((T + 3) / 4), dim3(kThreads), 0, (hipStream_t)stream, logits, T,
                     E, k, ids, w);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route_topk");
}

int moe_build_plan(void* stream, const int32_t* ids, const float* w, const int32_t* dst_of_token,
                   int T, int k, int E, int entry_base, const moe_plan* P) {
  int rc = check_plan(P);
  if (rc) return rc;
  if (!ids || !w || T < 0 || k < 1 || E < 1 || entry_base < 0) return MOE_E_ARG;
  if (T * k > P->cap_entries || T * k > P->cap_groups || T * k > 64) return MOE_E_ARG;
  const PlanOut po{P->n_groups, P->grp_expert, P->grp_start, P->ent_src, P->ent_dst, P->ent_w, P->err};
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(64), 0, (hipStream_t)stream, ids, w, dst_of_token, T, k, E,
                     entry_base, po);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_build_plan");
}

int moe_gate_up(void* stream, const moe_layer* L, const moe_plan* P, const void* xq, int n_tokens,
                float* g, float* u, int ld, int grid_limit) {
  int rc = check_layer(L, false);
  if (rc) return rc;
  if ((rc = check_plan(P))) return rc;
  if (!xq || !g || !u || ld < L->n_ff || n_tokens < 0 || grid_limit < 0) return MOE_E_ARG;
  if ((uintptr_t)xq & 3) return MOE_E_ARG;
  const Geom G = make_geom(L->fmt_gate_up, L->n_embd, L->n_ff, true);
  const int umax = G.U;
  const int wbuf = wbuf_for(G, true);
  const int bytes = smem_bytes(wbuf, umax);
  const int cap_items = P->cap_groups * G.ntiles;
  hipError_t e = hipSuccess;
  auto launch = [&](auto kern) {
    if ((e = allow_smem(kern, bytes)) != hipSuccess) return;
    int grid = grid_limit ? grid_limit : occupancy(kern, bytes) * num_cus();
    grid = std::max(1, std::min(grid, cap_items));
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), bytes, (hipStream_t)stream, layer_args(L),
                       plan_args(P), G, wbuf, umax, (const uint8_t*)xq, n_tokens, g, u, ld);
    e = hipGetLastError();
  };
  switch (L->fmt_gate_up) {
    case Q8_0: launch(k_gate_up<Q8_0>); break;
    case NL4: launch(k_gate_up<NL4>); break;
    case CB2: launch(k_gate_up<CB2>); break;
    default: launch(k_gate_up<CB3>); break;
  }
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_gate_up");
}

int moe_swiglu_q8_1(void* stream, const moe_plan* P, const float* g, const float* u, int n_ff, int ld,
                    float* h, void* hq) {
  int rc = check_plan(P);
  if (rc) return rc;
  if (!g || !u || !hq || n_ff <= 0 || n_ff % 32 || n_ff > MOE_MAX_DIM || ld < n_ff) return MOE_E_ARG;
  if ((uintptr_t)hq & 3) return MOE_E_ARG;
  const int total = P->cap_entries * (n_ff / 32);
  const int grid = std::max(1, std::min((total + 7) / 8, 2048));
  hipLaunchKernelGGL(k_swiglu, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, plan_args(P), g, u,
                     n_ff, ld, h, (uint8_t*)hq);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_swiglu_q8_1");
}

size_t moe_workspace_bytes(const moe_layer* L, const moe_plan* P) {
  if (check_layer(L, true) || check_plan(P)) return 0;
  const Geom GD = make_geom(L->fmt_down, L->n_ff, L->n_embd, false);
  return ws_layout(L, P, GD).total;
}

int moe_workspace_layout(const moe_layer* L, const moe_plan* P, size_t off[4]) {
  int rc = check_layer(L, true);
  if (rc) return rc;
  if ((rc = check_plan(P))) return rc;
  if (!off) return MOE_E_ARG;
  const Geom GD = make_geom(L->fmt_down, L->n_ff, L->n_embd, false);
  const WsLayout w = ws_layout(L, P, GD);
  off[0] = w.g;
  off[1] = w.u;
  off[2] = w.hq;
  off[3] = w.o;
  return MOE_OK;
}

int moe_workspace_init(void* stream, void* ws, size_t ws_bytes) {
  if (!ws || ws_bytes < 256 || ((uintptr_t)ws & 255)) return MOE_E_WS;
  // counters live in the first ctrl + hq_cnt + dt_cnt bytes; clearing all of it is simplest
  const size_t n = ws_bytes / 4;
  hipLaunchKernelGGL(k_fill_zero, dim3(256), dim3(256), 0, (hipStream_t)stream, (uint32_t*)ws, n);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_workspace_init");
}

int moe_down_scatter(void* stream, const moe_layer* L, const moe_plan* P, const void* hq, float* Y,
                     int n_rows, int ldy, void* ws, size_t ws_bytes, int grid_limit) {
  int rc = check_layer(L, true);
  if (rc) return rc;
  if ((rc = check_plan(P))) return rc;
  if (!hq || !Y || n_rows < 0 || ldy < L->n_embd || grid_limit < 0) return MOE_E_ARG;
  if ((uintptr_t)hq & 3) return MOE_E_ARG;
  const Geom G = make_geom(L->fmt_down, L->n_ff, L->n_embd, false);
  const WsLayout wl = ws_layout(L, P, G);
  if (!ws || ws_bytes < wl.total || ((uintptr_t)ws & 255)) return MOE_E_WS;
  const Work wk = work_ptrs(ws, wl);
  const int umax = G.U;
  const int wbuf = wbuf_for(G, false);
  const int bytes = smem_bytes(wbuf, umax);
  const int cap_items = P->cap_groups * G.ntiles;
  hipError_t e = hipSuccess;
  auto launch = [&](auto kern) {
    if ((e = allow_smem(kern, bytes)) != hipSuccess) return;
    int grid = grid_limit ? grid_limit : occupancy(kern, bytes) * num_cus();
    grid = std::max(1, std::min(grid, cap_items));
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), bytes, (hipStream_t)stream, layer_args(L),
                       plan_args(P), G, wbuf, umax, (const uint8_t*)hq, wk, Y, n_rows, ldy);
    e = hipGetLastError();
  };
  switch (L->fmt_down) {
    case Q8_0: launch(k_down<Q8_0>); break;
    case NL4: launch(k_down<NL4>); break;
    case CB2: launch(k_down<CB2>); break;
    default: launch(k_down<CB3>); break;
  }
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_down_scatter");
}

int moe_layer_decode(void* stream, const moe_layer* L, const moe_plan* P, const float* x, int n_tokens,
                     float* Y, int n_rows, int ldy, void* ws, size_t ws_bytes, int grid_limit) {
  int rc = check_layer(L, true);
  if (rc) return rc;
  if ((rc = check_plan(P))) return rc;
  if (!x || !Y || n_tokens < 0 || n_rows < 0 || ldy < L->n_embd || grid_limit < 0) return MOE_E_ARG;
  if ((uintptr_t)x & 15) return MOE_E_ARG;
  const Geom GU = make_geom(L->fmt_gate_up, L->n_embd, L->n_ff, true);
  const Geom GD = make_geom(L->fmt_down, L->n_ff, L->n_embd, false);
  const WsLayout wl = ws_layout(L, P, GD);
  if (!ws || ws_bytes < wl.total || ((uintptr_t)ws & 255)) return MOE_E_WS;
  const Work wk = work_ptrs(ws, wl);
  const int umax = std::max(GU.U, GD.U);
  const int wbuf = std::max(wbuf_for(GU, true), wbuf_for(GD, false));
  const int bytes = smem_bytes(wbuf, umax);
  const int cap_items = P->cap_groups * (GU.ntiles + GD.ntiles);
  hipError_t e = hipSuccess;
  auto launch = [&](auto kern) {
    if ((e = allow_smem(kern, bytes)) != hipSuccess) return;
    int grid = grid_limit ? grid_limit : occupancy(kern, bytes) * num_cus();
    grid = std::max(1, std::min(grid, cap_items));
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), bytes, (hipStream_t)stream, layer_args(L),
                       plan_args(P), GU, GD, wbuf, umax, x, n_tokens, wk, Y, n_rows, ldy);
    e = hipGetLastError();
  };
#define MOE_CASE(a, b)                 \
  if (L->fmt_gate_up == a && L->fmt_down == b) { \
    launch(k_layer<a, b>);             \
  } else
  MOE_CASE(Q8_0, Q8_0) MOE_CASE(Q8_0, NL4) MOE_CASE(Q8_0, CB2) MOE_CASE(Q8_0, CB3)
  MOE_CASE(NL4, Q8_0) MOE_CASE(NL4, NL4) MOE_CASE(NL4, CB2) MOE_CASE(NL4, CB3)
  MOE_CASE(CB2, Q8_0) MOE_CASE(CB2, NL4) MOE_CASE(CB2, CB2) MOE_CASE(CB2, CB3)
  MOE_CASE(CB3, Q8_0) MOE_CASE(CB3, NL4) MOE_CASE(CB3, CB2) MOE_CASE(CB3, CB3)
  { return MOE_E_FMT; }
#undef MOE_CASE
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_layer_decode");
}

}  // extern "C"
