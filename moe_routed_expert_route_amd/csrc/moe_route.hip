// Grouped routed-expert MoE decode for MI355X (gfx950): kernels and the C-ABI entry points.
//
// The step ("#363 experts: smaller and fewer launches for the verify window's PCIe call", opening
// paragraph and "What changes"; "#2058 Verify window: the routed experts' gate/up with the group's
// q8_1 rows in shared memory", "Why"): token-expert entries grouped by expert; each expert's
// gate/up weights streamed once per group and dotted with the group's q8_1 activation rows;
// SwiGLU + q8_1 fused; the down projection grouped the same way; its rows scatter-added into the
// destination rows with the router weights.
//
// Design for gfx950 (the pages' CUDA kernels are prior art, not the blueprint):
//  * Two launches per layer, no cross-workgroup synchronisation inside a kernel (a grid-wide
//    release/acquire costs tens of microseconds on this part; the kernel boundary is cheaper):
//      gate/up kernel: one work item = one 32-row h block of one group (rows of gate and up), so
//        SwiGLU and the q8_1 quantization of that h block finish in the same workgroup;
//      down kernel: one work item = a tile of rows of Y across every group of the call, so each
//        output element is summed by one workgroup in ascending entry order (deterministic, no
//        atomics, no partial buffers).
//  * Each wave streams its own weight rows HBM -> LDS with direct-to-LDS 16-byte loads
//    (global_load_lds_dwordx4, fully coalesced whatever the block size: 18/34/70/110-byte blocks
//    do not align to 16 bytes) through a private ring of slots. Every chunk costs exactly M load
//    instructions per wave, so "chunk k has landed" is a vmcnt wait with a known count: loads of
//    later chunks stay in flight while the wave computes, with no workgroup barrier in the loop.
//  * Weight units are decoded out of LDS at any byte alignment (v_alignbyte); activations sit in
//    LDS as q8_1 (split 16-byte halves + float scale for the gate/up kernel, raw 36-byte blocks
//    next to the weights for the down kernel).
//  * A row is split over L lanes (a power of two chosen from the shape only); lane l takes units
//    l, l+L, ...; per unit v_dot4 (int8) per 4 weights, then scale * d_x * isum in float32; the L
//    partial sums meet in a fixed DPP tree. The lane map depends only on the shape, so every
//    kernel variant and every grid produces the same bits.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/moe_route.h"
#include "moe_device.hpp"

namespace moe {

constexpr int kWaves = 4;                      // every heavy kernel runs 4 waves (256 threads)
constexpr int kMaxEnt = MOE_MAX_CALL_ENTRIES;  // 64
constexpr int kChunkCap = 8192;                // weight bytes per streamed chunk (target)

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

struct PlanArgs {
  int cap_groups, cap_entries;
  int32_t* n_groups;
  int32_t* grp_expert;
  int32_t* grp_start;
  int32_t* ent_src;
  int32_t* ent_dst;
  float* ent_w;
  uint32_t* err;
};

// Row geometry of one matrix kind (gate/up rows have n_embd columns, down rows n_ff), decided on
// the host from the shape alone.
struct Geom {
  int U;      // 32-weight units per row
  int L;      // lanes per row
  int lgL;    // log2 L
  int upl;    // units per lane, ceil(U / L)
  int rb;     // bytes per row
  int rp;     // rows per wave pass (64 / L)
};

// Per-wave stream: NS slots of M KB each.
struct Stream {
  int M, NS;
};

// ------------------------------------------------------------------ small helpers -----------

// Values broadcast through LDS are the same in every lane; readfirstlane puts them in scalar
// registers, so branches and loop bounds built from them are whole-wave (scalar) branches and
// every barrier stays in control flow the compiler sees as uniform.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const uint8_t* uni_ptr(const uint8_t* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void set_err(uint32_t* err, uint32_t bit) {
  if (err) atomicOr(err, bit);
}

// s_waitcnt vmcnt(n) for n = 0..63, leaving expcnt and lgkmcnt alone (gfx9 encoding: vmcnt low
// bits [3:0], high bits [15:14], expcnt [6:4], lgkmcnt [11:8]).
#define MOE_VM(n) (((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
#define MOE_W1(n) case n: __builtin_amdgcn_s_waitcnt(MOE_VM(n)); break;
#define MOE_W8(b) MOE_W1(b) MOE_W1(b + 1) MOE_W1(b + 2) MOE_W1(b + 3) MOE_W1(b + 4) MOE_W1(b + 5) \
  MOE_W1(b + 6) MOE_W1(b + 7)
__device__ __forceinline__ void wait_vm(int n) {
  switch (n < 0 ? 0 : (n > 63 ? 63 : n)) {
    MOE_W8(0) MOE_W8(8) MOE_W8(16) MOE_W8(24) MOE_W8(32) MOE_W8(40) MOE_W8(48) MOE_W8(56)
    default: __builtin_amdgcn_s_waitcnt(MOE_VM(0)); break;
  }
}
#undef MOE_W8
#undef MOE_W1
// lgkmcnt(0) only: this wave's LDS reads have returned
#define MOE_WAIT_LGKM0 __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4))

// Issue exactly M 1-KB direct-to-LDS load instructions of this wave into `slot`: span a lands at
// slot offset (a & 15) (whole aligned 16-byte chunks), span b at chunk index cb (16-byte units),
// every other lane reloads span a's first chunk into the unused tail of the slot. Reading whole
// aligned 16-byte chunks never leaves the pages that hold a span.
__device__ __forceinline__ void issue_chunk(MOE_LDS uint8_t* slot, int M, const uint8_t* a, uint32_t na,
                                            const uint8_t* b, uint32_t nb, uint32_t cb) {
  const uint32_t lane = threadIdx.x & 63;
  const uintptr_t a0 = (uintptr_t)a & ~(uintptr_t)15;
  const uint32_t ca = ((uint32_t)((uintptr_t)a & 15) + na + 15) >> 4;
  const uintptr_t b0 = (uintptr_t)b & ~(uintptr_t)15;
  const uint32_t cbn = nb ? (((uint32_t)((uintptr_t)b & 15) + nb + 15) >> 4) : 0u;
  for (int i = 0; i < M; ++i) {
    const uint32_t c = (uint32_t)i * 64 + lane;
    uintptr_t src = a0;
    if (c < ca)
      src = a0 + 16ull * c;
    else if (c >= cb && c < cb + cbn)
      src = b0 + 16ull * (c - cb);
    __builtin_amdgcn_global_load_lds((const void*)src, (MOE_LDS void*)(slot + i * 1024), 16, 0, 0);
  }
}

__device__ void load_tables(const LayerArgs& A, bool need2, bool need3, MOE_LDS uint32_t* g2,
                            MOE_LDS uint32_t* g3, Tables& tb) {
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
    for (int i = threadIdx.x; i < 512; i += kThreads) g2[i] = ((const uint32_t*)A.cb2)[i];
  if (need3)
    for (int i = threadIdx.x; i < 512; i += kThreads) g3[i] = ((const uint32_t*)A.cb3)[i];
  tb.cb2 = g2;
  tb.cb3 = g3;
}

// ------------------------------------------------------------------ one row-pass of dots ----

// Activation slots in split form (gate/up kernel): 16-byte halves of the quants and the float
// scale per 32-value block, entry slot stride `umax`.
struct ActSplit {
  const MOE_LDS u32x4* lo;
  const MOE_LDS u32x4* hi;
  const MOE_LDS float* d;
  int umax;
  __device__ __forceinline__ void get(int e, int u, uint32_t q[8], float& dx) const {
    const u32x4 a = lo[e * umax + u], b = hi[e * umax + u];
    q[0] = a.x; q[1] = a.y; q[2] = a.z; q[3] = a.w;
    q[4] = b.x; q[5] = b.y; q[6] = b.z; q[7] = b.w;
    dx = d[e * umax + u];
  }
};

// Activation rows as raw 36-byte q8_1 blocks in LDS (down kernel): entry e's row at byte offset
// base + e * rowb, 4-byte aligned.
struct ActRaw {
  const MOE_LDS uint32_t* W;
  uint32_t base, rowb;
  __device__ __forceinline__ void get(int e, int u, uint32_t q[8], float& dx) const {
    const uint32_t o = (base + (uint32_t)e * rowb + 36u * (uint32_t)u) >> 2;
    dx = h2f(W[o] & 0xFFFFu);
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = W[o + 1 + i];
  }
};

// Dot the rows of one wave pass with ne (<= 4) activation entries. The wave's lanes cover rp rows
// (row i = lane >> lgL, i < nrows) of L lanes; row i's bytes start at LDS byte `row0 + i * rb`.
// out(i, e, value) is called by one lane per (row, entry) after the fixed-order lane reduction.
template <int FMT, class Act, class Out>
__device__ __forceinline__ void dot_pass(const MOE_LDS uint32_t* W, uint32_t row0, int nrows,
                                         const Geom& G, const Tables& tb, const Act& act, int ne,
                                         Out out) {
  const int lane = threadIdx.x & 63;
  const int i = lane >> G.lgL, li = lane & (G.L - 1);
  float acc[kMaxSlots] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (i < nrows) {
    const uint32_t row = row0 + (uint32_t)(i * G.rb);
    for (int k = 0; k < G.upl; ++k) {
      const int u = li + (k << G.lgL);
      if (u < G.U) {
        uint32_t c[8];
        float sc;
        decode_unit<FMT>(W, row, u, tb, c, sc);
#pragma unroll
        for (int e = 0; e < kMaxSlots; ++e) {
          if (e < ne) {
            uint32_t q[8];
            float dx;
            act.get(e, u, q, dx);
            int s = __builtin_amdgcn_sdot4((int)c[0], (int)q[0], 0, false);
            s = __builtin_amdgcn_sdot4((int)c[1], (int)q[1], s, false);
            s = __builtin_amdgcn_sdot4((int)c[2], (int)q[2], s, false);
            s = __builtin_amdgcn_sdot4((int)c[3], (int)q[3], s, false);
            s = __builtin_amdgcn_sdot4((int)c[4], (int)q[4], s, false);
            s = __builtin_amdgcn_sdot4((int)c[5], (int)q[5], s, false);
            s = __builtin_amdgcn_sdot4((int)c[6], (int)q[6], s, false);
            s = __builtin_amdgcn_sdot4((int)c[7], (int)q[7], s, false);
            acc[e] = acc[e] + (sc * dx) * (float)s;
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
      if (e < ne && (e & (G.L - 1)) == li) out(i, e, acc[e]);
  }
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
      *(uint32_t*)blk = d16 | (sum_field(d16, isum) << 16);
    }
  }
}

// ------------------------------------------------------------------ routing (workgroup) -----

// Top-k of one token's E logits by (logit descending, expert id ascending) with the whole
// workgroup: each expert's rank is the number of experts that beat it; ranks < k are selected.
// Weights: ex_j = exp(l_j - l_top) in rank order, w_j = ex_j / (((ex_0 + ex_1) + ex_2) + ...).
// lg: the token's logits staged in LDS. Writes ids/w (LDS) in rank order.
__device__ void route_token_wg(const MOE_LDS float* lg, int E, int k, MOE_LDS int* ids, MOE_LDS float* w,
                               MOE_LDS float* ex) {
  for (int e = threadIdx.x; e < E; e += kThreads) {
    const float v = lg[e];
    int rank = 0;
    for (int o = 0; o < E; ++o) {
      const float lo = lg[o];
      rank += (lo > v) | ((lo == v) & (o < e));
    }
    if (rank < k) ids[rank] = e;
  }
  __syncthreads();
  if ((int)threadIdx.x < k) ex[threadIdx.x] = expf(lg[ids[threadIdx.x]] - lg[ids[0]]);
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.0f;
    for (int j = 0; j < k; ++j) s = s + ex[j];
    ex[32] = s;
  }
  __syncthreads();
  if ((int)threadIdx.x < k) w[threadIdx.x] = ex[threadIdx.x] / ex[32];
  __syncthreads();
}

// Group n = T * k entries (ids/w in LDS, token-major) by expert into plan arrays in LDS: groups
// ascending by expert id, entries ascending by token inside a group; absolute entry indices start
// at entry_base. Invalid ids (out of [0, E)) are dropped and reported.
struct PlanLds {
  MOE_LDS int* ids;     // [64] in: entry expert (token-major)
  MOE_LDS float* w;     // [64] in: entry weight
  MOE_LDS int* first;   // [64] scratch
  MOE_LDS int* gexp;    // [64] out: group expert
  MOE_LDS int* gstart;  // [65] out: group start (absolute)
  MOE_LDS int* esrc;    // [64] out (relative to entry_base)
  MOE_LDS int* edst;
  MOE_LDS float* ew;
  MOE_LDS int* ng;      // [1]
};
constexpr int kPlanLdsInts = 64 * 8 + 2;

__device__ inline PlanLds plan_lds(MOE_LDS int* base) {
  return PlanLds{base, (MOE_LDS float*)(base + 64), base + 128, base + 192, base + 256, base + 321,
                 base + 385, (MOE_LDS float*)(base + 449), base + 513};
}

__device__ void group_entries_wg(const PlanLds& p, int T, int k, int E, const int32_t* dst_of_token,
                                 int entry_base, uint32_t* err) {
  const int n = T * k;
  const int i = threadIdx.x;
  int e = -1;
  if (i < n) {
    e = p.ids[i];
    if (e < 0 || e >= E) {
      set_err(err, MOE_ERR_EXPERT);
      e = -1;
    }
  }
  if (i < 64) p.first[i] = 0;
  __syncthreads();
  if (i < n) {
    int first = e >= 0;
    for (int q = 0; q < i && first; ++q) first = p.ids[q] != e;
    p.first[i] = first;
  }
  __syncthreads();
  if (i < n) {
    int grp = 0, before = 0, pos = 0, nvalid = 0, ngroups = 0;
    for (int m = 0; m < n; ++m) {
      const int em = p.ids[m];
      if (em < 0 || em >= E) continue;
      ++nvalid;
      ngroups += p.first[m];
      if (e < 0) continue;
      if (m < i && em == e) ++pos;
      if (em < e) {
        ++before;
        grp += p.first[m];
      }
    }
    if (e >= 0) {
      const int t = i / k;
      const int slot = before + pos;
      p.esrc[slot] = t;
      p.edst[slot] = dst_of_token ? dst_of_token[t] : t;
      p.ew[slot] = p.w[i];
      if (p.first[i]) {
        p.gexp[grp] = e;
        p.gstart[grp] = entry_base + before;
      }
    }
    if (i == 0) {
      p.gstart[ngroups] = entry_base + nvalid;
      *p.ng = ngroups;
    }
  }
  __syncthreads();
}

// Copy a plan built in LDS out to the caller's plan arrays.
__device__ void publish_plan(const PlanLds& p, const PlanArgs& P, int entry_base) {
  const int ng = uni(*p.ng);
  const int nv = uni(p.gstart[ng]) - entry_base;
  const int i = threadIdx.x;
  if (i < ng) {
    P.grp_expert[i] = p.gexp[i];
    P.grp_start[i] = p.gstart[i];
  }
  if (i == 0) {
    P.grp_start[ng] = p.gstart[ng];
    *P.n_groups = ng;
  }
  if (i < nv) {
    P.ent_src[entry_base + i] = p.esrc[i];
    P.ent_dst[entry_base + i] = p.edst[i];
    P.ent_w[entry_base + i] = p.ew[i];
  }
}

// ------------------------------------------------------------------ call validation ---------

struct Call {
  int ng, e0, e1;
};

// Validate the call's group table (thread 0) and broadcast it. Bad tables make the call empty.
__device__ Call read_call(const PlanArgs& P, MOE_LDS int* misc) {
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
        const int s = P.grp_start[g];
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
    misc[0] = ng;
    misc[1] = e0;
    misc[2] = e1;
  }
  __syncthreads();
  const Call c{uni(misc[0]), uni(misc[1]), uni(misc[2])};
  __syncthreads();
  return c;
}

// ------------------------------------------------------------------ gate/up kernel ----------

enum GuMode : int { GU_COMPOSED = 0, GU_FUSED = 1, GU_ROUTED = 2 };

struct GuArgs {
  LayerArgs A;
  PlanArgs P;
  Geom G;
  Stream S;
  int umax;             // activation slot stride (units)
  int n_tokens;
  const uint8_t* xq;    // composed: q8_1 rows per token
  const float* x;       // fused / routed: float rows per token
  float* g;             // composed: g rows (absolute entry, stride ld); fused: workspace rows
  float* u;
  int ld;
  uint8_t* hq;          // fused / routed: workspace q8_1 rows (relative entry)
  const float* logits;  // routed mode: [T][E] router logits
  int T, E, k;
  const int32_t* dst_of_token;
  int entry_base;
};

struct GuSmem {
  MOE_LDS uint8_t* ring;     // kWaves * NS * M KB
  MOE_LDS u32x4* qlo;        // [kMaxSlots][umax]
  MOE_LDS u32x4* qhi;
  MOE_LDS float* xd;
  MOE_LDS float* gu;         // [kMaxSlots][64]: g rows 0..31, u rows 32..63 of the h block
  MOE_LDS uint32_t* g2;      // 512 dwords
  MOE_LDS uint32_t* g3;      // 512 dwords
  MOE_LDS int* misc;         // [64]
  MOE_LDS int* plan;         // routed mode: kPlanLdsInts
  MOE_LDS float* lg;         // routed mode: logits [E] + ex [64]
};

__host__ __device__ inline int gu_smem_bytes(const Stream& S, int umax, int E) {
  return kWaves * S.NS * S.M * 1024 + kMaxSlots * umax * 36 + kMaxSlots * 64 * 4 + 4096 + 256 +
         (E > 0 ? kPlanLdsInts * 4 + (E + 64) * 4 : 0);
}

__device__ GuSmem gu_layout(const Stream& S, int umax) {
  extern __shared__ __align__(16) uint8_t smem[];
  GuSmem s;
  MOE_LDS uint8_t* p = (MOE_LDS uint8_t*)smem;
  s.ring = p;
  p += kWaves * S.NS * S.M * 1024;
  s.qlo = (MOE_LDS u32x4*)p;
  p += kMaxSlots * umax * 16;
  s.qhi = (MOE_LDS u32x4*)p;
  p += kMaxSlots * umax * 16;
  s.xd = (MOE_LDS float*)p;
  p += kMaxSlots * umax * 4;
  s.gu = (MOE_LDS float*)p;
  p += kMaxSlots * 64 * 4;
  s.g2 = (MOE_LDS uint32_t*)p;
  p += 2048;
  s.g3 = (MOE_LDS uint32_t*)p;
  p += 2048;
  s.misc = (MOE_LDS int*)p;
  p += 256;
  s.plan = (MOE_LDS int*)p;
  p += kPlanLdsInts * 4;
  s.lg = (MOE_LDS float*)p;
  return s;
}

// This h block's activations are loaded into registers before the weight stream is issued, so
// "they landed" is a vmcnt wait that leaves the stream in flight; they are then quantized (fused)
// or split (composed) into LDS.
constexpr int kActBlocks = 512;                          // ne * U handled in registers
constexpr int kXPass = kActBlocks * 8 / kThreads;        // float4 per lane (fused)
constexpr int kQPass = kActBlocks * 9 / kThreads;        // dwords per lane (composed)

template <int FMT, int MODE>
__global__ __launch_bounds__(kThreads) void k_gate_up(GuArgs a) {
  const GuSmem sm = gu_layout(a.S, a.umax);
  Tables tb;
  load_tables(a.A, FMT == CB2, FMT == CB3, sm.g2, sm.g3, tb);
  const Geom& G = a.G;
  const int nb = a.A.n_ff / 32;   // h blocks per group
  const int wave = threadIdx.x >> 6;
  const PlanLds pl = plan_lds(sm.plan);
  Call call;
  if constexpr (MODE == GU_ROUTED) {
    // route every token and group the entries here (every workgroup derives the same plan from
    // the same logits); workgroup 0 publishes it for the down kernel and the caller
    for (int t = 0; t < a.T; ++t) {
      for (int e = threadIdx.x; e < a.E; e += kThreads) sm.lg[e] = a.logits[(size_t)t * a.E + e];
      __syncthreads();
      route_token_wg(sm.lg, a.E, a.k, pl.ids + t * a.k, pl.w + t * a.k, sm.lg + a.E);
    }
    group_entries_wg(pl, a.T, a.k, a.E, a.dst_of_token, a.entry_base, a.P.err);
    if (blockIdx.x == 0) publish_plan(pl, a.P, a.entry_base);
    const int ng = uni(*pl.ng);
    call = Call{ng, a.entry_base, uni(pl.gstart[ng])};
  } else {
    call = read_call(a.P, sm.misc);
  }
  const int items = call.ng * nb;
  MOE_LDS uint8_t* myring = sm.ring + wave * a.S.NS * a.S.M * 1024;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int g = it / nb, j = it - g * nb;
    // group info (thread 0), broadcast
    if (threadIdx.x == 0) {
      int e, a0, a1;
      if constexpr (MODE == GU_ROUTED) {
        e = pl.gexp[g];
        a0 = pl.gstart[g];
        a1 = pl.gstart[g + 1];
      } else {
        e = a.P.grp_expert[g];
        a0 = a.P.grp_start[g];
        a1 = a.P.grp_start[g + 1];
      }
      int ok = 1;
      const uint8_t* w0 = nullptr;
      const uint8_t* w1 = nullptr;
      if (e < 0 || e >= a.A.n_experts) {
        set_err(a.P.err, MOE_ERR_EXPERT);
        ok = 0;
      } else {
        w0 = (const uint8_t*)a.A.gate[e];
        w1 = (const uint8_t*)a.A.up[e];
        if ((((uintptr_t)w0) | ((uintptr_t)w1)) & 1) {
          set_err(a.P.err, MOE_ERR_ALIGN);
          ok = 0;
        }
      }
      sm.misc[4] = ok;
      sm.misc[5] = a0;
      sm.misc[6] = a1;
      *(MOE_LDS uint64_t*)(sm.misc + 8) = (uint64_t)(uintptr_t)w0;
      *(MOE_LDS uint64_t*)(sm.misc + 10) = (uint64_t)(uintptr_t)w1;
    }
    __syncthreads();
    const int ok = uni(sm.misc[4]);
    const int a0 = uni(sm.misc[5]), a1 = uni(sm.misc[6]);
    const uint8_t* wg = uni_ptr((const uint8_t*)(uintptr_t)(*(const MOE_LDS uint64_t*)(sm.misc + 8)));
    const uint8_t* wu = uni_ptr((const uint8_t*)(uintptr_t)(*(const MOE_LDS uint64_t*)(sm.misc + 10)));
    __syncthreads();
    if (!ok) continue;
    for (int c0 = a0; c0 < a1; c0 += kMaxSlots) {
      const int ne = min(kMaxSlots, a1 - c0);
      // entry sources (invalid -> no activation, nothing written)
      if (threadIdx.x < kMaxSlots) {
        int src = -1;
        if ((int)threadIdx.x < ne) {
          if constexpr (MODE == GU_ROUTED)
            src = pl.esrc[c0 + threadIdx.x - a.entry_base];
          else
            src = a.P.ent_src[c0 + threadIdx.x];
          if (src < 0 || src >= a.n_tokens) {
            set_err(a.P.err, MOE_ERR_SRC);
            src = -1;
          }
        }
        sm.misc[12 + threadIdx.x] = src;
      }
      __syncthreads();
      int srcs[kMaxSlots];
#pragma unroll
      for (int e = 0; e < kMaxSlots; ++e) srcs[e] = uni(sm.misc[12 + e]);
      __builtin_amdgcn_s_waitcnt(MOE_VM(0));   // nothing of ours in flight before the stream
      // 1. activation loads into registers, older than every weight load issued below, with a
      //    fixed unrolled shape (constant register indices): fused, one float4 of x per lane and
      //    pass (8 lanes per 32-value block); composed, one dword of a q8_1 block per lane and pass
      const int nblk = ne * G.U;
      const bool in_regs = nblk <= kActBlocks;
      float4 xr[kXPass];
      uint32_t qr[kQPass];
      if (in_regs) {
        if constexpr (MODE == GU_COMPOSED) {
#pragma unroll
          for (int p = 0; p < kQPass; ++p) {
            const int f = threadIdx.x + p * kThreads;   // dword f % 9 of block f / 9
            qr[p] = 0;
            if (f < nblk * 9) {
              const int b = f / 9, e = b / G.U, u = b - e * G.U;
              if (srcs[e] >= 0)
                qr[p] = ((const uint32_t*)(a.xq + ((size_t)srcs[e] * G.U + u) * 36))[f - b * 9];
            }
          }
        } else {
#pragma unroll
          for (int p = 0; p < kXPass; ++p) {
            const int f = threadIdx.x + p * kThreads;   // float4 f % 8 of block f / 8
            xr[p] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (f < nblk * 8) {
              const int b = f >> 3, e = b / G.U, u = b - e * G.U;
              if (srcs[e] >= 0)
                xr[p] = ((const float4*)(a.x + (size_t)srcs[e] * a.A.n_embd + 32 * u))[f & 7];
            }
          }
        }
      }
      // 2. this wave's rows of the h block: gate rows [32 j + 8 wave, +8) then the same up rows,
      //    in chunks of up to rp rows, streamed through the wave's ring
      const int cpm = (8 + G.rp - 1) / G.rp;   // chunks per matrix
      const int nch = 2 * cpm;
      const int r_base = 32 * j + 8 * wave;
      const int pre = min(a.S.NS, nch);
      for (int kc = 0; kc < pre; ++kc) {
        const int m = kc / cpm, r0 = r_base + (kc - m * cpm) * G.rp;
        const int rows = min(G.rp, r_base + 8 - r0);
        issue_chunk(myring + kc * a.S.M * 1024, a.S.M, (m == 0 ? wg : wu) + (size_t)r0 * G.rb,
                    (uint32_t)(rows * G.rb), nullptr, 0, 0);
      }
      // 3. activations -> LDS split form once they have landed
      MOE_LDS uint32_t* qlo32 = (MOE_LDS uint32_t*)sm.qlo;
      MOE_LDS uint32_t* qhi32 = (MOE_LDS uint32_t*)sm.qhi;
      if (in_regs) {
        wait_vm(pre * a.S.M);
        if constexpr (MODE == GU_COMPOSED) {
#pragma unroll
          for (int p = 0; p < kQPass; ++p) {
            const int f = threadIdx.x + p * kThreads;
            if (f < nblk * 9) {
              const int b = f / 9, k = f - b * 9, e = b / G.U, u = b - e * G.U;
              const int slotw = e * a.umax + u;
              if (k == 0)
                sm.xd[slotw] = srcs[e] >= 0 ? h2f(qr[p] & 0xFFFFu) : 0.0f;
              else if (k <= 4)
                qlo32[slotw * 4 + k - 1] = qr[p];
              else
                qhi32[slotw * 4 + k - 5] = qr[p];
            }
          }
        } else {
#pragma unroll
          for (int p = 0; p < kXPass; ++p) {
            // every lane of the wave takes part in the 8-lane max (full-wave DPP)
            const int f = threadIdx.x + p * kThreads;
            const float4 v = xr[p];
            float m = fmaxf(fmaxf(__builtin_fabsf(v.x), __builtin_fabsf(v.y)),
                            fmaxf(__builtin_fabsf(v.z), __builtin_fabsf(v.w)));
            m = fmaxf(m, dpp<0xB1>(m));    // xor 1
            m = fmaxf(m, dpp<0x4E>(m));    // xor 2
            m = fmaxf(m, dpp<0x141>(m));   // the other quad of the 8
            if (p * kThreads < nblk * 8 && f < nblk * 8) {
              const int b = f >> 3, part = f & 7, e = b / G.U, u = b - e * G.U;
              const int slotw = e * a.umax + u;
              const float d = m / 127.0f;
              uint32_t packed = 0;
              if (m != 0.0f) {
                const float xs[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                  float r = round_half_away(xs[jj] / d);
                  r = r > 127.0f ? 127.0f : r;
                  r = r < -127.0f ? -127.0f : r;
                  packed |= ((uint32_t)(int)r & 0xFFu) << (8 * jj);
                }
              }
              if (part < 4)
                qlo32[slotw * 4 + part] = packed;
              else
                qhi32[slotw * 4 + part - 4] = packed;
              if (part == 0) sm.xd[slotw] = srcs[e] >= 0 ? h2f(f2h(d)) : 0.0f;
            }
          }
        }
      } else {
        // large activation sets: plain loads now (they wait behind the stream)
        for (int idx = threadIdx.x; idx < nblk; idx += kThreads) {
          const int e = idx / G.U, u = idx - e * G.U;
          u32x4 lo = {0u, 0u, 0u, 0u}, hi = lo;
          float d = 0.0f;
          if (srcs[e] >= 0) {
            uint32_t qq[9];
            if constexpr (MODE == GU_COMPOSED) {
              const uint32_t* pp = (const uint32_t*)(a.xq + ((size_t)srcs[e] * G.U + u) * 36);
#pragma unroll
              for (int q = 0; q < 9; ++q) qq[q] = pp[q];
              d = h2f(qq[0] & 0xFFFFu);
            } else {
              const float4* pp = (const float4*)(a.x + (size_t)srcs[e] * a.A.n_embd + 32 * u);
              float v[32];
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                const float4 ff = pp[q];
                v[4 * q] = ff.x;
                v[4 * q + 1] = ff.y;
                v[4 * q + 2] = ff.z;
                v[4 * q + 3] = ff.w;
              }
              const QBlock bq = quant_block(v);
#pragma unroll
              for (int q = 0; q < 8; ++q) qq[1 + q] = bq.q[q];
              d = bq.d;
            }
            lo = u32x4{qq[1], qq[2], qq[3], qq[4]};
            hi = u32x4{qq[5], qq[6], qq[7], qq[8]};
          }
          sm.qlo[e * a.umax + u] = lo;
          sm.qhi[e * a.umax + u] = hi;
          sm.xd[e * a.umax + u] = d;
        }
      }
      __syncthreads();
      // 4. compute chunk by chunk as they land; refill the freed slot
      const ActSplit act{sm.qlo, sm.qhi, sm.xd, a.umax};
      int issued = pre;
      for (int kc = 0; kc < nch; ++kc) {
        const int m = kc / cpm, r0 = r_base + (kc - m * cpm) * G.rp;
        const int rows = min(G.rp, r_base + 8 - r0);
        const uint8_t* src = (m == 0 ? wg : wu) + (size_t)r0 * G.rb;
        wait_vm((issued - 1 - kc) * a.S.M);
        MOE_LDS uint8_t* slot = myring + (kc % a.S.NS) * a.S.M * 1024;
        const uint32_t row0 = (uint32_t)(slot - sm.ring) + (uint32_t)((uintptr_t)src & 15);
        const int rrel = 32 * m + (r0 - 32 * j);   // row of the h block, g: 0..31, u: 32..63
        dot_pass<FMT>((const MOE_LDS uint32_t*)sm.ring, row0, rows, G, tb, act, ne,
                      [&](int i, int e, float v) { sm.gu[e * 64 + rrel + i] = v; });
        if (kc + a.S.NS < nch) {
          MOE_WAIT_LGKM0;   // this wave's LDS reads of the slot have returned
          const int k2 = kc + a.S.NS;
          const int m2 = k2 / cpm, r2 = r_base + (k2 - m2 * cpm) * G.rp;
          const int rows2 = min(G.rp, r_base + 8 - r2);
          issue_chunk(slot, a.S.M, (m2 == 0 ? wg : wu) + (size_t)r2 * G.rb, (uint32_t)(rows2 * G.rb),
                      nullptr, 0, 0);
          ++issued;
        }
      }
      __syncthreads();
      // 5. outputs of the h block: g/u rows and, fused, SwiGLU + q8_1 of the block
      for (int idx = threadIdx.x; idx < ne * 64; idx += kThreads) {
        const int e = idx >> 6, r = idx & 63;
        if (srcs[e] < 0) continue;
        const float v = sm.gu[e * 64 + r];
        const int row = 32 * j + (r & 31);
        if constexpr (MODE == GU_COMPOSED)
          (r < 32 ? a.g : a.u)[(size_t)(c0 + e) * a.ld + row] = v;
        else
          (r < 32 ? a.g : a.u)[(size_t)(c0 + e - call.e0) * a.A.n_ff + row] = v;
      }
      if constexpr (MODE != GU_COMPOSED) {
        const int e = threadIdx.x >> 5, l32 = threadIdx.x & 31;
        if (e < kMaxSlots) {   // 128 threads: 4 entries x 32 rows
          const bool live = e < ne && srcs[e] >= 0;
          const float gv = live ? sm.gu[e * 64 + l32] : 0.0f;
          const float uv = live ? sm.gu[e * 64 + 32 + l32] : 0.0f;
          uint8_t* blk = a.hq + (size_t)(c0 + e - call.e0) * nb * 36 + (size_t)j * 36;
          swiglu_q81_lanes(gv, uv, l32, live, blk, nullptr);
        }
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ down + scatter kernel ---

struct DnArgs {
  LayerArgs A;
  PlanArgs P;
  Geom G;
  Stream S;
  const uint8_t* hq;   // q8_1 rows of h
  int hq_abs;          // 1: rows by absolute entry; 0: by entry - grp_start[0]
  float* Y;
  int n_rows, ldy;
  int n_tokens;        // >= 0: also skip entries whose token is out of range
};

__host__ __device__ inline int dn_smem_bytes(const Stream& S, int rp) {
  return kWaves * S.NS * S.M * 1024 + kMaxEnt * rp * 4 + 4096 + kMaxEnt * 12 + 256 +
         (MOE_MAX_GROUPS + 2) * 4 + MOE_MAX_GROUPS * 8;
}

// One work item: rows [rp t, rp t + rp) of Y. Wave w takes the groups g = w, w + 4, ... in order;
// a chunk is a group's down rows of the tile plus the q8_1 rows of (up to 4 of) its entries.
// Per-entry rows of o stay in LDS; at the end every destination row is summed in ascending entry
// order: Y[d][r] = ((Y[d][r] + w_a o_a[r]) + w_b o_b[r]) + ...
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_down(DnArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const Geom& G = a.G;
  MOE_LDS uint8_t* ring = (MOE_LDS uint8_t*)smem;
  MOE_LDS float* ores = (MOE_LDS float*)(ring + kWaves * a.S.NS * a.S.M * 1024);   // [kMaxEnt][rp]
  MOE_LDS uint32_t* g2 = (MOE_LDS uint32_t*)(ores + kMaxEnt * G.rp);
  MOE_LDS uint32_t* g3 = g2 + 512;
  MOE_LDS int* mdst = (MOE_LDS int*)(g3 + 512);          // [kMaxEnt] dst (-1 = skip)
  MOE_LDS int* mown = mdst + kMaxEnt;                     // [kMaxEnt] owner flag
  MOE_LDS float* mw = (MOE_LDS float*)(mown + kMaxEnt);   // [kMaxEnt]
  MOE_LDS int* misc = (MOE_LDS int*)(mw + kMaxEnt);       // [64]
  MOE_LDS int* gs = misc + 64;                            // [MOE_MAX_GROUPS + 1] group starts
  // [MOE_MAX_GROUPS] down pointers, 8-byte aligned after one pad int
  MOE_LDS uint64_t* gw = (MOE_LDS uint64_t*)(gs + MOE_MAX_GROUPS + 2);
  Tables tb;
  load_tables(a.A, FMT == CB2, FMT == CB3, g2, g3, tb);
  const Call call = read_call(a.P, misc);
  if (call.ng == 0) return;
  const int n = call.e1 - call.e0;
  // the call's group table (starts and down pointers; 0 = skipped group), then entry metadata:
  // destination (or -1), weight, owner = first live entry naming its dst
  {
    const int i = threadIdx.x;
    if (i <= call.ng) gs[i] = a.P.grp_start[i];
    if (i < call.ng) {
      const int e = a.P.grp_expert[i];
      uint64_t w = 0;
      if (e < 0 || e >= a.A.n_experts) {
        set_err(a.P.err, MOE_ERR_EXPERT);
      } else {
        w = (uint64_t)(uintptr_t)a.A.down[e];
        if (w & 1) {
          set_err(a.P.err, MOE_ERR_ALIGN);
          w = 0;
        }
      }
      gw[i] = w;
    }
    __syncthreads();
    if (i < n) {
      const int ab = call.e0 + i;
      int gg = 0;
      while (gg + 1 < call.ng && gs[gg + 1] <= ab) ++gg;
      int dst = a.P.ent_dst[ab];
      if (dst < 0 || dst >= a.n_rows) {
        set_err(a.P.err, MOE_ERR_DST);
        dst = -1;
      }
      if (gw[gg] == 0) dst = -1;
      if (a.n_tokens >= 0) {
        const int src = a.P.ent_src[ab];
        if (src < 0 || src >= a.n_tokens) dst = -1;
      }
      mdst[i] = dst;
      mw[i] = a.P.ent_w[ab];
    }
    __syncthreads();
    if (i < n) {
      const int d = mdst[i];
      int owner = d >= 0;
      for (int q = 0; q < i && owner; ++q) owner = mdst[q] != d;
      mown[i] = owner;
    }
    __syncthreads();
  }
  const int wave = threadIdx.x >> 6;
  MOE_LDS uint8_t* myring = ring + wave * a.S.NS * a.S.M * 1024;
  const int hstride = G.U * 36;   // bytes per q8_1 row of h
  const int ntiles = (a.A.n_embd + G.rp - 1) / G.rp;
  // this wave's chunks: (group g = wave + 4 q, entries [c0, c0 + 4)), in ascending order
  int nch = 0;
  for (int g = wave; g < call.ng; g += kWaves) {
    const int a0 = uni(gs[g]), a1 = uni(gs[g + 1]);
    nch += (a1 - a0 + kMaxSlots - 1) / kMaxSlots;
  }
  struct Ck {
    int c0, ne;
    const uint8_t* w;
  };
  auto chunk_at = [&](int kc) -> Ck {
    int k = 0;
    for (int g = wave; g < call.ng; g += kWaves) {
      const int a0 = uni(gs[g]), a1 = uni(gs[g + 1]);
      const int np = (a1 - a0 + kMaxSlots - 1) / kMaxSlots;
      if (kc < k + np) {
        Ck c;
        c.c0 = a0 + (kc - k) * kMaxSlots;
        c.ne = min(kMaxSlots, a1 - c.c0);
        c.w = uni_ptr((const uint8_t*)(uintptr_t)gw[g]);
        return c;
      }
      k += np;
    }
    return Ck{0, 0, nullptr};
  };
  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int r0 = t * G.rp;
    const int nr = min(G.rp, a.A.n_embd - r0);
    const uint32_t nw = (uint32_t)(nr * G.rb);
    auto hsrc_of = [&](const Ck& c) {
      return a.hq + (size_t)(a.hq_abs ? c.c0 : c.c0 - call.e0) * hstride;
    };
    auto issue = [&](const Ck& c, MOE_LDS uint8_t* slot) {
      const uint8_t* hsrc = hsrc_of(c);
      if (c.w) {
        const uint8_t* wsrc = c.w + (size_t)r0 * G.rb;
        const uint32_t cb = (((uint32_t)((uintptr_t)wsrc & 15) + nw + 15) >> 4) + 1;
        issue_chunk(slot, a.S.M, wsrc, nw, hsrc, (uint32_t)(c.ne * hstride), cb);
      } else {
        issue_chunk(slot, a.S.M, hsrc, (uint32_t)(c.ne * hstride), nullptr, 0, 0);
      }
    };
    __builtin_amdgcn_s_waitcnt(MOE_VM(0));
    const int pre = min(a.S.NS, nch);
    for (int kc = 0; kc < pre; ++kc) issue(chunk_at(kc), myring + kc * a.S.M * 1024);
    int issued = pre;
    for (int kc = 0; kc < nch; ++kc) {
      const Ck c = chunk_at(kc);
      wait_vm((issued - 1 - kc) * a.S.M);
      MOE_LDS uint8_t* slot = myring + (kc % a.S.NS) * a.S.M * 1024;
      if (c.w) {
        const uint32_t sb = (uint32_t)(slot - ring);
        const uint8_t* wsrc = c.w + (size_t)r0 * G.rb;
        const uint32_t cb = (((uint32_t)((uintptr_t)wsrc & 15) + nw + 15) >> 4) + 1;
        const ActRaw act{(const MOE_LDS uint32_t*)ring, sb + 16 * cb + (uint32_t)((uintptr_t)hsrc_of(c) & 15),
                         (uint32_t)hstride};
        const int rel = c.c0 - call.e0;
        dot_pass<FMT>((const MOE_LDS uint32_t*)ring, sb + (uint32_t)((uintptr_t)wsrc & 15), nr, G, tb,
                      act, c.ne, [&](int i, int e, float v) { ores[(rel + e) * G.rp + i] = v; });
      }
      if (kc + a.S.NS < nch) {
        MOE_WAIT_LGKM0;
        issue(chunk_at(kc + a.S.NS), slot);
        ++issued;
      }
    }
    __syncthreads();
    // scatter: one thread per (owner entry, row)
    for (int idx = threadIdx.x; idx < n * nr; idx += kThreads) {
      const int i = idx / nr, m = idx - i * nr;
      if (!mown[i]) continue;
      const int d = mdst[i];
      float* y = a.Y + (size_t)d * a.ldy + r0 + m;
      float acc = *y;
      for (int q = i; q < n; ++q)
        if (mdst[q] == d) acc = acc + mw[q] * ores[q * G.rp + m];
      *y = acc;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ small kernels -----------

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

// One workgroup per token.
__global__ __launch_bounds__(kThreads) void k_route(const float* __restrict__ logits, int E, int k,
                                                    int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ float s_lg[1024 + 64];
  __shared__ int s_ids[32];
  __shared__ float s_w[32];
  const int t = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kThreads) s_lg[e] = logits[(size_t)t * E + e];
  __syncthreads();
  route_token_wg((MOE_LDS float*)s_lg, E, k, (MOE_LDS int*)s_ids, (MOE_LDS float*)s_w,
                 (MOE_LDS float*)(s_lg + 1024));
  if ((int)threadIdx.x < k) {
    ids[(size_t)t * k + threadIdx.x] = s_ids[threadIdx.x];
    w[(size_t)t * k + threadIdx.x] = s_w[threadIdx.x];
  }
}

__global__ __launch_bounds__(kThreads) void k_plan(const int32_t* __restrict__ ids, const float* __restrict__ w,
                                                   const int32_t* __restrict__ dst_of_token, int T, int k,
                                                   int E, int entry_base, PlanArgs P) {
  __shared__ int s_plan[kPlanLdsInts];
  const PlanLds p = plan_lds((MOE_LDS int*)s_plan);
  const int n = T * k;
  if ((int)threadIdx.x < n) {
    p.ids[threadIdx.x] = ids[threadIdx.x];
    p.w[threadIdx.x] = w[threadIdx.x];
  }
  __syncthreads();
  group_entries_wg(p, T, k, E, dst_of_token, entry_base, P.err);
  publish_plan(p, P, entry_base);
}

// Over (entry, h block) of the call: two blocks per wave.
__global__ __launch_bounds__(kThreads) void k_swiglu(PlanArgs P, const float* __restrict__ g,
                                                     const float* __restrict__ u, int n_ff, int ld,
                                                     float* h, uint8_t* hq) {
  __shared__ int s_misc[64];
  const Call call = read_call(P, (MOE_LDS int*)s_misc);
  const int nb = n_ff / 32;
  const int total = (call.e1 - call.e0) * nb;
  const int half = threadIdx.x >> 5, l32 = threadIdx.x & 31;
  // every wave runs the loop the same number of times (shuffles need both halves present)
  for (int base = blockIdx.x * 8; base < total; base += gridDim.x * 8) {
    const int it = base + half;
    const bool live = it < total;
    const int a = live ? call.e0 + it / nb : call.e0;
    const int b = live ? it % nb : 0;
    const float gv = live ? g[(size_t)a * ld + 32 * b + l32] : 0.0f;
    const float uv = live ? u[(size_t)a * ld + 32 * b + l32] : 0.0f;
    swiglu_q81_lanes(gv, uv, l32, live, hq + (size_t)a * nb * 36 + (size_t)b * 36,
                     h ? h + (size_t)a * ld + 32 * b : nullptr);
  }
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

// Lanes per row from the shape alone: among L = 4..64 whose wave pass (64 / L rows) keeps a chunk
// within kChunkCap bytes (and, for gate/up, at most the 8 rows a wave owns), the best lane
// utilisation U / (L ceil(U / L)); ties go to the smaller L.
Geom make_geom(int fmt, int ncols, bool gate_up) {
  Geom G{};
  G.U = ncols / 32;
  G.rb = ncols / block_weights(fmt) * block_bytes(fmt);
  int bestL = 64;
  double best = -1.0;
  for (int L = 4; L <= 64; L <<= 1) {
    const int rp = 64 / L;
    if (gate_up && rp > 8) continue;
    if (rp * G.rb > kChunkCap && L < 64) continue;
    const double util = (double)G.U / (double)(L * ((G.U + L - 1) / L));
    if (util > best + 1e-9) {
      best = util;
      bestL = L;
    }
  }
  G.L = bestL;
  G.lgL = ilog2(bestL);
  G.upl = (G.U + G.L - 1) / G.L;
  G.rp = 64 / G.L;
  return G;
}

// Per-wave stream: a slot holds the largest chunk (+ alignment slack) in whole KB; as many slots
// (up to 4) as fit in `budget` bytes per wave, and never more outstanding loads than vmcnt counts.
Stream make_stream(int chunk_bytes, int budget) {
  Stream S;
  S.M = (chunk_bytes + 32 + 1023) / 1024;
  S.NS = std::max(1, std::min(4, budget / (S.M * 1024)));
  while (S.NS > 1 && S.M * (S.NS - 1) > 63) --S.NS;
  return S;
}

Stream gu_stream(const Geom& G) { return make_stream(G.rp * G.rb, 24 * 1024); }
Stream dn_stream(const Geom& G) {
  // weights + one 16-byte gap + the q8_1 rows of up to 4 entries, each span 16-byte aligned
  return make_stream(G.rp * G.rb + kMaxSlots * G.U * 36 + 96, 24 * 1024);
}

struct WsLayout {
  size_t g, u, hq, total;
};

size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(const moe_layer* L, const moe_plan* P) {
  WsLayout w{};
  size_t p = 256;
  const size_t ce = (size_t)P->cap_entries;
  w.g = p;
  p += al256(ce * L->n_ff * 4);
  w.u = p;
  p += al256(ce * L->n_ff * 4);
  w.hq = p;
  p += al256(ce * (L->n_ff / 32) * 36);
  w.total = p;
  return w;
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

template <class K>
hipError_t allow_smem(K kern, int bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t launch_gu(int fmt, int mode, const GuArgs& ga, int grid, int bytes, hipStream_t st) {
  auto go = [&](auto kern) -> hipError_t {
    hipError_t e = allow_smem(kern, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), bytes, st, ga);
    return hipGetLastError();
  };
#define MOE_GU(F)                                              \
  case F:                                                      \
    return mode == GU_COMPOSED ? go(k_gate_up<F, GU_COMPOSED>) \
           : mode == GU_FUSED  ? go(k_gate_up<F, GU_FUSED>)    \
                               : go(k_gate_up<F, GU_ROUTED>);
  switch (fmt) {
    MOE_GU(Q8_0)
    MOE_GU(NL4)
    MOE_GU(CB2)
    MOE_GU(CB3)
  }
#undef MOE_GU
  return hipErrorInvalidValue;
}

hipError_t launch_dn(int fmt, const DnArgs& da, int grid, int bytes, hipStream_t st) {
  auto go = [&](auto kern) -> hipError_t {
    hipError_t e = allow_smem(kern, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), bytes, st, da);
    return hipGetLastError();
  };
  switch (fmt) {
    case Q8_0: return go(k_down<Q8_0>);
    case NL4: return go(k_down<NL4>);
    case CB2: return go(k_down<CB2>);
    case CB3: return go(k_down<CB3>);
  }
  return hipErrorInvalidValue;
}

// The gate/up kernel of `mode` over one grid sized for the plan's capacity.
int run_gate_up(hipStream_t st, const moe_layer* L, const moe_plan* P, int mode, const void* act,
                int n_tokens, float* g, float* u, int ld, uint8_t* hq, const float* logits, int T,
                int k, const int32_t* dst_of_token, int entry_base, int grid_limit) {
  const Geom G = make_geom(L->fmt_gate_up, L->n_embd, true);
  const Stream S = gu_stream(G);
  GuArgs ga{};
  ga.A = layer_args(L);
  ga.P = plan_args(P);
  ga.G = G;
  ga.S = S;
  ga.umax = G.U;
  ga.n_tokens = n_tokens;
  ga.xq = mode == GU_COMPOSED ? (const uint8_t*)act : nullptr;
  ga.x = mode == GU_COMPOSED ? nullptr : (const float*)act;
  ga.g = g;
  ga.u = u;
  ga.ld = ld;
  ga.hq = hq;
  ga.logits = logits;
  ga.T = T;
  ga.E = L->n_experts;
  ga.k = k;
  ga.dst_of_token = dst_of_token;
  ga.entry_base = entry_base;
  const int bytes = gu_smem_bytes(S, G.U, mode == GU_ROUTED ? L->n_experts : 0);
  const int items = P->cap_groups * (L->n_ff / 32);
  const int grid = std::max(1, grid_limit ? std::min(grid_limit, items) : items);
  const hipError_t e = launch_gu(L->fmt_gate_up, mode, ga, grid, bytes, st);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "gate/up kernel");
}

int run_down(hipStream_t st, const moe_layer* L, const moe_plan* P, const uint8_t* hq, int hq_abs,
             float* Y, int n_rows, int ldy, int n_tokens, int grid_limit) {
  const Geom G = make_geom(L->fmt_down, L->n_ff, false);
  const Stream S = dn_stream(G);
  DnArgs da{};
  da.A = layer_args(L);
  da.P = plan_args(P);
  da.G = G;
  da.S = S;
  da.hq = hq;
  da.hq_abs = hq_abs;
  da.Y = Y;
  da.n_rows = n_rows;
  da.ldy = ldy;
  da.n_tokens = n_tokens;
  const int bytes = dn_smem_bytes(S, G.rp);
  const int tiles = (L->n_embd + G.rp - 1) / G.rp;
  const int grid = std::max(1, grid_limit ? std::min(grid_limit, tiles) : tiles);
  const hipError_t e = launch_dn(L->fmt_down, da, grid, bytes, st);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "down kernel");
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
  hipLaunchKernelGGL(k_route, dim3(T), dim3(kThreads), 0, (hipStream_t)stream, logits, E, k, ids, w);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route_topk");
}

int moe_build_plan(void* stream, const int32_t* ids, const float* w, const int32_t* dst_of_token,
                   int T, int k, int E, int entry_base, const moe_plan* P) {
  int rc = check_plan(P);
  if (rc) return rc;
  if (!ids || !w || T < 0 || k < 1 || E < 1 || entry_base < 0) return MOE_E_ARG;
  if (T * k > P->cap_entries || T * k > P->cap_groups || T * k > 64) return MOE_E_ARG;
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kThreads), 0, (hipStream_t)stream, ids, w, dst_of_token, T, k,
                     E, entry_base, plan_args(P));
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
  return run_gate_up((hipStream_t)stream, L, P, GU_COMPOSED, xq, n_tokens, g, u, ld, nullptr,
                     nullptr, 0, 0, nullptr, 0, grid_limit);
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
  return ws_layout(L, P).total;
}

int moe_workspace_layout(const moe_layer* L, const moe_plan* P, size_t off[3]) {
  int rc = check_layer(L, true);
  if (rc) return rc;
  if ((rc = check_plan(P))) return rc;
  if (!off) return MOE_E_ARG;
  const WsLayout w = ws_layout(L, P);
  off[0] = w.g;
  off[1] = w.u;
  off[2] = w.hq;
  return MOE_OK;
}

int moe_down_scatter(void* stream, const moe_layer* L, const moe_plan* P, const void* hq, float* Y,
                     int n_rows, int ldy, int grid_limit) {
  int rc = check_layer(L, true);
  if (rc) return rc;
  if ((rc = check_plan(P))) return rc;
  if (!hq || !Y || n_rows < 0 || ldy < L->n_embd || grid_limit < 0) return MOE_E_ARG;
  if ((uintptr_t)hq & 3) return MOE_E_ARG;
  return run_down((hipStream_t)stream, L, P, (const uint8_t*)hq, 1, Y, n_rows, ldy, -1, grid_limit);
}

int moe_layer_decode(void* stream, const moe_layer* L, const moe_plan* P, const float* x, int n_tokens,
                     float* Y, int n_rows, int ldy, void* ws, size_t ws_bytes, int grid_limit) {
  int rc = check_layer(L, true);
  if (rc) return rc;
  if ((rc = check_plan(P))) return rc;
  if (!x || !Y || n_tokens < 0 || n_rows < 0 || ldy < L->n_embd || grid_limit < 0) return MOE_E_ARG;
  if ((uintptr_t)x & 15) return MOE_E_ARG;
  const WsLayout wl = ws_layout(L, P);
  if (!ws || ws_bytes < wl.total || ((uintptr_t)ws & 255)) return MOE_E_WS;
  uint8_t* b = (uint8_t*)ws;
  rc = run_gate_up((hipStream_t)stream, L, P, GU_FUSED, x, n_tokens, (float*)(b + wl.g),
                   (float*)(b + wl.u), L->n_ff, b + wl.hq, nullptr, 0, 0, nullptr, 0, grid_limit);
  if (rc) return rc;
  return run_down((hipStream_t)stream, L, P, b + wl.hq, 0, Y, n_rows, ldy, n_tokens, grid_limit);
}

int moe_layer_decode_routed(void* stream, const moe_layer* L, const moe_plan* P, const float* logits,
                            int T, int k, const int32_t* dst_of_token, int entry_base, const float* x,
                            float* Y, int n_rows, int ldy, void* ws, size_t ws_bytes, int grid_limit) {
  int rc = check_layer(L, true);
  if (rc) return rc;
  if ((rc = check_plan(P))) return rc;
  if (!logits || !x || !Y || T < 1 || k < 1 || k > 32 || k > L->n_experts || L->n_experts > 1024 ||
      entry_base < 0 || n_rows < 0 || ldy < L->n_embd || grid_limit < 0)
    return MOE_E_ARG;
  if (T * k > P->cap_entries || T * k > P->cap_groups || T * k > 64) return MOE_E_ARG;
  if ((uintptr_t)x & 15) return MOE_E_ARG;
  const WsLayout wl = ws_layout(L, P);
  if (!ws || ws_bytes < wl.total || ((uintptr_t)ws & 255)) return MOE_E_WS;
  uint8_t* b = (uint8_t*)ws;
  rc = run_gate_up((hipStream_t)stream, L, P, GU_ROUTED, x, T, (float*)(b + wl.g), (float*)(b + wl.u),
                   L->n_ff, b + wl.hq, logits, T, k, dst_of_token, entry_base, grid_limit);
  if (rc) return rc;
  return run_down((hipStream_t)stream, L, P, b + wl.hq, 0, Y, n_rows, ldy, T, grid_limit);
}

}  // extern "C"
