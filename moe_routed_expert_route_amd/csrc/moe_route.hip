// Grouped routed-expert MoE decode for MI355X (gfx950): kernels and the C-ABI entry points.
//
// The step ("#363 experts: smaller and fewer launches for the verify window's PCIe call", opening
// paragraph and "What changes"; "#2058 Verify window: the routed experts' gate/up with the group's
// q8_1 rows in shared memory", "Why"): token-expert entries grouped by expert; each expert's
// gate/up weights streamed once per group and dotted with the group's q8_1 activation rows;
// SwiGLU fused; the down projection grouped the same way; its rows scatter-added into the
// destination rows with the router weights.
//
// Design for gfx950 (the pages' CUDA kernels are prior art, not the blueprint):
//  * Two launches per layer. The gate/up kernel (16 waves, one workgroup per CU) routes the
//    tokens, groups the entries, quantizes x, streams the routed experts' gate and up rows, and
//    writes SwiGLU + q8_1 of h into the caller's workspace; its last workgroup also writes the
//    plan and a one-read descriptor of the call. The down kernel (8 waves) reads the descriptor
//    and the h rows and owns a tile of Y rows across every group, so each output element is
//    summed by one workgroup in ascending entry order (deterministic, no atomics).
//  * Work items: gate/up, one 32-row block of h of one group (SwiGLU and the block's q8_1 finish
//    inside the workgroup); down, tr = ceil(n_embd / CUs) rows of Y.
//  * Latency first: a layer call moves tens of MB, so every dependent round trip shows. The
//    leading kernel arguments (logits, NL4 table, x, the gate / up pointer arrays, T, E, n_embd)
//    arrive preloaded in scalar registers, so the first loads go out before the argument block
//    is read. Every workgroup routes the window itself: one wave per token (group-maxima
//    threshold, then exact ranks of the candidates), or for one-token windows all eight routing
//    waves rank every expert at once; after one workgroup barrier each wave finds its item's
//    expert and entries from the tokens' selection bitmaps and issues its weight loads.
//  * Weight streams: row-major rows (any byte alignment) come HBM -> LDS by direct-to-LDS 16-byte
//    loads (global_load_lds_dwordx4, one uniform base per span) through a private ring per wave;
//    loads complete in issue order, so "chunk k has landed" is a vmcnt wait on the loads issued
//    after it. Planar NL4 rows (codes on 16-byte boundaries) go straight into registers, one
//    16-byte load per lane and unit, their scale planes by one direct-to-LDS instruction.
//  * A row is split over L lanes (a power of two chosen from the shape only); lane l takes units
//    l, l+L, ...; per unit v_dot4 (int8) per 4 weights, then scale * d_x * isum in float32; the L
//    partial sums meet in a fixed DPP tree. The lane map depends only on the shape, so every
//    kernel variant, layout and grid produces the same bits.
//  * The prompt path (hundreds of tokens) runs the same per-entry computation as grouped GEMMs
//    on the matrix cores (v_mfma_i32_16x16x32_i8, one instruction per 32-weight block).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe_route.h"
#include "moe_device.hpp"

namespace moe {

constexpr int kGuWaves = 16, kGuThreads = 64 * kGuWaves;  // gate/up workgroup (one per CU)
constexpr int kDnWaves = 8, kDnThreads = 64 * kDnWaves;   // down workgroup
constexpr int kSlots = kMaxSlots;                         // entries per dot pass (4)
constexpr int kMaxEnt = MOE_MAX_CALL_ENTRIES;             // 64
constexpr int kMaxGrp = MOE_MAX_GROUPS;                   // 64
constexpr int kChunkCap = 8192;          // weight bytes per streamed chunk (target)
constexpr int kDnTileMax = 16;           // down: most rows of Y in one tile
constexpr int kGuActMax = 48 * 1024;     // LDS for the call's token activations (q8_1)
constexpr int kDnActMax = 64 * 1024;     // LDS for the call's h rows (q8_1)
constexpr int kLdsMax = 160 * 1024;      // LDS per workgroup on gfx950
constexpr int kMaxE = 1024;              // most experts a routed call handles
constexpr int kRtWaves = 8;              // routed mode: waves that route tokens (w, w + 8, ...)

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
  Lay ly;     // where a row's scales and codes sit (row-major or planar)
};

// Per-wave stream: NS slots of M KB each.
struct Stream {
  int M, NS;
};

// The call as the gate/up launch leaves it for the down launch (device memory, at the start of
// the workspace): int words, then the down pointers.
constexpr int kDescNg = 0, kDescE0 = 1, kDescN = 2;
constexpr int kDescGs = 4;                    // [kMaxGrp + 1] group starts, relative to e0
constexpr int kDescDst = kDescGs + 68;        // [kMaxEnt] destination row
constexpr int kDescW = kDescDst + kMaxEnt;    // [kMaxEnt] router weight (float)
constexpr int kDescLive = kDescW + kMaxEnt;   // [kMaxEnt] 1 = compute and scatter this entry
constexpr int kDescPtrByte = 4 * (kDescLive + kMaxEnt);   // [kMaxGrp] down pointers (u64)
constexpr int kDescBytes = kDescPtrByte + 8 * kMaxGrp;
constexpr int kDescReserve = 2048;            // workspace bytes reserved for it
// Layer mode, in the workspace after the descriptor (all zero before the first call): one arrival
// flag per workgroup (set to the call's tag once its q8_1 rows of h are in memory: plain stores,
// no read-modify-write on a shared line), the tag of the last call on a line of its own, and the
// done count in two levels (kCtrGroups group counts, then a top count of complete groups), one
// count per kCtrLine bytes (atomics on one line are served one after another).
constexpr int kLyMaxGrid = 1024;
constexpr int kCtrGroups = 16;
constexpr int kCtrLine = 256;
constexpr int kCtrOff = kDescReserve;
constexpr int kCtrFlags = 0;                          // u32 index: [kLyMaxGrid] arrival flags
constexpr int kCtrEpoch = kLyMaxGrid;                 // u32 index: tag of the last call
constexpr int kCtrDone = kLyMaxGrid + kCtrLine / 4;   // u32 index: the done counts
constexpr int kCtrBytes = 4 * kCtrDone + (kCtrGroups + 1) * kCtrLine;
static_assert(kDescPtrByte % 16 == 0 && kDescBytes % 16 == 0 && kDescBytes <= kDescReserve, "desc");
static_assert(kDescBytes <= kCtrOff && kCtrOff % kCtrLine == 0, "counts");

// ------------------------------------------------------------------ small helpers -----------

// Values broadcast through LDS are the same in every lane; readfirstlane puts them in scalar
// registers, so branches and loop bounds built from them are whole-wave (scalar) branches and
// every barrier stays in control flow the compiler sees as uniform.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uni64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ void set_err(uint32_t* err, uint32_t bit) {
  if (err) atomicOr(err, bit);
}

// Layer mode: count this workgroup into a two-level count at ctr + base lines (group blockIdx %
// kCtrGroups, then the top count of complete groups). True for the workgroup that completes the
// top count. One thread calls it.
__device__ __forceinline__ bool count_in(uint32_t* ctr, int base) {
  constexpr int kW = kCtrLine / 4;
  const int gi = (int)blockIdx.x % kCtrGroups;
  const int ngrp = min((int)gridDim.x, kCtrGroups);
  const uint32_t gsz = (gridDim.x - (uint32_t)gi + kCtrGroups - 1) / kCtrGroups;
  const uint32_t c = __hip_atomic_fetch_add(ctr + (base + gi) * kW, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (c != gsz - 1) return false;
  const uint32_t t =
      __hip_atomic_fetch_add(ctr + (base + kCtrGroups) * kW, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return t == (uint32_t)ngrp - 1;
}

// The launch's argument block, every 64-byte line requested at once. The compiler reads the
// fields where they are first used, and at the start of a launch each such read is a trip to
// memory that the next one waits behind; after this they hit the scalar cache.
template <typename Args>
__device__ __forceinline__ void warm_args() {
  typedef const __attribute__((address_space(4))) uint32_t* KP;
  const KP k = (KP)__builtin_amdgcn_kernarg_segment_ptr();
  uint32_t s = 0u;
#pragma unroll
  for (int o = 0; o < (int)sizeof(Args); o += 64) s ^= k[o / 4];
  asm volatile("" ::"s"(s));
}

// The argument struct at byte `off` of the launch's argument block, read only after the code
// before the call: the block's address goes through an empty asm the compiler cannot see into,
// so no field read can be scheduled ahead of it (loads of launch arguments are otherwise hoisted
// to the kernel's entry, with their waits). Every 64-byte line is requested at once first.
template <typename Args>
__device__ __forceinline__ Args args_after(uint32_t off) {
  typedef const __attribute__((address_space(4))) uint32_t* KP;
  uint64_t p = (uint64_t)(uintptr_t)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  const KP k = (KP)(p + off);
  uint32_t s = 0u;
#pragma unroll
  for (int o = 0; o < (int)sizeof(Args); o += 64) s ^= k[o / 4];
  asm volatile("" ::"s"(s));
  Args r;
  __builtin_memcpy(&r, (const void*)k, sizeof(Args));
  return r;
}

// The 16-byte NL4 table with vector loads (a scalar load would hold up every later wait on the
// scalar counter, which the argument reads also use, until it returns from memory).
__device__ __forceinline__ void load_nl4(const int8_t* p, uint32_t t[4]) {
  t[0] = t[1] = t[2] = t[3] = 0u;
  if (!p) return;
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));   // an offset the compiler cannot see is uniform
  const uint32_t* q = (const uint32_t*)(p + z);
  t[0] = q[0];
  t[1] = q[1];
  t[2] = q[2];
  t[3] = q[3];
}

// LDS written by some lanes of a wave, then read by other lanes of the same wave: a wave's LDS
// operations execute in order; this keeps the compiler from moving them across each other.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier for handing LDS between waves while global loads stay in flight: each wave's
// LDS operations before it have completed (lgkmcnt(0)), and the asm's memory clobber keeps the
// compiler from moving memory operations across it. (__syncthreads would also wait for every
// outstanding vector-memory load, direct-to-LDS stream chunks included.) Data a wave loaded into
// LDS directly must have been waited for (vmcnt) by that wave before the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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

// Ring slot of chunk kc for ns slots per wave (one or two slots: no division).
__device__ __forceinline__ int slot_of(int kc, int ns) {
  return ns == 1 ? 0 : ns == 2 ? (kc & 1) : kc % ns;
}

// Cache policy of the weight stream: non-temporal (each weight byte is read once per call), so the
// stream does not push the launch's code, arguments and small tables out of L2.
constexpr int kAuxStream = 2;

// Issue exactly n 1-KB direct-to-LDS load instructions of this wave into `dst`: the span of na
// bytes at `a` lands at dst offset (a & 15) as whole aligned 16-byte pieces (reading whole aligned
// pieces never leaves the pages that hold the span); lanes past the span reload its first piece
// into the rest of the n KB. Each instruction takes one uniform base and a 32-bit offset per lane.
__device__ __forceinline__ void issue_span(MOE_LDS uint8_t* dst, int n, const uint8_t* a, uint32_t na) {
  const uint32_t lane = threadIdx.x & 63;
  // the same in every lane: scalar registers (the compiler cannot tell by itself)
  const uint8_t* a0 = (const uint8_t*)(uintptr_t)uni64((uint64_t)(uintptr_t)a & ~15ull);
  const uint32_t ca = (uint32_t)uni((int)((((uint32_t)(uintptr_t)a & 15u) + na + 15u) >> 4));
  MOE_LDS uint8_t* d0 = (MOE_LDS uint8_t*)(uintptr_t)(uint32_t)uni((int)(uint32_t)(uintptr_t)dst);
  for (int i = 0; i < n; ++i) {
    const uint32_t c = (uint32_t)i * 64 + lane;
    __builtin_amdgcn_global_load_lds((const void*)(a0 + (c < ca ? 16u * c : 0u)), (MOE_LDS void*)(d0 + i * 1024),
                                     16, 0, kAuxStream);
  }
}

// Copy `bytes` (a multiple of 16) from a 16-byte aligned global span into LDS with direct-to-LDS
// 16-byte loads, 1 KB per instruction, the pieces spread over waves [0, nw); lanes past the end
// stay masked off. Every instruction is issued before anything the caller issues afterwards.
// DEV: device-scope loads (sc1: data another XCD wrote during this launch, not a stale L2 copy).
template <bool DEV = false>
__device__ __forceinline__ void dma_span(const uint8_t* src, uint32_t bytes, MOE_LDS uint8_t* dst, int wave,
                                         int nw) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t nc = bytes >> 4;
  for (uint32_t p = (uint32_t)wave; 64 * p < nc; p += (uint32_t)nw) {
    const uint32_t c = 64 * p + lane;
    if (c < nc)
      __builtin_amdgcn_global_load_lds((const void*)(src + 16ull * c), (MOE_LDS void*)(dst + 1024 * p), 16, 0,
                                       DEV ? 16 : 0);
  }
}

// ------------------------------------------------------------------ activations in LDS ------

// q8_1 activations in split form: 16-byte halves of the quants and the float scale per 32-value
// block; act row r (a token or an entry), unit u at slot r * U + u.
struct ActSplit {
  MOE_LDS u32x4* lo;
  MOE_LDS u32x4* hi;
  MOE_LDS float* d;
  MOE_LDS float* s;   // the blocks' sum fields f(s16), staged only for a Q5_1 matrix (else null)
  int U;
  __device__ __forceinline__ void get(int r, int u, uint32_t q[8], float& dx) const {
    const u32x4 a = lo[r * U + u], b = hi[r * U + u];
    q[0] = a.x; q[1] = a.y; q[2] = a.z; q[3] = a.w;
    q[4] = b.x; q[5] = b.y; q[6] = b.z; q[7] = b.w;
    dx = d[r * U + u];
  }
};

// with_s: also a region for the blocks' sum fields (the Q5_1 offset term reads them)
__device__ __forceinline__ ActSplit act_layout(MOE_LDS uint8_t* p, int rows, int U, bool with_s = false) {
  ActSplit a;
  a.lo = (MOE_LDS u32x4*)p;
  a.hi = a.lo + rows * U;
  a.d = (MOE_LDS float*)(a.hi + rows * U);
  a.s = with_s ? a.d + rows * U : nullptr;
  a.U = U;
  return a;
}
__host__ __device__ inline int act_bytes(int rows, int U, bool with_s = false) {
  return (rows * U * (with_s ? 40 : 36) + 15) & ~15;
}

// The same split form with each of its three regions padded to whole KB, so that whole-KB
// direct-to-LDS pieces land inside it.
__host__ __device__ inline int kb_pad(int b) { return (b + 1023) & ~1023; }
__device__ __forceinline__ ActSplit act_layout_kb(MOE_LDS uint8_t* p, int rows, int U, bool with_s = false) {
  ActSplit a;
  a.lo = (MOE_LDS u32x4*)p;
  a.hi = (MOE_LDS u32x4*)(p + kb_pad(rows * U * 16));
  a.d = (MOE_LDS float*)(p + 2 * kb_pad(rows * U * 16));
  a.s = with_s ? (MOE_LDS float*)(p + 2 * kb_pad(rows * U * 16) + kb_pad(rows * U * 4)) : nullptr;
  a.U = U;
  return a;
}
__host__ __device__ inline int act_bytes_kb(int rows, int U, bool with_s = false) {
  return 2 * kb_pad(rows * U * 16) + (with_s ? 2 : 1) * kb_pad(rows * U * 4);
}

// Activation rows are staged in a fixed unrolled shape (constant register indices, no scratch):
// float rows as one float4 per lane and pass (8 lanes per 32-value block, quantized with an
// 8-lane DPP max), q8_1 rows as one dword per lane and pass (9 per 36-byte block).
// Loads are branch-free (an index past the data reloads element 0, whose value is never used),
// so they all issue back to back and the register arrays stay plain registers. `q` is the
// thread's index among the NT threads (whole waves) that stage.
// The rows are contiguous (row r, unit u is block r U + u at base + 32 (r U + u)), so float4 f of
// the staged blocks sits at base + 4 f.
template <int NT, int NP>
__device__ __forceinline__ void act_issue_f(const float* base, int nblk, int q, float4 (&xr)[NP]) {
  if (nblk <= 0) return;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    int f = q + p * NT;   // float4 f % 8 of block f / 8
    f = f < nblk * 8 ? f : 0;
    xr[p] = ((const float4*)base)[f];
  }
}

template <int NT, int NP>
__device__ __forceinline__ void act_store_f(const float4 (&xr)[NP], int nblk, int q, const ActSplit& act) {
  if (nblk <= 0) return;
  MOE_LDS uint32_t* lo32 = (MOE_LDS uint32_t*)act.lo;
  MOE_LDS uint32_t* hi32 = (MOE_LDS uint32_t*)act.hi;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    // every lane of the wave takes part in the 8-lane max (full-wave DPP)
    const int f = q + p * NT;
    const float4 v = xr[p];
    float m = fmaxf(fmaxf(__builtin_fabsf(v.x), __builtin_fabsf(v.y)),
                    fmaxf(__builtin_fabsf(v.z), __builtin_fabsf(v.w)));
    m = fmaxf(m, dpp<0xB1>(m));    // xor 1
    m = fmaxf(m, dpp<0x4E>(m));    // xor 2
    m = fmaxf(m, dpp<0x141>(m));   // the other quad of the 8
    if (p * NT < nblk * 8 && f < nblk * 8) {
      const int b = f >> 3, part = f & 7;
      const QScale qs = q_scale(m);
      uint32_t packed = 0;
      if (m != 0.0f) {
        const float xs[4] = {v.x, v.y, v.z, v.w};
        packed = quant_pack4(xs, qs);
      }
      if (part < 4)
        lo32[b * 4 + part] = packed;
      else
        hi32[b * 4 + part - 4] = packed;
      if (part == 0) act.d[b] = h2f(f2h(qs.d));
    }
  }
}

// The blocks past what the registers held: plain loads and the scalar quantizer.
template <int NT>
__device__ void act_rest_f(const float* base, int b0, int nblk, int q, ActSplit act) {
  for (int b = b0 + q; b < nblk; b += NT) {
    const float4* pp = (const float4*)(base + 32 * (long)b);
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 ff = pp[i];
      v[4 * i] = ff.x;
      v[4 * i + 1] = ff.y;
      v[4 * i + 2] = ff.z;
      v[4 * i + 3] = ff.w;
    }
    const QBlock bq = quant_block(v);
    act.lo[b] = u32x4{bq.q[0], bq.q[1], bq.q[2], bq.q[3]};
    act.hi[b] = u32x4{bq.q[4], bq.q[5], bq.q[6], bq.q[7]};
    act.d[b] = bq.d;
  }
}

// q8_1 rows: block b (= row * U + unit) at base + b * 36.
template <int NT, int NP>
__device__ __forceinline__ void act_issue_q(const uint8_t* base, int nblk, uint32_t (&qr)[NP]) {
  if (nblk <= 0) return;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int f = (int)threadIdx.x + p * NT;   // dword f % 9 of block f / 9
    qr[p] = ((const uint32_t*)base)[f < nblk * 9 ? f : 0];
  }
}

template <int NT, int NP>
__device__ __forceinline__ void act_store_q(const uint32_t (&qr)[NP], int nblk, const ActSplit& act) {
  if (nblk <= 0) return;
  MOE_LDS uint32_t* lo32 = (MOE_LDS uint32_t*)act.lo;
  MOE_LDS uint32_t* hi32 = (MOE_LDS uint32_t*)act.hi;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int f = (int)threadIdx.x + p * NT;
    if (f < nblk * 9) {
      const int b = f / 9, k = f - b * 9;
      if (k == 0) {
        act.d[b] = h2f(qr[p] & 0xFFFFu);
        if (act.s) act.s[b] = h2f(qr[p] >> 16);
      } else if (k <= 4)
        lo32[b * 4 + k - 1] = qr[p];
      else
        hi32[b * 4 + k - 5] = qr[p];
    }
  }
}

template <int NT>
__device__ void act_rest_q(const uint8_t* base, int b0, int nblk, ActSplit act) {
  for (int b = b0 + (int)threadIdx.x; b < nblk; b += NT) {
    const uint32_t* pp = (const uint32_t*)(base + (size_t)b * 36);
    uint32_t qq[9];
#pragma unroll
    for (int q = 0; q < 9; ++q) qq[q] = pp[q];
    act.lo[b] = u32x4{qq[1], qq[2], qq[3], qq[4]};
    act.hi[b] = u32x4{qq[5], qq[6], qq[7], qq[8]};
    act.d[b] = h2f(qq[0] & 0xFFFFu);
    if (act.s) act.s[b] = h2f(qq[0] >> 16);
  }
}

// Stage activation blocks into `act`: the register loads of the first blocks (float rows: nreg
// blocks in NP passes; q8_1 rows: up to NT * NPMAX / 9 blocks in a pass count rounded up to a power
// of two) go out at once (straight-line code, no register array merges), then mid() runs (work
// that must not wait for those loads), then the blocks are quantized or split into LDS; blocks
// past the register passes follow with plain loads.
template <int NT, int NP, class Mid>
__device__ __forceinline__ void act_stage_f_np(const float* base, int nreg, int q, const ActSplit& act, Mid& mid) {
  float4 xr[NP];
  act_issue_f<NT, NP>(base, nreg, q, xr);
  mid(NP);
  act_store_f<NT, NP>(xr, nreg, q, act);
}
template <int NT, int NP, class Mid>
__device__ __forceinline__ void act_stage_q_np(const uint8_t* base, int nreg, const ActSplit& act, Mid& mid) {
  uint32_t qr[NP];
  act_issue_q<NT, NP>(base, nreg, qr);
  mid(NP);
  act_store_q<NT, NP>(qr, nreg, act);
}
template <int NT, int NPMAX, class Mid>
__device__ __forceinline__ void act_stage_q(const uint8_t* base, int nblk, const ActSplit& act, Mid mid) {
  const int nreg = min(nblk, NT * NPMAX / 9);
  const int np = (nreg * 9 + NT - 1) / NT;
  if (np == 0)
    mid(0);
  else if (np == 1)
    act_stage_q_np<NT, 1>(base, nreg, act, mid);
  else if (np == 2)
    act_stage_q_np<NT, 2>(base, nreg, act, mid);
  else if (np <= 4 || NPMAX < 8)
    act_stage_q_np<NT, (NPMAX < 4 ? NPMAX : 4)>(base, nreg, act, mid);
  else if (np <= 8 || NPMAX < 16)
    act_stage_q_np<NT, (NPMAX < 8 ? NPMAX : 8)>(base, nreg, act, mid);
  else
    act_stage_q_np<NT, NPMAX>(base, nreg, act, mid);
  if (nblk > nreg) act_rest_q<NT>(base, nreg, nblk, act);
}

// ------------------------------------------------------------------ one row-pass of dots ----

// Dot the rows of one wave pass with NE (<= 4) activation rows sidx[0..NE). The wave's lanes
// cover nrows rows (row i = lane >> lgL) of L lanes; rows i < half start at LDS byte ra + i rb,
// the others at rb0 + (i - half) rb. Lane li takes units li, li + L, ... of its row, in that order;
// the weight reads of the next unit and the activation reads of this one are in flight while this
// unit is decoded (straight-line reads: past the row's end a lane rereads unit 0 and drops the
// result). out(i, e, value) is called by one lane per (row, entry) after the fixed-order lane
// reduction.
template <int FMT, int NE, class Out>
__device__ __forceinline__ void dot_pass_n(const MOE_LDS uint32_t* W, uint32_t ra, uint32_t rb0, int half,
                                           int nrows, const Geom& G, const Tables& tb, const ActSplit& act,
                                           const int (&sidx)[kSlots], Out& out) {
  const int lane = threadIdx.x & 63;
  const int i = lane >> G.lgL, li = lane & (G.L - 1);
  float acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = 0.0f;
  if (i < nrows) {
    const uint32_t row = i < half ? ra + (uint32_t)(i * G.rb) : rb0 + (uint32_t)((i - half) * G.rb);
    auto unit_at = [&](int k) {
      const int u = li + (k << G.lgL);
      return u < G.U ? u : 0;
    };
    auto step = [&](const URaw<FMT>& r, int k) {
      const bool valid = li + (k << G.lgL) < G.U;
      const int u = unit_at(k);
      uint32_t q[NE][8];
      float dx[NE], sx[NE];
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        act.get(sidx[e], u, q[e], dx[e]);
        sx[e] = FMT == Q5_1 ? act.s[sidx[e] * act.U + u] : 0.0f;
      }
      __builtin_amdgcn_sched_barrier(0);   // keep the reads above ahead of the decode
      uint32_t c[8];
      float sc, mo;
      unit_decode<FMT>(r, u, tb, c, sc, mo);
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        // two independent chains (an integer sum: the order does not change it), so a wave
        // alone on its SIMD is not held up by one chain of eight dependent dot instructions
        int s0 = __builtin_amdgcn_sdot4((int)c[0], (int)q[e][0], 0, false);
        int s1 = __builtin_amdgcn_sdot4((int)c[1], (int)q[e][1], 0, false);
        s0 = __builtin_amdgcn_sdot4((int)c[2], (int)q[e][2], s0, false);
        s1 = __builtin_amdgcn_sdot4((int)c[3], (int)q[e][3], s1, false);
        s0 = __builtin_amdgcn_sdot4((int)c[4], (int)q[e][4], s0, false);
        s1 = __builtin_amdgcn_sdot4((int)c[5], (int)q[e][5], s1, false);
        s0 = __builtin_amdgcn_sdot4((int)c[6], (int)q[e][6], s0, false);
        s1 = __builtin_amdgcn_sdot4((int)c[7], (int)q[e][7], s1, false);
        const int s = s0 + s1;
        // a unit past the row's end adds +0.0f: acc never holds -0 (it starts at +0), so this
        // equals skipping the add
        float prod = (sc * dx[e]) * (float)s;
        // Q5_1: the block's offset times the activations' sum field, added after the product
        if constexpr (FMT == Q5_1) prod = prod + mo * sx[e];
        acc[e] = acc[e] + (valid ? prod : 0.0f);
      }
    };
    URaw<FMT> r0, r1;
    unit_load<FMT>(W, row, unit_at(0), G.ly, r0);
    // (landed before the loop: the loop is entered with no read of r0 in flight, as it leaves
    // each trip, so the waits inside it count only the reads issued in the trip)
    MOE_WAIT_LGKM0;
    for (int k = 0; k < G.upl; k += 2) {
      unit_load<FMT>(W, row, unit_at(k + 1), G.ly, r1);
      __builtin_amdgcn_sched_barrier(0);
      step(r0, k);
      if (k + 1 < G.upl) {
        unit_load<FMT>(W, row, unit_at(k + 2), G.ly, r0);
        __builtin_amdgcn_sched_barrier(0);
        step(r1, k + 1);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = group_sum(acc[e], G.L);
  // every lane of the row holds every sum; lane li stores the entries e = li (mod L)
  if (i < nrows) {
#pragma unroll
    for (int e = 0; e < NE; ++e)
      if ((e & (G.L - 1)) == li) out(i, e, acc[e]);
  }
}

// dot_pass_n for planar NL4 rows that start on a 16-byte boundary of LDS (ra, rb0 and the row
// stride multiples of 16): a unit's codes are one aligned 16-byte read at row + 16 u, its scale a
// 2-byte read at row + d_b + 2 u (no realignment of unaligned dwords). The same lane map, unit
// order and sums as dot_pass_n, so the same bits.
template <int NE, class Out>
__device__ __forceinline__ void dot_pass_pa(const MOE_LDS uint8_t* W8, uint32_t ra, uint32_t rb0, int half,
                                            int nrows, const Geom& G, const Tables& tb, const ActSplit& act,
                                            const int (&sidx)[kSlots], Out& out) {
  const int lane = threadIdx.x & 63;
  const int i = lane >> G.lgL, li = lane & (G.L - 1);
  float acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = 0.0f;
  if (i < nrows) {
    const MOE_LDS uint8_t* row = W8 + (i < half ? ra + (uint32_t)(i * G.rb) : rb0 + (uint32_t)((i - half) * G.rb));
    const MOE_LDS u32x4* cp = (const MOE_LDS u32x4*)row;
    const MOE_LDS uint16_t* sp = (const MOE_LDS uint16_t*)(row + G.ly.d_b);
    auto unit_at = [&](int k) {
      const int u = li + (k << G.lgL);
      return u < G.U ? u : 0;
    };
    auto step = [&](const u32x4& c4, uint32_t s16, int k) {
      const bool valid = li + (k << G.lgL) < G.U;
      const int u = unit_at(k);
      uint32_t q[NE][8];
      float dx[NE];
#pragma unroll
      for (int e = 0; e < NE; ++e) act.get(sidx[e], u, q[e], dx[e]);
      __builtin_amdgcn_sched_barrier(0);   // keep the reads above ahead of the decode
      const float sc = h2f(s16);
      uint32_t c[8];
      c[0] = lut16(c4.x, tb);
      c[1] = lut16(c4.y, tb);
      c[2] = lut16(c4.z, tb);
      c[3] = lut16(c4.w, tb);
      c[4] = lut16(c4.x >> 4, tb);
      c[5] = lut16(c4.y >> 4, tb);
      c[6] = lut16(c4.z >> 4, tb);
      c[7] = lut16(c4.w >> 4, tb);
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        int s0 = __builtin_amdgcn_sdot4((int)c[0], (int)q[e][0], 0, false);
        int s1 = __builtin_amdgcn_sdot4((int)c[1], (int)q[e][1], 0, false);
        s0 = __builtin_amdgcn_sdot4((int)c[2], (int)q[e][2], s0, false);
        s1 = __builtin_amdgcn_sdot4((int)c[3], (int)q[e][3], s1, false);
        s0 = __builtin_amdgcn_sdot4((int)c[4], (int)q[e][4], s0, false);
        s1 = __builtin_amdgcn_sdot4((int)c[5], (int)q[e][5], s1, false);
        s0 = __builtin_amdgcn_sdot4((int)c[6], (int)q[e][6], s0, false);
        s1 = __builtin_amdgcn_sdot4((int)c[7], (int)q[e][7], s1, false);
        const float prod = (sc * dx[e]) * (float)(s0 + s1);
        acc[e] = acc[e] + (valid ? prod : 0.0f);
      }
    };
    u32x4 c0 = cp[unit_at(0)], c1;
    uint32_t s0 = sp[unit_at(0)], s1;
    MOE_WAIT_LGKM0;
    for (int k = 0; k < G.upl; k += 2) {
      c1 = cp[unit_at(k + 1)];
      s1 = sp[unit_at(k + 1)];
      __builtin_amdgcn_sched_barrier(0);
      step(c0, s0, k);
      if (k + 1 < G.upl) {
        c0 = cp[unit_at(k + 2)];
        s0 = sp[unit_at(k + 2)];
        __builtin_amdgcn_sched_barrier(0);
        step(c1, s1, k + 1);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = group_sum(acc[e], G.L);
  if (i < nrows) {
#pragma unroll
    for (int e = 0; e < NE; ++e)
      if ((e & (G.L - 1)) == li) out(i, e, acc[e]);
  }
}

// pa: planar NL4 rows at 16-byte boundaries (dot_pass_pa)
template <int FMT, class Out>
__device__ __forceinline__ void dot_pass(const MOE_LDS uint32_t* W, uint32_t ra, uint32_t rb0, int half,
                                         int nrows, const Geom& G, const Tables& tb, const ActSplit& act,
                                         const int (&sidx)[kSlots], int ne, Out out, bool pa = false) {
  if constexpr (FMT == NL4) {
    if (pa) {
      const MOE_LDS uint8_t* W8 = (const MOE_LDS uint8_t*)W;
      switch (ne) {
        case 1: dot_pass_pa<1>(W8, ra, rb0, half, nrows, G, tb, act, sidx, out); break;
        case 2: dot_pass_pa<2>(W8, ra, rb0, half, nrows, G, tb, act, sidx, out); break;
        case 3: dot_pass_pa<3>(W8, ra, rb0, half, nrows, G, tb, act, sidx, out); break;
        default: dot_pass_pa<4>(W8, ra, rb0, half, nrows, G, tb, act, sidx, out); break;
      }
      return;
    }
  }
  switch (ne) {
    case 1: dot_pass_n<FMT, 1>(W, ra, rb0, half, nrows, G, tb, act, sidx, out); break;
    case 2: dot_pass_n<FMT, 2>(W, ra, rb0, half, nrows, G, tb, act, sidx, out); break;
    case 3: dot_pass_n<FMT, 3>(W, ra, rb0, half, nrows, G, tb, act, sidx, out); break;
    default: dot_pass_n<FMT, 4>(W, ra, rb0, half, nrows, G, tb, act, sidx, out); break;
  }
}

// ------------------------------------------------------------------ register-direct pass ---

// The planar NL4 layout puts every unit's 16 code bytes on a 16-byte boundary (the row's code
// plane first, then its fp16 scales), so a lane can load its own units straight into registers:
// one 16-byte load per unit, no LDS on the code side. The scale planes of the wave's rows (2 U
// bytes each, whole 16-byte pieces when U % 8 == 0) come in one direct-to-LDS instruction issued
// first, so the wait for a lane's code loads covers them. The lane map is the LDS pass's (row
// i = lane >> lgL, lane li takes units li, li + L, ... in order; past the row's end it reloads unit
// 0 and drops the result), and so are the dot and the sums: the same bits.
constexpr int kRegUnits = 5;   // most units per lane the register path holds (n_embd <= 2560 at 16 lanes a row)
constexpr int kRegSlots = 2;   // entries per register pass (more would spill next to the held units)
struct RegW {
  u32x4 c[kRegUnits];   // the unit's 16 code bytes
};
// (The down rows do not take this path: at their 4 lanes a row, one 16-byte load per lane and
// unit touches every row's line in 64-byte halves, which streamed measurably slower than the
// direct-to-LDS spans of whole contiguous chunks.)

// Issue the wave's loads (planar NL4): the scale planes of its rows into LDS at `sbuf` (row i's
// at sbuf + 2 U i; lane j < rows * U / 8 takes piece j % (U / 8) of row j / (U / 8), whose first
// byte is srow), then this lane's G.upl units of its row `row` into registers.
__device__ __forceinline__ void reg_issue(RegW& w, const uint8_t* row, const uint8_t* srow, int sj,
                                          MOE_LDS uint8_t* sbuf, const Geom& G, int li) {
  const int lane = threadIdx.x & 63;
  if (lane < G.rp * (G.U >> 3))
    __builtin_amdgcn_global_load_lds((const void*)(srow + G.ly.d_b + 16u * (uint32_t)sj), (MOE_LDS void*)sbuf, 16, 0,
                                     kAuxStream);
#pragma unroll
  for (int k = 0; k < kRegUnits; ++k) {
    if (k < G.upl) {
      int u = li + (k << G.lgL);
      u = u < G.U ? u : 0;
      w.c[k] = __builtin_nontemporal_load((const u32x4*)(row + G.ly.c_a * (uint32_t)u + G.ly.c_b));
    }
  }
}

// Dot the wave's rows (loaded by reg_issue) with NE <= 4 activation rows; out as dot_pass_n.
template <int NE, class Out>
__device__ __forceinline__ void dot_pass_reg_n(const RegW& w, const MOE_LDS uint16_t* sbuf, int nrows, const Geom& G,
                                               const Tables& tb, const ActSplit& act, const int (&sidx)[kSlots],
                                               Out& out) {
  const int lane = threadIdx.x & 63;
  const int i = lane >> G.lgL, li = lane & (G.L - 1);
  float acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = 0.0f;
  if (i < nrows) {
#pragma unroll
    for (int k = 0; k < kRegUnits; ++k) {
      if (k < G.upl) {
        const bool valid = li + (k << G.lgL) < G.U;
        const int u = valid ? li + (k << G.lgL) : 0;
        uint32_t q[NE][8];
        float dx[NE];
        __builtin_amdgcn_sched_barrier(0);   // one unit at a time: its activation reads, then its dots
#pragma unroll
        for (int e = 0; e < NE; ++e) act.get(sidx[e], u, q[e], dx[e]);
        uint32_t n[4] = {w.c[k].x, w.c[k].y, w.c[k].z, w.c[k].w};
        uint32_t sw = sbuf[i * G.U + u];
        // opaque to the optimiser: the decode stays here, per pass over the entries, instead of
        // being hoisted for every unit at once (which would hold all the decoded units live)
        asm volatile("" : "+v"(n[0]), "+v"(n[1]), "+v"(n[2]), "+v"(n[3]), "+v"(sw));
        uint32_t c[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = lut16(n[j], tb);            // weights 4j..4j+3 (low nibbles)
          c[j + 4] = lut16(n[j] >> 4, tb);   // weights 16+4j..16+4j+3 (high nibbles)
        }
        const float sc = h2f(sw & 0xFFFFu);
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          int s0 = __builtin_amdgcn_sdot4((int)c[0], (int)q[e][0], 0, false);
          int s1 = __builtin_amdgcn_sdot4((int)c[1], (int)q[e][1], 0, false);
          s0 = __builtin_amdgcn_sdot4((int)c[2], (int)q[e][2], s0, false);
          s1 = __builtin_amdgcn_sdot4((int)c[3], (int)q[e][3], s1, false);
          s0 = __builtin_amdgcn_sdot4((int)c[4], (int)q[e][4], s0, false);
          s1 = __builtin_amdgcn_sdot4((int)c[5], (int)q[e][5], s1, false);
          s0 = __builtin_amdgcn_sdot4((int)c[6], (int)q[e][6], s0, false);
          s1 = __builtin_amdgcn_sdot4((int)c[7], (int)q[e][7], s1, false);
          const float prod = (sc * dx[e]) * (float)(s0 + s1);
          acc[e] = acc[e] + (valid ? prod : 0.0f);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = group_sum(acc[e], G.L);
  if (i < nrows) {
#pragma unroll
    for (int e = 0; e < NE; ++e)
      if ((e & (G.L - 1)) == li) out(i, e, acc[e]);
  }
}

template <class Out>
__device__ __forceinline__ void dot_pass_reg(const RegW& w, const MOE_LDS uint16_t* sbuf, int nrows, const Geom& G,
                                             const Tables& tb, const ActSplit& act, const int (&sidx)[kSlots], int ne,
                                             Out out) {
  if (ne == 1)
    dot_pass_reg_n<1>(w, sbuf, nrows, G, tb, act, sidx, out);
  else
    dot_pass_reg_n<2>(w, sbuf, nrows, G, tb, act, sidx, out);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// ------------------------------------------------------------------ weighted scatter --------

// Row m of destination d, summed by its owner entry i: acc (the row's value in Y) plus w_q o_q[m]
// for the entries q >= i that name d, in ascending q ("#2058 ...", "Why": the down outputs of a
// token's experts are weighted by its router weights and added up). The LDS reads go out eight
// entries at a time, one wait per batch; the additions keep their order.
__device__ __forceinline__ float dst_sum(float acc, int i, int n, int d, int m, int tr, const MOE_LDS int* mdst,
                                         const MOE_LDS float* mw, const MOE_LDS float* ores) {
  for (int q0 = i; q0 < n; q0 += 8) {
    int dd[8];
    float ww[8], oo[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = min(q0 + j, n - 1);
      dd[j] = mdst[q];
      ww[j] = mw[q];
      oo[j] = ores[q * tr + m];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (q0 + j < n && dd[j] == d) acc = acc + ww[j] * oo[j];
  }
  return acc;
}

// ------------------------------------------------------------------ SwiGLU + q8_1 -----------

// 32 lanes (an aligned half-wave) turn 32 (g, u) pairs into one q8_1 block of h. Same arithmetic
// as quant_block: amax and the integer sum are order-free, so the bytes match it exactly.
__device__ __forceinline__ void swiglu_q81_lanes(float gv, float uv, int l32, bool live,
                                                 uint8_t* blk, float* hrow) {
  const float h = live ? swiglu(gv, uv) : 0.0f;
  if (live && hrow) hrow[l32] = h;
  const float amax = wave_max32(__builtin_fabsf(h));
  const QScale qs = q_scale(amax);
  const float d = qs.d;
  const int q = amax != 0.0f ? quant_code(h, qs) : 0;
  const int isum = wave_sum32(q);
  if (live) {
    blk[4 + l32] = (uint8_t)(q & 0xFF);
    if (l32 == 0) {
      const uint32_t d16 = f2h(d);
      *(uint32_t*)blk = d16 | (sum_field(d16, isum) << 16);
    }
  }
}

// Same block, stored in split form: quants 0-15 to lo, 16-31 to hi, the scale as float f(d16).
// Each quad of lanes packs its four quants into a dword; the stores are device-scope (they reach
// memory past this XCD's L2), so another workgroup of the same launch can read them once it has
// seen this workgroup's count.
// DEV: device-scope stores (the one-launch step reads them back in the same launch); otherwise
// plain stores, which the end of the launch makes visible to the next one.
template <bool DEV>
// ds (null, or a place per block): also the block's sum field f(s16), for a Q5_1 down matrix.
__device__ __forceinline__ void swiglu_q81_split(float gv, float uv, int l32, bool live, uint32_t* lo,
                                                 uint32_t* hi, float* dq, float* ds) {
  const float h = live ? swiglu(gv, uv) : 0.0f;
  const float amax = wave_max32(__builtin_fabsf(h));
  const QScale qs = q_scale(amax);
  const float d = qs.d;
  const int q = amax != 0.0f ? quant_code(h, qs) : 0;
  const uint32_t b = (uint32_t)q & 0xFFu;
  const uint32_t w = b | (dppu<0x55>(b) << 8) | (dppu<0xAA>(b) << 16) | (dppu<0xFF>(b) << 24);   // quad lanes 1, 2, 3
  uint32_t sw = 0u;
  if (ds) {   // (uniform) every lane of the 32 takes part in the sum
    const int isum = wave_sum32(q);
    sw = __float_as_uint(h2f(sum_field(f2h(d), isum)));
  }
  if (live) {
    uint32_t* qw = (l32 < 16 ? lo : hi) + ((l32 >> 2) & 3);
    const uint32_t dw = __float_as_uint(h2f(f2h(d)));
    if constexpr (DEV) {
      if ((l32 & 3) == 0) __hip_atomic_store(qw, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (l32 == 0) __hip_atomic_store((uint32_t*)dq, dw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (ds && l32 == 0) __hip_atomic_store((uint32_t*)ds, sw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if ((l32 & 3) == 0) *qw = w;
      if (l32 == 0) *(uint32_t*)dq = dw;
      if (ds && l32 == 0) *(uint32_t*)ds = sw;
    }
  }
}

// ------------------------------------------------------------------ routing (one wave per token)

// Unsigned key with the order of the float (-0 and +0 share a key). Finite floats map to keys of at
// least 0x00800000, so 0 sorts below every real key.
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t b = __float_as_uint(f + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unkey(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Exclusive prefix sum over the wave's lanes of values in [0, 2^bits), from ballots of their bit
// planes (lane l gets the sum over lanes below l); and the whole wave's sum (uniform).
__device__ __forceinline__ int lane_prefix(int v, int bits) {
  int s = 0;
  for (int b = 0; b < bits; ++b) {
    const uint64_t m = __ballot((v >> b) & 1);
    s += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
  }
  return s;
}
__device__ __forceinline__ int lane_sum(int v, int bits) {
  int s = 0;
  for (int b = 0; b < bits; ++b) s += __popcll(__ballot((v >> b) & 1)) << b;
  return s;
}

// One token's E (<= 1024) logits into LDS (dst[e], e < 64 ceil(E / 64)) with direct-to-LDS 4-byte
// loads of one wave; past E a lane reloads row[0], which the routing ignores.
__device__ __forceinline__ void issue_logits(const float* row, int E, MOE_LDS float* dst) {
  const int lane = threadIdx.x & 63;
  for (int j = 0; 64 * j < E; ++j) {
    const int e = 64 * j + lane;
    __builtin_amdgcn_global_load_lds((const void*)(row + (e < E ? e : 0)), (MOE_LDS void*)(dst + 64 * j), 4,
                                     0, 0);
  }
}
__host__ __device__ inline int logits_pad(int E) { return (E + 63) & ~63; }

// LDS words of one routing wave's scratch: the logits, the candidates' (key, id) pairs plus the
// words a candidate batch may read past them, 64 group maxima, 32 selected logits.
__host__ __device__ inline int route_scr_words(int E) { return 3 * logits_pad(E) + 32 + 64 + 32; }

// Top-k (k <= min(E, 32)) of one token's logits by one wave, by (logit descending, expert id
// ascending), then the router weights over the k chosen ("#363 ...", opening paragraph: each
// token of the window picks its top-k experts). Lane l holds experts e = 64 j + l, j < V. The
// steps are data-parallel over the lanes (every lane compares against values read from LDS by
// broadcast), so the wave runs short dependent chains:
//  1. threshold: the lanes form G groups (G a power of two, at least 2k and enough that k groups
//     hold experts); the k-th largest of the G group maxima is a key that at least k keys reach,
//     so every key among the top k reaches it;
//  2. the keys that reach it are the candidates (typically a little over k); an expert's rank is
//     the number of candidates that beat it (larger key, or equal key and lower id: one 64-bit
//     comparison of (key, ~id)), which equals its rank among all E since whatever beats a
//     candidate is a candidate;
//  3. weights in rank order: ex_j = exp(l_j - l_0), w_j = ex_j / (((ex_0 + ex_1) + ex_2) + ...).
// scr: route_scr_words(E) words holding the logits (issue_logits into its start). Writes ids[0..k)
// and w[0..k) in rank order and this token's selection as a bitmap bits[0..ceil(E / 32)) (bit e of
// word e / 32), all in LDS.
template <int V>
__device__ __forceinline__ void route_token_v(MOE_LDS uint32_t* scr, int E, int k, MOE_LDS int* ids,
                                              MOE_LDS float* w, MOE_LDS uint32_t* bits, bool need_w) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = (1ull << lane) - 1ull;
  const int Epad = logits_pad(E);
  const MOE_LDS float* lg = (const MOE_LDS float*)scr;
  MOE_LDS uint32_t* cand = scr + Epad;          // [2 Epad + 32] candidates' (key, ~id) pairs
  MOE_LDS uint32_t* gmx = cand + 2 * Epad + 32; // [64] group maxima
  MOE_LDS float* lsel = (MOE_LDS float*)(gmx + 64);   // [32] chosen logits in rank order
  uint32_t key[V];
  uint32_t m = 0u;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int e = 64 * j + lane;
    key[j] = e < E ? fkey(lg[64 * j + lane]) : 0u;   // 0: no expert (past E the word is ignored)
    m = max(m, key[j]);
  }
  // (key, ~id) of slot j: larger means ranked higher
  auto K = [&](int j) { return ((uint64_t)key[j] << 32) | (uint32_t)~(uint32_t)(64 * j + lane); };
  // 1. threshold
  int G = 4;
  while (G < 64 && (G < 2 * k || E * G < 64 * k)) G <<= 1;
  const int gsz = 64 / G;
  if (gsz >= 2) m = max(m, dppu<0xB1>(m));    // xor 1
  if (gsz >= 4) m = max(m, dppu<0x4E>(m));    // xor 2
  if (gsz >= 8) m = max(m, dppu<0x141>(m));   // row_half_mirror
  if (gsz >= 16) m = max(m, dppu<0x140>(m));  // row_mirror
  if ((lane & (gsz - 1)) == 0) gmx[lane / gsz] = m;
  wave_lds_sync();
  // how many group maxima exceed this lane's (broadcast reads, G <= 16 or G <= 64)
  int above = 0;
  for (int g0 = 0; g0 < G; g0 += 16) {   // 16 maxima a batch: 4 broadcast reads, one wait
    u32x4 v[4];
#pragma unroll
    for (int o = 0; o < 4; ++o) v[o] = *(const MOE_LDS u32x4*)(gmx + g0 + 4 * o);
#pragma unroll
    for (int o = 0; o < 4; ++o)
      above += (g0 + 4 * o < G) ? (int)(v[o].x > m) + (int)(v[o].y > m) + (int)(v[o].z > m) + (int)(v[o].w > m) : 0;
  }
  uint32_t thr = above < k ? m : 0xFFFFFFFFu;
  thr = min(thr, dppu<0xB1>(thr));
  thr = min(thr, dppu<0x4E>(thr));
  thr = min(thr, dppu<0x141>(thr));
  thr = min(thr, dppu<0x140>(thr));
  thr = min(min((uint32_t)__builtin_amdgcn_readlane((int)thr, 0), (uint32_t)__builtin_amdgcn_readlane((int)thr, 16)),
            min((uint32_t)__builtin_amdgcn_readlane((int)thr, 32), (uint32_t)__builtin_amdgcn_readlane((int)thr, 48)));
  // 2. candidates, packed in LDS in (j, lane) order, then each counts the candidates beating it
  bool cnd[V];
  int C = 0;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    cnd[j] = key[j] != 0u && key[j] >= thr;
    const uint64_t bm = __ballot(cnd[j]);
    if (cnd[j]) {
      const int pos = C + __popcll(bm & lt);
      cand[2 * pos] = (uint32_t)K(j);
      cand[2 * pos + 1] = key[j];
    }
    C += __popcll(bm);
  }
  wave_lds_sync();
  int r[V];
#pragma unroll
  for (int j = 0; j < V; ++j) r[j] = 0;
  constexpr int kB = V <= 4 ? 8 : 2;   // candidate pairs a batch (fewer registers for wide V)
  for (int c0 = 0; c0 < C; c0 += 2 * kB) {   // broadcast reads, one wait a batch
    u32x4 v[kB];
#pragma unroll
    for (int o = 0; o < kB; ++o) v[o] = *(const MOE_LDS u32x4*)(cand + 2 * c0 + 4 * o);
#pragma unroll
    for (int o = 0; o < kB; ++o) {
      const uint64_t ka = ((uint64_t)v[o].y << 32) | v[o].x, kb = ((uint64_t)v[o].w << 32) | v[o].z;
      const bool va = c0 + 2 * o < C, vb = c0 + 2 * o + 1 < C;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const uint64_t kj = K(j);
        r[j] += (int)(va && ka > kj) + (int)(vb && kb > kj);
      }
    }
  }
  // the chosen experts in rank order, and this token's selection as a bitmap (word = lane)
  uint32_t bw = 0u;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const bool sel = cnd[j] && r[j] < k;
    if (sel) {
      ids[r[j]] = 64 * j + lane;
      lsel[r[j]] = unkey(key[j]);
    }
    const uint64_t sm = __ballot(sel);
    if ((lane >> 1) == j) bw = (lane & 1) ? (uint32_t)(sm >> 32) : (uint32_t)sm;
  }
  const int nW = (E + 31) >> 5;
  if (lane < nW) bits[lane] = bw;
  // 3. weights
  if (!need_w) return;
  wave_lds_sync();
  float ex = 0.0f;
  if (lane < k) ex = expf(lsel[lane] - lsel[0]);
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum = sum + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
  if (lane < k) w[lane] = ex / sum;
  wave_lds_sync();
}

// Routing spread over the routing waves of a workgroup ("#363 ...", opening paragraph: each token
// of the window picks its top-k experts), for T (rounded up to a power of two, Tp) tokens of E
// experts (Ep: E rounded up to a power of two, at least 64) when Tp Ep <= nthreads: thread rt is
// (token t, expert e, part p) with parts = nthreads / (Tp Ep) adjacent lanes per (t, e); it counts
// the experts of its part of the row that beat e (a larger logit, or an equal one with a lower id),
// the parts' counts are summed over the lanes, and e is chosen iff fewer than k beat it (its rank).
// Exact, and the same selection as route_token.
// Writes the selection bitmaps bits[t nW ..] (each wave its slice of one token's row) and, in rank
// order, ids[t k + r] = e and lsel[t k + r] = the logit (the router weights follow from those).
// lg(t): token t's logits in LDS (read by broadcast).
__device__ __forceinline__ int pow2ceil(int v) { return v <= 1 ? 1 : 1 << (32 - __builtin_clz((uint32_t)(v - 1))); }
__device__ __forceinline__ int route_parts(int T, int E, int nthreads) {
  const int p = min(4, nthreads / (pow2ceil(T) * max(64, pow2ceil(E))));
  return p == 4 ? p : 0;   // four parts of at least 16 experts (else one wave per token)
}
template <class LgOf>
__device__ __forceinline__ void route_ranked(int rt, int T, int E, int k, int parts, LgOf lg, MOE_LDS int* ids,
                                             MOE_LDS float* lsel, MOE_LDS uint32_t* bits) {
  const int lane = threadIdx.x & 63;
  const int Ep = max(64, pow2ceil(E));
  const int lgP = __builtin_ctz((uint32_t)parts), lgE = __builtin_ctz((uint32_t)Ep);
  const int part = rt & (parts - 1), e = (rt >> lgP) & (Ep - 1), t = rt >> (lgP + lgE);
  const int chunk = Ep >> lgP;   // a multiple of 16
  const bool live = t < T && e < E;
  // (each row holds -inf from E to Ep: those never beat a logit)
  const MOE_LDS float* row = lg(live ? t : 0);
  // the floats order like their keys (fkey: -0 == +0), so a part counts the larger logits with one
  // compare each, and the equal ones (a tie goes to the lower id) are looked at again only in a
  // wave where some lane has one
  const float le = live ? row[e] + 0.0f : __builtin_huge_valf();
  const int j00 = part * chunk;
  int gt = 0, eq = 0;
  for (int i0 = 0; i0 < chunk; i0 += 16) {   // the same trip count in every lane
    f32x4 v[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) v[b] = *(const MOE_LDS f32x4*)(row + j00 + i0 + 4 * b);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      gt += (int)(v[b].x > le) + (int)(v[b].y > le) + (int)(v[b].z > le) + (int)(v[b].w > le);
      eq += (int)(v[b].x == le) + (int)(v[b].y == le) + (int)(v[b].z == le) + (int)(v[b].w == le);
    }
  }
  const int self = (e >= j00 && e < j00 + chunk) ? 1 : 0;   // e itself is equal to le
  int beats = gt;
  if (__ballot(live && eq > self)) {   // (rare) the equal logits of lower id beat e as well
    for (int i0 = 0; i0 < chunk; ++i0) {
      const int j = j00 + i0;
      beats += (j < e && row[j] + 0.0f == le) ? 1 : 0;
    }
  }
  beats += __builtin_amdgcn_update_dpp(0, beats, 0xB1, 0xF, 0xF, false);   // xor 1
  beats += __builtin_amdgcn_update_dpp(0, beats, 0x4E, 0xF, 0xF, false);   // xor 2
  const bool sel = live && beats < k;
  if (sel && part == 0) {
    ids[t * k + beats] = e;
    lsel[t * k + beats] = le;
  }
  // this wave's slice of the bitmap: its 16 experts e0.. of token t0 (lane i of the slice takes
  // the selection of lane 4 i)
  const int rt0 = rt - lane;
  const int e0 = (rt0 >> lgP) & (Ep - 1), t0 = rt0 >> (lgP + lgE);
  const int sv = __shfl(sel ? 1 : 0, (lane & 15) << 2);
  const uint64_t m = __ballot(lane < 16 && sv);
  const int nW = (E + 31) >> 5;
  if (t0 < T && e0 < 32 * nW && lane == 0)
    *((MOE_LDS uint16_t*)(bits + t0 * nW) + (e0 >> 4)) = (uint16_t)m;
}

// need_w: also the weights (a caller that only needs the selection skips them)
__device__ __forceinline__ void route_token(MOE_LDS uint32_t* scr, int E, int k, MOE_LDS int* ids,
                                            MOE_LDS float* w, MOE_LDS uint32_t* bits, bool need_w = true) {
  if (E <= 128)
    route_token_v<2>(scr, E, k, ids, w, bits, need_w);
  else if (E <= 256)
    route_token_v<4>(scr, E, k, ids, w, bits, need_w);
  else
    route_token_v<16>(scr, E, k, ids, w, bits, need_w);
}

// ------------------------------------------------------------------ plan in LDS -------------

struct PlanL {
  MOE_LDS int* rid;        // [64] routed expert of entry i (token-major: token i / k)
  MOE_LDS float* rw;       // [64] its router weight
  MOE_LDS uint32_t* skey;  // [64] grouping scratch
  MOE_LDS int* sidx;       // [64]
  MOE_LDS int* sexp;       // [64]
  MOE_LDS int* gexp;       // [64] group expert
  MOE_LDS int* gstart;     // [65] group start (absolute entry)
  MOE_LDS int* esrc;       // [64] entry (relative to e0): token
  MOE_LDS int* edst;       // [64] destination row
  MOE_LDS float* ew;       // [64] router weight
  MOE_LDS int* elive;      // [64] entry computed (source in range)
  MOE_LDS int* dtok;       // [64] destination of each token (routing)
  MOE_LDS int* misc;       // [16] 0: n_groups, 1: e0 (absolute), 2: e1, 3: raw n_groups
};
constexpr int kPlanLInts = 64 * 5 + 64 + 68 + 64 * 5 + 16;
constexpr int kPlanLBytes = (4 * kPlanLInts + 15) & ~15;

__device__ inline PlanL plan_l(MOE_LDS int* b) {
  PlanL p;
  p.rid = b;
  p.rw = (MOE_LDS float*)(b + 64);
  p.skey = (MOE_LDS uint32_t*)(b + 128);
  p.sidx = b + 192;
  p.sexp = b + 256;
  p.gexp = b + 320;
  p.gstart = b + 384;
  p.esrc = b + 452;
  p.edst = b + 516;
  p.ew = (MOE_LDS float*)(b + 580);
  p.elive = b + 644;
  p.dtok = b + 708;
  p.misc = b + 772;
  return p;
}
static_assert(788 == kPlanLInts, "plan layout");

// Group n (<= 64) entries (rid/rw, token-major with k per token) by expert with one wave: each
// entry's key (expert, entry index) gets its rank among all keys, the entries land in key order
// (groups ascending by expert, entries ascending by token inside a group), and a group starts
// where the expert changes. Ids out of [0, E) are dropped and reported. Entry indices are
// absolute from entry_base; esrc/edst/ew are relative to it.
__device__ __forceinline__ void group_wave(const PlanL& p, int n, int k, int E, int entry_base, uint32_t* err) {
  const int lane = threadIdx.x & 63;
  const uint64_t lt = (1ull << lane) - 1ull;
  int e = -1;
  uint32_t key = 0xFFFFFFFFu;
  if (lane < n) {
    e = p.rid[lane];
    if (e >= 0 && e < E) {
      key = ((uint32_t)e << 6) | (uint32_t)lane;
    } else {
      set_err(err, MOE_ERR_EXPERT);
      e = -1;
    }
  }
  p.skey[lane] = key;   // every lane: keys past n stay above every real key
  wave_lds_sync();
  int r = 0;
  u32x4 kk[16];
#pragma unroll
  for (int o4 = 0; o4 < 16; ++o4) kk[o4] = ((const MOE_LDS u32x4*)p.skey)[o4];
#pragma unroll
  for (int o4 = 0; o4 < 16; ++o4)
    r += (kk[o4].x < key) + (kk[o4].y < key) + (kk[o4].z < key) + (kk[o4].w < key);
  const bool valid = e >= 0;
  const int nv = __popcll(__ballot(valid));
  if (valid) {
    p.sexp[r] = e;
    p.sidx[r] = lane;
  }
  wave_lds_sync();
  // lane = position in key order
  const bool live = lane < nv;
  const int se = live ? p.sexp[lane] : -1;
  const int prev = (live && lane > 0) ? p.sexp[lane - 1] : -2;
  const bool first = live && se != prev;
  const uint64_t fm = __ballot(first);
  const int ng = __popcll(fm);
  if (first) {
    const int g = __popcll(fm & lt);
    p.gexp[g] = se;
    p.gstart[g] = entry_base + lane;
  }
  if (live) {
    const int i = p.sidx[lane];
    const int t = i / k;
    p.esrc[lane] = t;
    p.edst[lane] = p.dtok[t];
    p.ew[lane] = p.rw[i];
    p.elive[lane] = 1;
  }
  if (lane == 0) {
    p.gstart[ng] = entry_base + nv;
    p.misc[0] = ng;
    p.misc[1] = entry_base;
    p.misc[2] = entry_base + nv;
  }
  wave_lds_sync();
}

// Copy the plan built in LDS out to the caller's plan arrays (NT threads).
template <int NT>
__device__ __forceinline__ void publish_plan(const PlanL& p, const PlanArgs& P) {
  const int ng = uni(p.misc[0]), e0 = uni(p.misc[1]), n = uni(p.misc[2]) - e0;
  for (int i = threadIdx.x; i < ng; i += NT) {
    P.grp_expert[i] = p.gexp[i];
    P.grp_start[i] = p.gstart[i];
  }
  if (threadIdx.x == 0) {
    P.grp_start[ng] = p.gstart[ng];
    *P.n_groups = ng;
  }
  for (int i = threadIdx.x; i < n; i += NT) {
    P.ent_src[e0 + i] = p.esrc[i];
    P.ent_dst[e0 + i] = p.edst[i];
    P.ent_w[e0 + i] = p.ew[i];
  }
}

// A plan the caller built: validate the group table (thread 0; raw values in gs[0..cap] and
// raw_ng) and write n_groups, e0, e1 to out[0..2]. A bad table makes the call empty.
__device__ __forceinline__ void validate_groups(const MOE_LDS int* gs, int raw_ng, const PlanArgs& P, MOE_LDS int* out) {
  if (threadIdx.x == 0) {
    int ng = raw_ng;
    int e0 = 0, e1 = 0;
    if (ng < 0 || ng > P.cap_groups) {
      set_err(P.err, MOE_ERR_NGROUPS);
      ng = 0;
    }
    if (ng > 0) {
      e0 = gs[0];
      bool ok = e0 >= 0;
      int prev = e0;
      for (int g = 1; g <= ng; ++g) {
        const int s = gs[g];
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
    out[0] = ng;
    out[1] = e0;
    out[2] = e1;
  }
}

__device__ __forceinline__ bool ptr_ok(uint64_t v, uint32_t* err) {
  if (v & 1) {
    set_err(err, MOE_ERR_ALIGN);
    return false;
  }
  return true;
}

// ------------------------------------------------------------------ gate/up kernel ----------

// GU_LAYER: routed, and after every workgroup has finished its blocks (a device-scope count in the
// workspace) the same launch runs the grouped down projection and the weighted scatter.
enum GuMode : int { GU_COMPOSED = 0, GU_FUSED = 1, GU_ROUTED = 2, GU_LAYER = 3 };

struct GuArgs {
  LayerArgs A;
  PlanArgs P;
  Geom G;
  Stream S;
  int n_tokens;         // act rows (tokens)
  const uint8_t* xq;    // composed: q8_1 rows per token
  const float* x;       // fused / routed: float rows per token
  float* g;             // composed: g rows (absolute entry, stride ld)
  float* u;
  int ld;
  uint32_t* hq_lo;      // fused / routed: workspace q8_1 rows of h in split form (relative entry):
  uint32_t* hq_hi;      //   16-byte low and high halves of each block's quants, float scales
  float* hq_d;
  float* hq_s;          //   and (a Q5_1 down matrix only, else null) the blocks' sum fields
  uint8_t* desc;        // fused / routed: the call's descriptor for the down launch
  const float* logits;  // routed: [T][E] router logits
  int T, E, k;
  const int32_t* dst_of_token;
  int entry_base;
  int lds_ring, lds_act;
  int sw;               // waves that stream items (the ring holds sw waves' slots)
  int regw;             // planar NL4: each lane loads its weight units into registers (no ring)
  // layer mode: the down half
  Geom Gd;              // down row geometry (rows of n_ff columns)
  Stream Sd;            // down stream: kDnWaves waves, NS slots of M KB each, in the ring
  int trd;              // rows of Y per down tile (<= kDnTileMax)
  int rcd;              // rows per streamed down chunk
  float* Y;
  int n_rows, ldy;
  int lds_tail;         // bytes of the routed tail (the down region follows it)
  uint32_t nb_magic;    // floor(2^32 / (n_ff / 32)) (all ones for 1): division by the blocks per group
  uint32_t* ctr;        // workspace: [0] workgroups done with their blocks, [1] workgroups done
  int spin_limit;       // bounded wait for the other workgroups (then MOE_ERR_WAIT)
};

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

// Byte offset of the struct in k_gate_up's argument block: kernel arguments sit in order at their
// natural alignment, after five pointers and three ints (then padding to 8 bytes).
constexpr uint32_t kGuArgsOff = 56;
static_assert(alignof(GuArgs) <= 8, "GuArgs must start right after the leading arguments");

constexpr int kGuStage = 64 * kMaxEnt;   // floats of output staging: a 32-row block of g and u per entry
constexpr int kGuFixed = 4096 + kPlanLBytes + 8 * 3 * kMaxGrp + 4 * kGuStage;
constexpr int kGuXPass = 8;    // float4 (or q8_1 dword) register passes: 1024 float blocks, 910 q8_1
constexpr int kGuQThreads = kGuThreads - 64 * kRtWaves;   // routed: the waves that quantize x

// Routed mode: LDS after the fixed part: [E] gate and up pointers, [E] down pointers (0: the
// expert's pointers are unusable), [T][ceil(E / 32)] each token's selection bitmap.
__host__ __device__ inline int gu_tail_bytes(int E, int T) {
  return 24 * E + ((4 * T * ((E + 31) >> 5) + 15) & ~15);
}
__host__ __device__ inline int gu_smem_bytes(int lds_ring, int lds_act, int lds_tail) {
  return lds_ring + lds_act + kGuFixed + lds_tail;
}
// Layer mode, after the tail: the q8_1 rows of h (split form, KB-padded regions), the per-entry
// outputs of a down tile, the entries' metadata and the first tile's destination rows of Y.
constexpr int kLyMeta = 4 * (5 * kMaxEnt + 16);
constexpr int kLyYBuf = 4 * kMaxEnt * kDnTileMax;
__host__ __device__ inline int ly_down_bytes(int cap_entries, int Ud, bool with_s) {
  return act_bytes_kb(cap_entries, Ud, with_s) + 4 * kMaxEnt * kDnTileMax + kLyMeta + kLyYBuf;
}

// Work item = one 32-row block of h of one group (so SwiGLU and the q8_1 quantization of the block
// finish in the workgroup). The block's 64 weight rows are 64 / rp passes of rp rows (rp / 2 gate
// rows and the same up rows, one two-span chunk); the first sw waves take the passes round
// robin, each streaming its chunks through its own ring across the workgroup's items.
//
// Routed mode: waves 0..7 route the tokens (one wave per token, its logits staged in the ring) while
// waves 8..15 quantize x into LDS; after one workgroup barrier every wave finds, from the tokens'
// selection bitmaps, the expert of each group it streams (groups ascending by expert id; the g-th
// set bit of the union of the bitmaps) and that group's entries (tokens ascending), so the weight
// loads go out with no further barrier. The last workgroup (which holds the fewest blocks) then
// writes the plan and the descriptor.
//
// Layer mode: the grid is at most one workgroup per CU and every workgroup is resident. After its
// blocks, a workgroup's q8_1 rows of h are in memory (device-scope stores) and it adds one to a
// count; its down chunks (the rows of its down tiles, taken from the last tile backwards so the
// workgroups without a block take the extra tiles) go out at once; it waits until the count reaches
// the grid (bounded), reads every entry's q8_1 rows of h and runs the down tiles and the scatter as
// the down launch does. The last workgroup to finish clears the counts for the next call.
// The first loads of the launch need only the logits, the NL4 table, x, the gate and up pointer
// arrays, T, E and n_embd: they come as the leading scalar arguments (copies of the struct's
// fields), which the launch preloads into scalar registers, so those loads go out before any read
// of the argument struct.
// ONE: the routed launch of a one-token window over at most 128 experts with n_embd <= 4096,
// compiled on its own: the ranked routing alone, x in two register passes, one-entry dot passes
// (the per-token routing, the other x stagings and the passes over several entries would only add
// code the launch never runs, and that code measurably slows it).
template <int FMT, int MODE, int FD = FMT, bool RW = false, bool ONE = false>
__global__ __launch_bounds__(kGuThreads) void k_gate_up(const float* __restrict__ logits0,
                                                        const int8_t* __restrict__ nl4_0,
                                                        const float* __restrict__ x0,
                                                        const void* const* __restrict__ gate0,
                                                        const void* const* __restrict__ up0, int T0,
                                                        int E0, int n_embd0, GuArgs a_) {
  constexpr bool RT = MODE == GU_ROUTED || MODE == GU_LAYER;
  extern __shared__ __align__(16) uint8_t smem[];
  // the wave index in a scalar register: everything derived from it is uniform over the wave
  const int tid = threadIdx.x, wave = uni(tid >> 6), lane = tid & 63;
  MOE_LDS uint8_t* ring = (MOE_LDS uint8_t*)smem;
  // ---- 1. every load that depends on nothing, at once. Routed: the routing waves (the first
  //         kRtWaves) send the NL4 table and their first logits rows before anything else (from
  //         the preloaded leading arguments) and load nothing more until they have routed (their
  //         wait then covers those alone); the other waves take the tables, the expert pointers
  //         and the destinations.
  const bool rw = RT && wave < kRtWaves;   // a routing wave
  MOE_LDS uint32_t* rscr = (MOE_LDS uint32_t*)ring + wave * route_scr_words(E0);
  // routed: the routing waves rank every token's experts together when the window is small
  // enough (then all waves meet once the logits rows are in LDS); else one wave per token
  static_assert(!ONE || MODE == GU_ROUTED, "the one-token launch is a routed one");
  const int rparts = ONE ? 4 : MODE == GU_ROUTED ? route_parts(T0, E0, 64 * kRtWaves) : 0;
  uint32_t t_nl4[4] = {0u, 0u, 0u, 0u};
  if constexpr (RT) {
    if (rw) {
      // the launch waits on the routing: a wave routing a token alone goes first on its SIMD (the
      // ranking of a small window shares the work with the x staging, which the launch waits on too)
      if (rparts == 0) __builtin_amdgcn_s_setprio(2);
      // the table (hot in L2) goes out just ahead of the logits, so the routing wave's one wait on
      // the logits covers it and nothing is loaded after the routing
      load_nl4(nl4_0, t_nl4);
      if (wave < T0) issue_logits(logits0 + (size_t)wave * E0, E0, (MOE_LDS float*)rscr);
    }
  }
  // routed, the other waves: x's rows (when they fit two register passes) and the gate and up
  // pointers of their experts, also from the preloaded arguments
  const int U0 = n_embd0 >> 5;
  const bool early_x = RT && (ONE || T0 * U0 * 8 <= 2 * kGuQThreads);
  float4 xr0[2];
  uint64_t pg = 0, pu = 0, pd = 0;   // routed: expert q0's pointers (experts past kGuQThreads later)
  if constexpr (RT) {
    if (!rw) {
      const int q = tid - 64 * kRtWaves;
      if (early_x) act_issue_f<kGuQThreads, 2>(x0, T0 * U0, q, xr0);
      if (q < E0) {
        pg = (uint64_t)(uintptr_t)gate0[q];
        pu = (uint64_t)(uintptr_t)up0[q];
      }
    }
  }
  (void)a_;
  const GuArgs a = args_after<GuArgs>(kGuArgsOff);
  const Geom& G = a.G;
  const uint64_t lt = (1ull << lane) - 1ull;
  const ActSplit act = act_layout(ring + a.lds_ring, a.n_tokens, G.U);
  MOE_LDS uint8_t* p8 = ring + a.lds_ring + a.lds_act;
  MOE_LDS uint32_t* g2 = (MOE_LDS uint32_t*)p8;
  MOE_LDS uint32_t* g3 = g2 + 512;
  const PlanL pl = plan_l((MOE_LDS int*)(p8 + 4096));
  MOE_LDS uint64_t* gptr = (MOE_LDS uint64_t*)(p8 + 4096 + kPlanLBytes);   // [group][gate, up, down]
  MOE_LDS float* stage = (MOE_LDS float*)(p8 + 4096 + kPlanLBytes + 8 * 3 * kMaxGrp);   // [entry][64]
  MOE_LDS uint8_t* tail = p8 + kGuFixed;
  MOE_LDS u64x2* ptab = (MOE_LDS u64x2*)tail;                        // routed: [E] gate, up
  MOE_LDS uint64_t* ptabd = (MOE_LDS uint64_t*)(tail + 16 * a.E);    // routed: [E] down
  const int nW = (a.E + 31) >> 5;
  MOE_LDS uint32_t* selT = (MOE_LDS uint32_t*)(tail + 24 * a.E);     // routed: [T][nW]

  const int q0 = RT ? tid - 64 * kRtWaves : tid;   // thread index among the waves that load tables
  if (!rw) load_nl4(nl4_0, t_nl4);
  uint32_t t_cb = 0;
  if constexpr (FMT == CB2 || FMT == CB3) {
    const uint32_t* src = (const uint32_t*)(FMT == CB2 ? a.A.cb2 : a.A.cb3);
    if (q0 >= 0 && q0 < 512) t_cb = src[q0];
  }
  uint32_t t_cbd = 0;   // layer mode: the down format's grid, when it differs
  if constexpr (MODE == GU_LAYER && FD != FMT && (FD == CB2 || FD == CB3)) {
    const uint32_t* src = (const uint32_t*)(FD == CB2 ? a.A.cb2 : a.A.cb3);
    if (q0 >= 0 && q0 < 512) t_cbd = src[q0];
  }
  int r_dt = 0, r_gs = 0, r_ge = 0, r_ng = 0;
  uint32_t r_ep = 0;
  // the destinations and the down pointers serve only the workgroup that writes the plan and the
  // descriptor (and layer mode, where every workgroup runs down tiles)
  const bool writer = MODE == GU_LAYER || blockIdx.x == gridDim.x - 1;
  if constexpr (RT) {
    if (q0 >= 0 && q0 < a.T) r_dt = a.dst_of_token ? a.dst_of_token[q0] : q0;
    if (MODE == GU_LAYER && q0 == 0)   // the last call's tag (this call's is one more)
      r_ep = __hip_atomic_load(a.ctr + kCtrEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (writer && q0 >= 0 && q0 < a.E) pd = (uint64_t)(uintptr_t)a.A.down[q0];
  } else {
    if (tid == 0) r_ng = *a.P.n_groups;
    if (tid <= a.P.cap_groups) r_gs = a.P.grp_start[tid];
    if (tid < a.P.cap_groups) r_ge = a.P.grp_expert[tid];
  }

  // ---- 2. routing and the activations' q8_1 blocks
  if constexpr (RT) {
    if (rw && rparts > 0) {
      __builtin_amdgcn_s_waitcnt(MOE_VM(0));   // this wave's logits row (and the NL4 table)
      if (wave < a.T) {   // its row from E to the power of two the ranking reads: -inf
        const int Ep = max(64, pow2ceil(a.E));
        for (int j = a.E + lane; j < Ep; j += 64) ((MOE_LDS float*)rscr)[j] = -__builtin_huge_valf();
      }
      lds_barrier();                           // every token's row is in LDS
      // ranks and selections; the last workgroup turns the chosen logits into weights later
      route_ranked(tid, a.T, a.E, a.k, rparts,
                   [&](int t) { return (const MOE_LDS float*)((MOE_LDS uint32_t*)ring + t * route_scr_words(a.E)); },
                   pl.rid, pl.rw, selT);
      __builtin_amdgcn_s_setprio(0);
    } else if (rw) {
      for (int t = wave; t < a.T; t += kRtWaves) {
        if (t != wave) issue_logits(a.logits + (size_t)t * a.E, a.E, (MOE_LDS float*)rscr);
        __builtin_amdgcn_s_waitcnt(MOE_VM(0));
        // routed: only the last workgroup writes the plan, so only it needs the router weights
        route_token(rscr, a.E, a.k, pl.rid + t * a.k, pl.rw + t * a.k, selT + t * nW,
                    MODE == GU_LAYER || blockIdx.x == gridDim.x - 1);
      }
      __builtin_amdgcn_s_setprio(0);
    } else {
      // two register passes cover one 4096-wide row; eight cover four (more: plain loads after)
      const int q = tid - 64 * kRtWaves, nblk = a.n_tokens * G.U;
      // (with the routing waves' ranking, every wave meets them once the logits are in LDS, while
      // the x loads are in flight)
      auto none = [&](int) {
        if (rparts > 0) lds_barrier();
      };
      if (early_x) {   // (the loads went out at the start)
        none(2);
        act_store_f<kGuQThreads, 2>(xr0, nblk, q, act);
      } else if (nblk * 8 <= 2 * kGuQThreads) {
        act_stage_f_np<kGuQThreads, 2>(a.x, nblk, q, act, none);
      } else {
        const int nreg = min(nblk, kGuQThreads * kGuXPass / 8);
        act_stage_f_np<kGuQThreads, kGuXPass>(a.x, nreg, q, act, none);
        if (nblk > nreg) act_rest_f<kGuQThreads>(a.x, nreg, nblk, q, act);
      }
    }
    if (q0 >= 0 && q0 < a.E) {
      const bool ok = ptr_ok(pg | pu, a.P.err);
      ptab[q0] = u64x2{ok ? pg : 0ull, ok ? pu : 0ull};
      if (writer) ptabd[q0] = ptr_ok(pd, a.P.err) ? pd : 0ull;
    }
    for (int e = q0 + kGuQThreads; q0 >= 0 && e < a.E; e += kGuQThreads) {
      const uint64_t g = (uint64_t)(uintptr_t)a.A.gate[e], u = (uint64_t)(uintptr_t)a.A.up[e];
      const bool ok = ptr_ok(g | u, a.P.err);
      ptab[e] = u64x2{ok ? g : 0ull, ok ? u : 0ull};
      if (writer) {
        const uint64_t d = (uint64_t)(uintptr_t)a.A.down[e];
        ptabd[e] = ptr_ok(d, a.P.err) ? d : 0ull;
      }
    }
    if (q0 >= 0 && q0 < a.T) pl.dtok[q0] = r_dt;
    if (MODE == GU_LAYER && q0 == 0) pl.misc[12] = (int)r_ep;
  } else if constexpr (MODE == GU_COMPOSED) {
    act_stage_q<kGuThreads, kGuXPass>(a.xq, a.n_tokens * G.U, act, [](int) {});
  } else {
    // float activation rows staged in the ring (free until the stream starts), then quantized
    MOE_LDS uint8_t* xs = ring;
    const int row_bytes = a.A.n_embd * 4;
    const int rows_per = max(1, a.lds_ring / row_bytes);
    const int nf4row = G.U * 8;
    for (int r0 = 0; r0 < a.n_tokens; r0 += rows_per) {
      const int nr = min(rows_per, a.n_tokens - r0);
      if (r0) __syncthreads();
      dma_span((const uint8_t*)(a.x + (size_t)r0 * a.A.n_embd), (uint32_t)(nr * row_bytes), xs, wave, kGuWaves);
      __syncthreads();   // (waits for every load issued so far, the staged rows included)
      const int nf4 = nr * nf4row;
      const MOE_LDS f32x4* xv = (const MOE_LDS f32x4*)xs;
      MOE_LDS uint32_t* lo32 = (MOE_LDS uint32_t*)act.lo;
      MOE_LDS uint32_t* hi32 = (MOE_LDS uint32_t*)act.hi;
      // trips are uniform per wave: the DPP max needs every lane of the wave
      for (int base = 0; base < nf4; base += kGuThreads) {
        const int f = base + tid;
        const f32x4 v = f < nf4 ? xv[f] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        float m = fmaxf(fmaxf(__builtin_fabsf(v.x), __builtin_fabsf(v.y)),
                        fmaxf(__builtin_fabsf(v.z), __builtin_fabsf(v.w)));
        m = fmaxf(m, dpp<0xB1>(m));    // xor 1
        m = fmaxf(m, dpp<0x4E>(m));    // xor 2
        m = fmaxf(m, dpp<0x141>(m));   // the other quad of the 8 lanes of a block
        if (f < nf4) {
          const int bk = r0 * G.U + (f >> 3), part = f & 7;
          const QScale qs = q_scale(m);
          uint32_t packed = 0;
          if (m != 0.0f) {
            const float xs4[4] = {v.x, v.y, v.z, v.w};
            packed = quant_pack4(xs4, qs);
          }
          if (part < 4)
            lo32[bk * 4 + part] = packed;
          else
            hi32[bk * 4 + part - 4] = packed;
          if (part == 0) act.d[bk] = h2f(f2h(qs.d));
        }
      }
    }
  }
  if constexpr (FMT == CB2 || FMT == CB3)
    if (q0 >= 0 && q0 < 512) (FMT == CB2 ? g2 : g3)[q0] = t_cb;
  if constexpr (MODE == GU_LAYER && FD != FMT && (FD == CB2 || FD == CB3))
    if (q0 >= 0 && q0 < 512) (FD == CB2 ? g2 : g3)[q0] = t_cbd;
  if constexpr (!RT) {
    if (tid == 0) pl.misc[3] = r_ng;
    if (tid <= a.P.cap_groups) pl.gstart[tid] = r_gs;
    if (tid < a.P.cap_groups) pl.gexp[tid] = r_ge;
  }
  Tables tb;
  tables_init(tb, t_nl4, g2, g3);
  __syncthreads();

  // ---- 3. the plan: the routed selections (every wave reads them itself), or the caller's,
  //         validated
  // routed: lane l < nW holds word l of the union of the tokens' selections, the groups and the
  // entries of the words below it
  uint32_t uw = 0u;
  int upc = 0, upre = 0, cpre = 0;
  int ng = 0, e0 = 0, n = 0;
  if constexpr (RT) {
    if (ONE || a.T == 1) {   // one token: the union is its selection, each group holds one entry
      if (lane < nW) uw = selT[lane];
      upc = __popc(uw);
      upre = lane_prefix(upc, 6);
      cpre = upre;
    } else {
      int ucnt = 0;
      if (lane < nW)
        for (int t = 0; t < a.T; ++t) {
          const uint32_t bw = selT[t * nW + lane];
          uw |= bw;
          ucnt += __popc(bw);
        }
      upc = __popc(uw);
      upre = lane_prefix(upc, 6);
      cpre = lane_prefix(ucnt, 7);   // at most 64 entries in all
    }
    ng = __builtin_amdgcn_readlane(upre + upc, 63);
    e0 = a.entry_base;
    n = a.T * a.k;
  } else {
    validate_groups(pl.gstart, pl.misc[3], a.P, pl.misc);
    __syncthreads();
    const int vng = uni(pl.misc[0]), ve0 = uni(pl.misc[1]), vn = uni(pl.misc[2]) - ve0;
    int r_src = 0, r_dst = 0;
    float r_w = 0.0f;
    uint64_t vg = 0, vu = 0, vd = 0;
    int e = -1;
    if (tid < vn) {
      r_src = a.P.ent_src[ve0 + tid];
      r_dst = a.P.ent_dst[ve0 + tid];
      r_w = a.P.ent_w[ve0 + tid];
    }
    if (tid < vng) {
      e = pl.gexp[tid];
      if (e >= 0 && e < a.A.n_experts) {
        vg = (uint64_t)(uintptr_t)a.A.gate[e];
        vu = (uint64_t)(uintptr_t)a.A.up[e];
        if (MODE == GU_FUSED) vd = (uint64_t)(uintptr_t)a.A.down[e];
      }
    }
    if (tid < vn) {
      const bool src_ok = r_src >= 0 && r_src < a.n_tokens;
      if (!src_ok) set_err(a.P.err, MOE_ERR_SRC);
      pl.esrc[tid] = src_ok ? r_src : 0;
      pl.edst[tid] = r_dst;
      pl.ew[tid] = r_w;
      pl.elive[tid] = src_ok;
    }
    if (tid < vng) {
      const bool e_ok = e >= 0 && e < a.A.n_experts;
      if (!e_ok) set_err(a.P.err, MOE_ERR_EXPERT);
      gptr[3 * tid] = (e_ok && ptr_ok(vg | vu, a.P.err)) ? vg : 0;
      gptr[3 * tid + 1] = vu;
      gptr[3 * tid + 2] = (e_ok && MODE == GU_FUSED && ptr_ok(vd, a.P.err)) ? vd : 0;
    }
    __syncthreads();
    ng = vng;
    e0 = ve0;
    n = vn;
  }
  // routed: the g-th group's expert (word l, bit b of the union) ...
  auto find_expert = [&](int g, int& l, int& b) {
    const uint64_t hit = __ballot(lane < nW && upre + upc > g);
    l = (int)__builtin_ctzll(hit);
    const uint32_t wv = (uint32_t)__builtin_amdgcn_readlane((int)uw, l);
    const int r = g - __builtin_amdgcn_readlane(upre, l);
    const uint32_t below = lane < 32 ? ((1u << (lane & 31)) - 1u) : 0u;
    const uint64_t bm = __ballot(lane < 32 && ((wv >> (lane & 31)) & 1u) && __popc(wv & below) == r);
    b = (int)__builtin_ctzll(bm);
  };
  // ... and its entries: the tokens that chose it (bit t of tm), first entry a0 (relative to e0)
  auto entries_of = [&](int l, int b, int& a0, int& cnt, uint64_t& tm) {
    const uint32_t mine = lane < a.T ? selT[lane * nW + l] : 0u;
    tm = __ballot((mine >> b) & 1u);
    cnt = __popcll(tm);
    a0 = __builtin_amdgcn_readlane(cpre, l) + lane_sum(__popc(mine & ((1u << b) - 1u)), 6);
  };
  // the gate and up pointers of group g (0 when the group is skipped)
  auto group_ptrs = [&](int g, uint64_t& wg, uint64_t& wu) {
    wg = 0;
    wu = 0;
    if (g >= ng) return;
    if constexpr (RT) {
      int l, b;
      find_expert(g, l, b);
      const u64x2 pp = ptab[32 * l + b];
      wg = uni64(pp.x);
      wu = uni64(pp.y);
    } else {
      wg = uni64(gptr[3 * g]);
      wu = uni64(gptr[3 * g + 1]);
    }
  };

  // ---- 4. items: the workgroup's blocks; this wave's passes of each, streamed through its ring
  const int half = G.rp >> 1;
  const int nb = a.A.n_ff / 32;          // blocks per group
  const int npass = 64 / G.rp;           // passes per block
  const int items = ng * nb;
  const int bid = (int)blockIdx.x, grid = (int)gridDim.x;
  // (the usual shapes need no division: at most one item per workgroup, one pass per wave)
  const int nit = bid >= items ? 0 : items <= grid ? 1 : (items - bid + grid - 1) / grid;
  const int cw = wave >= min(a.sw, npass) ? 0 : npass <= a.sw ? 1 : (npass - wave + a.sw - 1) / a.sw;
  const int nch = nit * cw;
  const int M = a.S.M, NS = a.S.NS;
  MOE_LDS uint8_t* myring = ring + wave * NS * M * 1024;
  const uint32_t nspan = (uint32_t)(half * G.rb);
  // a chunk's place: pass q of item kk, the item's group g and block blk (item bid + kk * grid),
  // stepped forward one chunk at a time (no division per chunk)
  struct Pos {
    int q, g, blk;
  };
  auto div_nb = [&](int x) {   // x / nb from the host's reciprocal, one correction step
    int q = (int)__umulhi((uint32_t)x, a.nb_magic);
    if ((q + 1) * nb <= x) ++q;
    return q;
  };
  const int gstep = div_nb(grid), bstep = grid - gstep * nb;
  const int g0 = div_nb(bid);
  const Pos first{0, g0, bid - g0 * nb};
  auto next_item = [&](Pos& p) {
    p.q = 0;
    p.g += gstep;
    p.blk += bstep;
    if (p.blk >= nb) {
      p.blk -= nb;
      ++p.g;
    }
  };
  auto step = [&](Pos& p) {
    if (++p.q >= cw) next_item(p);
  };
  Pos ip = first;   // the next chunk to issue
  auto issue = [&](MOE_LDS uint8_t* slot) {
    const int q = ip.q, g = ip.g, blk = ip.blk;
    step(ip);
    uint64_t wg, wu;
    group_ptrs(g, wg, wu);
    if (wg) {   // the gate rows in the slot's first half, the up rows in its second
      const uint64_t off = (uint64_t)(blk * 32 + (wave + q * a.sw) * half) * (uint64_t)G.rb;
      issue_span(slot, M / 2, (const uint8_t*)(uintptr_t)(wg + off), nspan);
      issue_span(slot + (M / 2) * 1024, M / 2, (const uint8_t*)(uintptr_t)(wu + off), nspan);
    } else {   // a skipped group keeps the count of loads: one 16-byte piece every lane reloads
      issue_span(slot, M, (const uint8_t*)a.P.grp_start, 1);
    }
  };
  // register-direct (planar NL4): this lane's units of the chunk's rows straight into registers
  constexpr bool regw = RW;
  // planar NL4 rows of a 16-byte multiple: a pass whose spans land 16-byte aligned takes the
  // aligned reads
  const bool pa_rows = FMT == NL4 && G.ly.c_a == 16u && G.ly.c_b == 0u && (G.rb & 15) == 0;
  RegW rwt;
  // the scale planes' lanes: lane j < rp U / 8 takes piece sj of the wave's row sri
  const int s16 = G.U >> 3, sri = lane / max(s16, 1), sj = lane - sri * s16;
  auto issue_reg = [&]() {
    const int q = ip.q, g = ip.g, blk = ip.blk;
    step(ip);
    uint64_t wg, wu;
    group_ptrs(g, wg, wu);
    const int i = lane >> G.lgL;
    if (wg) {
      const int r0 = blk * 32 + (wave + q * a.sw) * half;
      auto row_of = [&](int ii) {
        return (const uint8_t*)(uintptr_t)((ii < half ? wg : wu) +
                                           (uint64_t)(r0 + (ii < half ? ii : ii - half)) * (uint64_t)G.rb);
      };
      reg_issue(rwt, row_of(i < G.rp ? i : 0), row_of(sri < G.rp ? sri : 0), sj, myring, G, lane & (G.L - 1));
    }
  };
  __builtin_amdgcn_s_waitcnt(MOE_VM(0));   // nothing of ours in flight before the stream
  const int pre = regw ? 0 : min(NS, nch);
  // the first chunks go out ahead of the dots of waves whose chunks have already landed: a wave
  // issuing competes for its SIMD only with those, and its loads are what the stream waits on
  __builtin_amdgcn_s_setprio(3);
  if (regw) {
    if (nch > 0) issue_reg();
  } else {
    for (int kc = 0; kc < pre; ++kc) issue(myring + kc * M * 1024);
  }
  __builtin_amdgcn_s_setprio(0);
  int issued = pre;

  // ---- 5. the last workgroup (the fewest blocks: they are dealt in workgroup order) leaves the
  //         plan (routed) and the call's descriptor (fused / routed)
  if (MODE != GU_COMPOSED && blockIdx.x == gridDim.x - 1) {
    int* dw = (int*)a.desc;
    uint64_t* dp = (uint64_t*)(a.desc + kDescPtrByte);
    if constexpr (RT) {
      if (rparts > 0) {   // the ranking left each token's chosen logits: the router weights
        if (wave < a.T) {
          const int t = wave;
          const float l0 = pl.rw[t * a.k];
          float ex = 0.0f;
          if (lane < a.k) ex = expf(pl.rw[t * a.k + lane] - l0);
          float sum = 0.0f;
          for (int j = 0; j < a.k; ++j) sum = sum + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
          if (lane < a.k) pl.rw[t * a.k + lane] = ex / sum;
        }
        lds_barrier();
      }
      for (int g = wave; g < ng; g += kGuWaves) {
        int l, b, a0, cnt;
        uint64_t tm;
        find_expert(g, l, b);
        entries_of(l, b, a0, cnt, tm);
        const int e = 32 * l + b;
        const bool ok = uni64(ptab[e].x) != 0;
        if (lane == 0) {
          a.P.grp_expert[g] = e;
          a.P.grp_start[g] = e0 + a0;
          dw[kDescGs + g] = a0;
          dp[g] = ok ? ptabd[e] : 0ull;
        }
        if ((tm >> lane) & 1ull) {   // lane = token
          const int ent = a0 + __popcll(tm & lt);
          int r = 0;
          while (r < a.k - 1 && pl.rid[lane * a.k + r] != e) ++r;
          const float wv = pl.rw[lane * a.k + r];
          const int dst = pl.dtok[lane];
          a.P.ent_src[e0 + ent] = lane;
          a.P.ent_dst[e0 + ent] = dst;
          a.P.ent_w[e0 + ent] = wv;
          dw[kDescDst + ent] = dst;
          ((float*)dw)[kDescW + ent] = wv;
          dw[kDescLive + ent] = ok ? 1 : 0;
        }
      }
      if (tid == 0) {
        *a.P.n_groups = ng;
        a.P.grp_start[ng] = e0 + n;
        dw[kDescGs + ng] = n;
      }
    } else {
      if (tid <= ng) dw[kDescGs + tid] = pl.gstart[tid] - e0;
      if (tid < ng) dp[tid] = gptr[3 * tid] ? gptr[3 * tid + 2] : 0;
      if (tid < n) {
        int g = 0;
        while (g + 1 < ng && pl.gstart[g + 1] - e0 <= tid) ++g;
        dw[kDescDst + tid] = pl.edst[tid];
        ((float*)dw)[kDescW + tid] = pl.ew[tid];
        dw[kDescLive + tid] = pl.elive[tid] && gptr[3 * g] != 0;
      }
    }
    if (tid == 0) {
      dw[kDescNg] = ng;
      dw[kDescE0] = e0;
      dw[kDescN] = n;
    }
  }

  int kc = 0;
  Pos cp = first;   // the item being computed
  for (int kk = 0; kk < nit; ++kk) {
    const int g = cp.g, blk = cp.blk;
    next_item(cp);
    uint64_t wgv, wuv;
    group_ptrs(g, wgv, wuv);
    int a0 = 0, ne = 0;
    uint64_t tm = 0;
    if constexpr (RT) {
      int l, b;
      find_expert(g, l, b);
      entries_of(l, b, a0, ne, tm);
    } else {
      a0 = uni(pl.gstart[g]) - e0;
      ne = uni(pl.gstart[g + 1]) - e0 - a0;
    }
    for (int q = 0; q < cw; ++q, ++kc) {
      if (regw) {
        if (kc > 0) issue_reg();   // one chunk at a time (the registers hold one)
      } else {
        wait_vm((issued - 1 - kc) * M);
      }
      MOE_LDS uint8_t* slot = myring + slot_of(kc, NS) * M * 1024;
      if (wgv && regw && ONE) {   // a one-token window: the group's one entry (the token), one pass
        const int prow = (wave + q * a.sw) * half;
        const int sidx[kSlots] = {};
        MOE_LDS float* st = stage + prow;
        wait_vm(G.upl);   // the scale planes (issued before this lane's code loads)
        auto outr = [&](int i, int e, float v) { st[e * 64 + (i < half ? i : 32 + i - half)] = v; };
        dot_pass_reg_n<1>(rwt, (const MOE_LDS uint16_t*)myring, G.rp, G, tb, act, sidx, outr);
      } else if (wgv && regw) {
        const int prow = (wave + q * a.sw) * half;
        uint64_t rest = tm;
        for (int c0 = 0; c0 < ne; c0 += kRegSlots) {
          const int nc = min(kRegSlots, ne - c0);
          int sidx[kSlots];
#pragma unroll
          for (int e = 0; e < kSlots; ++e) {
            if constexpr (RT) {
              sidx[e] = 0;
              if (e < nc) {
                sidx[e] = (int)__builtin_ctzll(rest);
                rest &= rest - 1ull;
              }
            } else {
              sidx[e] = e < nc ? uni(pl.esrc[a0 + c0 + e]) : 0;
            }
          }
          MOE_LDS float* st = stage + c0 * 64 + prow;
          if (c0 == 0) wait_vm(G.upl);   // the scale planes (issued before this lane's code loads)
          auto outr = [&](int i, int e, float v) { st[e * 64 + (i < half ? i : 32 + i - half)] = v; };
          dot_pass_reg(rwt, (const MOE_LDS uint16_t*)myring, G.rp, G, tb, act, sidx, nc, outr);
        }
      } else if (wgv) {
        const int prow = (wave + q * a.sw) * half;   // first h row of the pass inside the block
        const uint64_t off = (uint64_t)(blk * 32 + prow) * (uint64_t)G.rb;
        const uint32_t sb = (uint32_t)(slot - ring);
        const uint32_t ra = sb + (uint32_t)((wgv + off) & 15);
        const uint32_t rb0 = sb + (M / 2) * 1024 + (uint32_t)((wuv + off) & 15);
        uint64_t rest = tm;   // routed: the group's tokens not yet dotted
        for (int c0 = 0; c0 < ne; c0 += kSlots) {
          const int nc = min(kSlots, ne - c0);
          int sidx[kSlots];
#pragma unroll
          for (int e = 0; e < kSlots; ++e) {
            if constexpr (RT) {
              sidx[e] = 0;
              if (e < nc) {
                sidx[e] = (int)__builtin_ctzll(rest);
                rest &= rest - 1ull;
              }
            } else {
              sidx[e] = e < nc ? uni(pl.esrc[a0 + c0 + e]) : 0;
            }
          }
          MOE_LDS float* st = stage + c0 * 64 + prow;
          auto outl = [&](int i, int e, float v) { st[e * 64 + (i < half ? i : 32 + i - half)] = v; };
          const bool pa = pa_rows && ((ra | rb0) & 15u) == 0;
          if constexpr (ONE && FMT == NL4) {
            if (pa)
              dot_pass_pa<1>((const MOE_LDS uint8_t*)ring, ra, rb0, half, G.rp, G, tb, act, sidx, outl);
            else
              dot_pass_n<FMT, 1>((const MOE_LDS uint32_t*)ring, ra, rb0, half, G.rp, G, tb, act, sidx, outl);
          } else if constexpr (ONE)
            dot_pass_n<FMT, 1>((const MOE_LDS uint32_t*)ring, ra, rb0, half, G.rp, G, tb, act, sidx, outl);
          else
            dot_pass<FMT>((const MOE_LDS uint32_t*)ring, ra, rb0, half, G.rp, G, tb, act, sidx, nc, outl, pa);
        }
      }
      if (!regw && kc + NS < nch) {
        MOE_WAIT_LGKM0;   // this wave's LDS reads of the slot have returned
        issue(slot);
        ++issued;
      }
    }
    lds_barrier();
    // the block's outputs: composed, g and u rows; fused / routed, SwiGLU + q8_1 of h
    if (wgv) {
      if constexpr (MODE == GU_COMPOSED) {
        for (int idx = tid; idx < ne * 64; idx += kGuThreads) {
          const int e = idx >> 6, r = idx & 63;
          if (!pl.elive[a0 + e]) continue;
          (r < 32 ? a.g : a.u)[(size_t)(e0 + a0 + e) * a.ld + blk * 32 + (r & 31)] = stage[idx];
        }
      } else {
        // (register-direct instances read the destinations again here rather than hold them in
        // scalar registers through the stream: measured faster there, slower in the others)
        const GuArgs ah = RW ? args_after<GuArgs>(kGuArgsOff) : a;
        // 32 lanes per entry; every half-wave runs each round (the shuffles need all 32 lanes)
        for (int base = 0; base < ne; base += kGuThreads / 32) {
          const int e = base + (tid >> 5), l32 = tid & 31;
          bool live = e < ne;
          if constexpr (!RT) live = live && pl.elive[a0 + (e < ne ? e : 0)] != 0;
          const float gv = live ? stage[e * 64 + l32] : 0.0f;
          const float uv = live ? stage[e * 64 + 32 + l32] : 0.0f;
          const size_t bk = (size_t)(a0 + (live ? e : 0)) * nb + blk;
          swiglu_q81_split<MODE == GU_LAYER>(gv, uv, l32, live, ah.hq_lo + 4 * bk, ah.hq_hi + 4 * bk, ah.hq_d + bk,
                                              ah.hq_s ? ah.hq_s + bk : nullptr);
        }
      }
    }
    lds_barrier();
  }

  // ---- 7. layer mode: the grouped down projection and the weighted scatter
  if constexpr (MODE == GU_LAYER) {
    const Geom& Gd = a.Gd;
    const int Ud = Gd.U;
    MOE_LDS uint8_t* dreg = tail + a.lds_tail;
    const ActSplit actd = act_layout_kb(dreg, a.P.cap_entries, Ud, FD == Q5_1);
    const int tr = a.trd;
    MOE_LDS float* ores = (MOE_LDS float*)(dreg + act_bytes_kb(a.P.cap_entries, Ud, FD == Q5_1));   // [kMaxEnt][tr]
    MOE_LDS int* mdst = (MOE_LDS int*)(ores + kMaxEnt * kDnTileMax);   // [kMaxEnt] dst or -1
    MOE_LDS int* mown = mdst + kMaxEnt;                           // first live entry of its dst
    MOE_LDS float* mw = (MOE_LDS float*)(mown + kMaxEnt);
    MOE_LDS int* omap = (MOE_LDS int*)(mw + kMaxEnt);             // owner index of an owner entry
    MOE_LDS int* ownl = omap + kMaxEnt;                           // owner entries in order
    MOE_LDS int* dmisc = ownl + kMaxEnt;                          // [16]
    MOE_LDS float* ybuf = (MOE_LDS float*)(dmisc + 16);           // [owner][tr] first tile's Y rows
    constexpr int kPollWave = kDnWaves;   // a wave that streams no down chunks
    const uint32_t tag = (uint32_t)uni(pl.misc[12]) + 1u;

    // (a) this workgroup's q8_1 rows of h have reached device scope: raise its flag
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    if (tid == 0) __hip_atomic_store(a.ctr + kCtrFlags + blockIdx.x, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // (b) the call in LDS: per group its first entry and down pointer, per entry its destination,
    //     weight and whether it was computed
    for (int g = wave; g < ng; g += kGuWaves) {
      int l, b, a0, cnt;
      uint64_t tm;
      find_expert(g, l, b);
      entries_of(l, b, a0, cnt, tm);
      const int e = 32 * l + b;
      const bool ok = uni64(ptab[e].x) != 0;
      if (lane == 0) {
        pl.gstart[g] = a0;
        gptr[3 * g + 2] = ok ? ptabd[e] : 0ull;
      }
      if ((tm >> lane) & 1ull) {   // lane = token
        const int ent = a0 + __popcll(tm & lt);
        int r = 0;
        while (r < a.k - 1 && pl.rid[lane * a.k + r] != e) ++r;
        pl.edst[ent] = pl.dtok[lane];
        pl.ew[ent] = pl.rw[lane * a.k + r];
        pl.elive[ent] = ok ? 1 : 0;
      }
    }
    if (tid == 0) pl.gstart[ng] = n;
    lds_barrier();

    // (c) this workgroup's down tiles (tile t goes to workgroup grid - 1 - t % grid, so the
    //     workgroups without a block take the extra tiles); waves 0..kDnWaves-1 take the groups
    //     g = w, w + kDnWaves, ...; their first chunks go out now, into the ring
    const int ntiles = (a.A.n_embd + tr - 1) / tr;
    const int rev = (int)gridDim.x - 1 - (int)blockIdx.x;
    const int ntw = rev < ntiles ? (ntiles - rev + (int)gridDim.x - 1) / (int)gridDim.x : 0;
    // per tile its groups g = wave + q kDnWaves, per group the tile's rows in nsub chunks of rc rows
    const int rc = a.rcd, nsub = (tr + rc - 1) / rc;
    const int qpt = (wave < kDnWaves && wave < ng) ? (ng - wave + kDnWaves - 1) / kDnWaves : 0;
    const int nchd = ntw * qpt * nsub;
    auto chunk_rows = [&](int t, int sub, int& r0, int& nr) {
      const int te = min(t * tr + tr, a.A.n_embd);
      r0 = t * tr + sub * rc;
      nr = min(rc, te - r0);
    };
    const int Md = a.Sd.M, NSd = a.Sd.NS;
    MOE_LDS uint8_t* dring = ring + (wave < kDnWaves ? wave : 0) * NSd * Md * 1024;
    struct Pos {
      int t, q, s;
    };
    Pos ip{rev, 0, 0};   // the next chunk to issue, stepped one chunk at a time
    auto dissue = [&](MOE_LDS uint8_t* slot) {
      const Pos p = ip;
      if (++ip.s == nsub) {
        ip.s = 0;
        if (++ip.q == qpt) {
          ip.q = 0;
          ip.t += (int)gridDim.x;
        }
      }
      const int g = wave + p.q * kDnWaves;
      int r0, nr;
      chunk_rows(p.t, p.s, r0, nr);
      const uint64_t w = uni64(gptr[3 * g + 2]);
      if (w && nr > 0)
        issue_span(slot, Md, (const uint8_t*)(uintptr_t)(w + (uint64_t)r0 * Gd.rb), (uint32_t)(nr * Gd.rb));
      else   // a skipped group (or rows past the end) keeps the count of loads
        issue_span(slot, Md, (const uint8_t*)a.P.err, 1);
    };
    // a workgroup that had blocks sends its first chunks only once the count is complete: its
    // polls go through the same memory queue and would wait behind them; one without blocks has
    // the whole gate/up phase to spare and sends them now
    const bool early = true;
    const int pred = min(NSd, nchd);
    if (early)
      for (int kc = 0; kc < pred; ++kc) dissue(dring + kc * Md * 1024);
    int dissued = pred;

    // (d) entries' destinations and owners (the first live entry naming a destination sums it)
    if (tid < n) {
      int g = 0;
      while (g + 1 < ng && pl.gstart[g + 1] <= tid) ++g;
      const int d = pl.edst[tid];
      int live = pl.elive[tid] && gptr[3 * g + 2] != 0;
      if (live && (d < 0 || d >= a.n_rows)) {
        set_err(a.P.err, MOE_ERR_DST);
        live = 0;
      }
      mdst[tid] = live ? d : -1;
      mw[tid] = pl.ew[tid];
    }
    lds_barrier();
    if (wave == 0) {   // n <= 64: one lane per entry
      int owner = 0;
      if (lane < n) {
        const int d = mdst[lane];
        owner = d >= 0;
        for (int q = 0; q < lane && owner; ++q) owner = mdst[q] != d;
        mown[lane] = owner;
      }
      const uint64_t om = __ballot(owner);
      if (owner) {
        const int o = __popcll(om & lt);
        omap[lane] = o;
        ownl[o] = lane;
      }
      if (lane == 0) dmisc[8] = __popcll(om);
    }

    // (e) every workgroup's q8_1 rows of h are in memory once every flag holds this call's tag (a
    //     wave with no down chunks in flight reads them all, a few per lane; the wait is bounded)
    if (wave == kPollWave) {
      int it = 0;
      bool all = false;
      do {
        int seen = 0, want = 0;
        for (int i = lane; i < (int)gridDim.x; i += 64, ++want)
          seen += __hip_atomic_load(a.ctr + kCtrFlags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag;
        all = __ballot(seen != want) == 0ull;
        if (all) break;
        __builtin_amdgcn_s_sleep(1);
      } while (++it < a.spin_limit);
      if (lane == 0) {
        dmisc[9] = all;
        if (!all) set_err(a.P.err, MOE_ERR_WAIT);
      }
    }
    lds_barrier();
    const bool go = uni(dmisc[9]) != 0;
    const int nown = uni(dmisc[8]);
    if (!early && go)
      for (int kc = 0; kc < pred; ++kc) dissue(dring + kc * Md * 1024);

    // (f) the waves with no down chunks read every entry's q8_1 rows of h (device scope) and the
    //     first tile's destination rows of Y into LDS
    const int r00 = rev * tr, nr0 = min(tr, a.A.n_embd - r00);
    if (go && wave >= kDnWaves) {
      const int dw = wave - kDnWaves, ndw = kGuWaves - kDnWaves;
      const uint32_t qb = (uint32_t)(n * Ud * 16), db = (uint32_t)((n * Ud * 4 + 15) & ~15);
      dma_span<true>((const uint8_t*)a.hq_lo, qb, (MOE_LDS uint8_t*)actd.lo, dw, ndw);
      dma_span<true>((const uint8_t*)a.hq_hi, qb, (MOE_LDS uint8_t*)actd.hi, (dw + 3) % ndw, ndw);
      dma_span<true>((const uint8_t*)a.hq_d, db, (MOE_LDS uint8_t*)actd.d, (dw + 6) % ndw, ndw);
      if constexpr (FD == Q5_1)
        dma_span<true>((const uint8_t*)a.hq_s, db, (MOE_LDS uint8_t*)actd.s, (dw + 7) % ndw, ndw);
      if (ntw > 0 && wave == kDnWaves) {   // one float per lane
        for (int p = 0; p * 64 < nown * nr0; ++p) {
          const int l = p * 64 + lane;
          if (l < nown * nr0) {
            const int o = l / nr0, m = l - o * nr0;
            const float* src = a.Y + (size_t)mdst[ownl[o]] * a.ldy + r00 + m;
            __builtin_amdgcn_global_load_lds((const void*)src, (MOE_LDS void*)(ybuf + 64 * p), 4, 0, 0);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(MOE_VM(0));   // these waves stream no down chunks
    }
    lds_barrier();

    // (g) tiles: each down wave dots its groups' rows of the tile with the group's h rows; then
    //     every destination row is summed in ascending entry order and written once
    int kc = 0;
    for (int kt = 0; go && kt < ntw; ++kt) {
      const int t = rev + kt * (int)gridDim.x;
      const int r0 = t * tr, nr = min(tr, a.A.n_embd - r0);
      for (int q = 0, sb = 0; q < qpt; ++kc, sb = sb + 1 < nsub ? sb + 1 : 0, q += sb == 0) {
        const int g = wave + q * kDnWaves;
        wait_vm((dissued - 1 - kc) * Md);
        MOE_LDS uint8_t* slot = dring + slot_of(kc, NSd) * Md * 1024;
        const uint64_t w = uni64(gptr[3 * g + 2]);
        int c_r0, c_nr;
        chunk_rows(t, sb, c_r0, c_nr);
        if (w && c_nr > 0) {
          const uint32_t ra = (uint32_t)(slot - ring) + (uint32_t)((w + (uint64_t)c_r0 * Gd.rb) & 15);
          const int a0 = uni(pl.gstart[g]), a1 = uni(pl.gstart[g + 1]);
          const int o0 = c_r0 - r0;   // the chunk's first row inside the tile
          for (int p0 = 0; p0 < c_nr; p0 += Gd.rp) {   // the chunk's rows in wave passes
            const int np = min(Gd.rp, c_nr - p0);
            const uint32_t rp0 = ra + (uint32_t)(p0 * Gd.rb);
            for (int c0 = a0; c0 < a1; c0 += kSlots) {
              const int ne = min(kSlots, a1 - c0);
              int sidx[kSlots];
#pragma unroll
              for (int e = 0; e < kSlots; ++e) sidx[e] = e < ne ? c0 + e : 0;
              dot_pass<FD>((const MOE_LDS uint32_t*)ring, rp0, rp0, np, np, Gd, tb, actd, sidx, ne,
                           [&](int i, int e, float v) { ores[(c0 + e) * tr + o0 + p0 + i] = v; });
            }
          }
        }
        if (kc + NSd < nchd) {
          MOE_WAIT_LGKM0;
          dissue(slot);
          ++dissued;
        }
      }
      lds_barrier();
      for (int idx = tid; idx < n * nr; idx += kGuThreads) {
        const int i = idx / nr, m = idx - i * nr;
        if (!mown[i]) continue;
        const int d = mdst[i];
        float* y = a.Y + (size_t)d * a.ldy + r0 + m;
        float acc = kt == 0 ? ybuf[omap[i] * nr + m] : *y;
        *y = dst_sum(acc, i, n, d, m, tr, mdst, mw, ores);
      }
      lds_barrier();
    }
    // a workgroup that gave up waiting still drains the chunks it issued
    __builtin_amdgcn_s_waitcnt(MOE_VM(0));

    // (h) the last workgroup out records this call's tag and clears the done counts for the next
    //     call (every other workgroup has read the old tag and made its count by then)
    if (tid == 0 && count_in(a.ctr + kCtrDone, 0)) {
      __hip_atomic_store(a.ctr + kCtrEpoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int i = 0; i <= kCtrGroups; ++i)
        __hip_atomic_store(a.ctr + kCtrDone + i * (kCtrLine / 4), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ------------------------------------------------------------------ down + scatter kernel ---

enum DnMode : int { DN_DESC = 0, DN_PLAN = 1 };

struct DnArgs {
  LayerArgs A;
  PlanArgs P;
  Geom G;
  Stream S;
  const uint8_t* desc;  // DN_DESC: the call's descriptor
  const uint8_t* hq;    // DN_PLAN: q8_1 rows of h by absolute entry
  const uint8_t* hq_lo; // DN_DESC: the workspace's split q8_1 rows of h (entry - e0)
  const uint8_t* hq_hi;
  const uint8_t* hq_d;
  const uint8_t* hq_s;  // DN_DESC, Q5_1 only: the blocks' sum fields
  float* Y;
  int n_rows, ldy;
  int lds_ring, lds_act;
  int tr;               // rows of Y per tile (<= kDnTileMax)
  int rc;               // rows per streamed chunk (a tile's rows of one group: nsub chunks)
  int nsub;             // ceil(tr / rc)
  int ntiles;           // ceil(n_embd / tr)
};

constexpr int kDnYBuf = kMaxEnt * kDnTileMax;   // floats: the first tile's destination rows, per owner
constexpr int kDnFixed = 4096 + kDescBytes + 4 * 5 * kMaxEnt + 256 + 4 * kDnYBuf;

__host__ __device__ inline int dn_smem_bytes(int lds_ring, int lds_act) {
  return lds_ring + lds_act + kMaxEnt * kDnTileMax * 4 + kDnFixed;
}

// One work item: rows [tr t, tr t + tr) of Y (tr is chosen so that the tiles spread evenly over
// the CUs). Wave w takes the groups g = w, w + 8, ... in order; a chunk is a group's down rows of
// the tile, dotted in wave passes of rp rows. Per-entry rows of o stay in LDS; at the end
// every destination row is summed in ascending entry order: Y[d][r] = ((Y[d][r] + w_a o_a[r]) +
// w_b o_b[r]) + ...
// ONE: a one-token call (n_tokens == 1), compiled on its own with one-entry dot passes: a token's
// groups hold one entry each (a larger group, from a caller's plan, takes one pass per entry: the
// same sums), and the passes over several entries would only add code the launch never runs.
template <int FMT, int MODE, bool ONE = false>
__global__ __launch_bounds__(kDnThreads) void k_down(DnArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const Geom& G = a.G;
  const int tid = threadIdx.x, wave = uni(tid >> 6);   // a scalar register (uniform over the wave)
  MOE_LDS uint8_t* ring = (MOE_LDS uint8_t*)smem;
  const int U = G.U;
  MOE_LDS uint8_t* actp = ring + a.lds_ring;
  const int tr = a.tr;
  MOE_LDS float* ores = (MOE_LDS float*)(actp + a.lds_act);   // [kMaxEnt][tr]
  MOE_LDS uint32_t* g2 = (MOE_LDS uint32_t*)(ores + kMaxEnt * kDnTileMax);
  MOE_LDS uint32_t* g3 = g2 + 512;
  MOE_LDS int* dsc = (MOE_LDS int*)(g3 + 512);                 // the descriptor, as in memory
  MOE_LDS uint64_t* dptr = (MOE_LDS uint64_t*)((MOE_LDS uint8_t*)dsc + kDescPtrByte);
  MOE_LDS int* mdst = (MOE_LDS int*)((MOE_LDS uint8_t*)dsc + kDescBytes);   // [kMaxEnt] dst or -1
  MOE_LDS int* mown = mdst + kMaxEnt;                        // [kMaxEnt] first live entry of its dst
  MOE_LDS float* mw = (MOE_LDS float*)(mown + kMaxEnt);      // [kMaxEnt]
  MOE_LDS int* omap = (MOE_LDS int*)(mw + kMaxEnt);          // [kMaxEnt] owner index of an owner entry
  MOE_LDS int* ownl = omap + kMaxEnt;                        // [kMaxEnt] owner entries in order
  MOE_LDS int* misc = ownl + kMaxEnt;                        // [64]
  MOE_LDS float* ybuf = (MOE_LDS float*)(misc + 64);         // [owner][tr] first tile's Y rows

  // ---- 1. tables and the call (descriptor: one read; caller's plan: validated, two reads)
  warm_args<DnArgs>();
  uint32_t t_nl4[4];
  load_nl4(a.A.nl4, t_nl4);
  uint32_t t_cb = 0;
  if constexpr (FMT == CB2 || FMT == CB3) {
    const uint32_t* src = (const uint32_t*)(FMT == CB2 ? a.A.cb2 : a.A.cb3);
    t_cb = src[tid];
  }
  if constexpr (MODE == DN_DESC) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (tid < kDescBytes / 16) v = ((const u32x4*)a.desc)[tid];
    if (tid < kDescBytes / 16) ((MOE_LDS u32x4*)dsc)[tid] = v;
  } else {
    // raw group table: starts into the descriptor's start slots, experts into its dst slots
    int r_ng = 0, r_gs = 0, r_ge = 0;
    if (tid == 0) r_ng = *a.P.n_groups;
    if (tid <= a.P.cap_groups) r_gs = a.P.grp_start[tid];
    if (tid < a.P.cap_groups) r_ge = a.P.grp_expert[tid];
    if (tid == 0) misc[3] = r_ng;
    if (tid <= a.P.cap_groups) dsc[kDescGs + tid] = r_gs;
    if (tid < a.P.cap_groups) dsc[kDescDst + tid] = r_ge;
  }
  Tables tb;
  tables_init(tb, t_nl4, g2, g3);
  if constexpr (FMT == CB2 || FMT == CB3) (FMT == CB2 ? g2 : g3)[tid] = t_cb;
  __syncthreads();
  if constexpr (MODE == DN_PLAN) {
    validate_groups(dsc + kDescGs, misc[3], a.P, misc);
    __syncthreads();
    const int ng = uni(misc[0]), e0 = uni(misc[1]), n = uni(misc[2]) - e0;
    int r_dst = 0;
    float r_w = 0.0f;
    uint64_t vd = 0;
    int e = -1;
    if (tid < n) {
      r_dst = a.P.ent_dst[e0 + tid];
      r_w = a.P.ent_w[e0 + tid];
    }
    if (tid < ng) {
      e = dsc[kDescDst + tid];
      if (e >= 0 && e < a.A.n_experts) vd = (uint64_t)(uintptr_t)a.A.down[e];
    }
    int gs = 0;
    if (tid <= ng) gs = dsc[kDescGs + tid] - e0;
    __syncthreads();
    if (tid == 0) {
      dsc[kDescNg] = ng;
      dsc[kDescE0] = e0;
      dsc[kDescN] = n;
    }
    if (tid <= ng) dsc[kDescGs + tid] = gs;
    if (tid < ng) {
      const bool e_ok = e >= 0 && e < a.A.n_experts;
      if (!e_ok) set_err(a.P.err, MOE_ERR_EXPERT);
      dptr[tid] = (e_ok && ptr_ok(vd, a.P.err)) ? vd : 0;
    }
    if (tid < n) {
      dsc[kDescDst + tid] = r_dst;
      ((MOE_LDS float*)dsc)[kDescW + tid] = r_w;
      dsc[kDescLive + tid] = 1;
    }
    __syncthreads();
  }
  const int ng = uni(dsc[kDescNg]), e0 = uni(dsc[kDescE0]), n = uni(dsc[kDescN]);
  if (ng == 0) return;
  const ActSplit act = MODE == DN_DESC ? act_layout_kb(actp, n, U, FMT == Q5_1) : act_layout(actp, n, U, FMT == Q5_1);
  const int ntiles = a.ntiles;
  const int bid = (int)blockIdx.x, grid = (int)gridDim.x;
  const int ntw = bid >= ntiles ? 0 : ntiles <= grid ? 1 : (ntiles - bid + grid - 1) / grid;   // tiles here
  // this wave's chunks, in order: per tile (t = bid + kt grid) its groups g = wave + q kDnWaves,
  // per group the tile's rows in nsub chunks of rc rows
  const int rc = a.rc, nsub = a.nsub;
  const int qpt = wave < ng ? (ng - wave + kDnWaves - 1) / kDnWaves : 0;   // groups per tile
  const int nch = ntw * qpt * nsub;
  const int M = a.S.M, NS = a.S.NS;
  MOE_LDS uint8_t* myring = ring + wave * NS * M * 1024;
  auto chunk_rows = [&](int t, int sub, int& r0, int& nr) {
    const int te = min(t * tr + tr, a.A.n_embd);
    r0 = t * tr + sub * rc;
    nr = min(rc, te - r0);
  };
  struct Pos {
    int t, q, s;
  };
  Pos ip{(int)blockIdx.x, 0, 0};   // the next chunk to issue, stepped one chunk at a time
  auto issue = [&](MOE_LDS uint8_t* slot) {
    const Pos p = ip;
    if (++ip.s == nsub) {
      ip.s = 0;
      if (++ip.q == qpt) {
        ip.q = 0;
        ip.t += (int)gridDim.x;
      }
    }
    const int g = wave + p.q * kDnWaves;
    int r0, nr;
    chunk_rows(p.t, p.s, r0, nr);
    const uint64_t w = uni64(dptr[g]);
    if (w && nr > 0)
      issue_span(slot, M, (const uint8_t*)(uintptr_t)(w + (uint64_t)r0 * G.rb), (uint32_t)(nr * G.rb));
    else   // a skipped group (or rows past the end) keeps the count of loads: one 16-byte chunk
      issue_span(slot, M, (const uint8_t*)a.P.err, 1);
  };
  const int pre = min(NS, nch);
  // ---- 2. descriptor path: the h rows and the first chunks of the stream go out at once; the
  //         entries' metadata is worked out while they are in flight
  if constexpr (MODE == DN_DESC) {
    const uint32_t qb = (uint32_t)(n * U * 16), db = (uint32_t)((n * U * 4 + 15) & ~15);
    dma_span(a.hq_lo, qb, (MOE_LDS uint8_t*)act.lo, wave, kDnWaves);
    dma_span(a.hq_hi, qb, (MOE_LDS uint8_t*)act.hi, (wave + 3) % kDnWaves, kDnWaves);
    dma_span(a.hq_d, db, (MOE_LDS uint8_t*)act.d, (wave + 6) % kDnWaves, kDnWaves);
    if constexpr (FMT == Q5_1) dma_span(a.hq_s, db, (MOE_LDS uint8_t*)act.s, (wave + 7) % kDnWaves, kDnWaves);
    for (int kc = 0; kc < pre; ++kc) issue(myring + kc * M * 1024);
  }
  // entry metadata: destination (or -1), weight, owner = first live entry naming its dst
  if (tid < n) {
    int g = 0;
    while (g + 1 < ng && dsc[kDescGs + g + 1] <= tid) ++g;
    const int d = dsc[kDescDst + tid];
    int live = dsc[kDescLive + tid] && dptr[g] != 0;
    if (live && (d < 0 || d >= a.n_rows)) {
      set_err(a.P.err, MOE_ERR_DST);
      live = 0;
    }
    mdst[tid] = live ? d : -1;
    mw[tid] = ((MOE_LDS float*)dsc)[kDescW + tid];
  }
  lds_barrier();
  if (wave == 0) {   // n <= 64: one lane per entry
    const int lane = tid;
    int owner = 0;
    if (lane < n) {
      const int d = mdst[lane];
      owner = d >= 0;
      for (int q = 0; q < lane && owner; ++q) owner = mdst[q] != d;
      mown[lane] = owner;
    }
    const uint64_t om = __ballot(owner);
    if (owner) {
      const int o = __popcll(om & ((1ull << lane) - 1ull));
      omap[lane] = o;
      ownl[o] = lane;
    }
    if (lane == 0) misc[8] = __popcll(om);
  }
  lds_barrier();
  const int nown = uni(misc[8]);

  // the first tile's rows of every destination (wave 0, one float per lane): ny loads
  const int r00 = (int)blockIdx.x * tr, nr0 = min(tr, a.A.n_embd - r00);   // first tile
  auto stage_y = [&]() {
    int ny = 0;
    if (wave == 0 && ntw > 0) {
      for (int p = 0; p * 64 < nown * nr0; ++p, ++ny) {
        const int l = p * 64 + (tid & 63);
        if (l < nown * nr0) {
          const int o = l / nr0, m = l - o * nr0;
          const float* src = a.Y + (size_t)mdst[ownl[o]] * a.ldy + r00 + m;
          __builtin_amdgcn_global_load_lds((const void*)src, (MOE_LDS void*)(ybuf + 64 * p), 4, 0, 0);
        }
      }
    }
    return ny;
  };
  int ny = 0;   // wave 0: loads issued after the first chunks (their waits allow for them)
  if constexpr (MODE == DN_DESC) {
    ny = uni(stage_y());
    wait_vm(pre * M + ny);   // this wave's pieces of the h rows, older than every chunk, have landed
  } else {
    // the caller's plan: q8_1 rows of h by absolute entry, staged after the first chunks go out
    auto mid = [&](int) {
      stage_y();
      for (int kc = 0; kc < pre; ++kc) issue(myring + kc * M * 1024);
      wait_vm(pre * M);   // the Y rows, older than every chunk, have landed
    };
    act_stage_q<kDnThreads, 16>(a.hq + (size_t)e0 * U * 36, n * U, act, mid);
  }
  int issued = pre;
  lds_barrier();

  // ---- 3. tiles
  // planar NL4 rows of a 16-byte multiple: a chunk that lands 16-byte aligned takes the aligned
  // reads (one-token launch)
  const bool pa = FMT == NL4 && G.ly.c_a == 16u && G.ly.c_b == 0u && (G.rb & 15) == 0;
  int kc = 0;
  for (int kt = 0; kt < ntw; ++kt) {
    const int t = (int)blockIdx.x + kt * (int)gridDim.x;
    const int r0 = t * tr, nr = min(tr, a.A.n_embd - r0);
    for (int q = 0, sb = 0; q < qpt; ++kc, sb = sb + 1 < nsub ? sb + 1 : 0, q += sb == 0) {
      const int g = wave + q * kDnWaves;
      wait_vm((issued - 1 - kc) * M + (kc < pre ? ny : 0));
      MOE_LDS uint8_t* slot = myring + slot_of(kc, NS) * M * 1024;
      const uint64_t w = uni64(dptr[g]);
      int c_r0, c_nr;
      chunk_rows(t, sb, c_r0, c_nr);
      if (w && c_nr > 0) {
        const uint32_t ra = (uint32_t)(slot - ring) + (uint32_t)((w + (uint64_t)c_r0 * G.rb) & 15);
        const int a0 = uni(dsc[kDescGs + g]), a1 = uni(dsc[kDescGs + g + 1]);
        const int o0 = c_r0 - r0;   // the chunk's first row inside the tile
        for (int p0 = 0; p0 < c_nr; p0 += G.rp) {   // the chunk's rows in wave passes
          const int np = min(G.rp, c_nr - p0);
          const uint32_t rp0 = ra + (uint32_t)(p0 * G.rb);
          for (int c0 = a0; c0 < a1; c0 += ONE ? 1 : kSlots) {
            const int ne = ONE ? 1 : min(kSlots, a1 - c0);
            int sidx[kSlots];
#pragma unroll
            for (int e = 0; e < kSlots; ++e) sidx[e] = e < ne ? c0 + e : 0;
            auto outd = [&](int i, int e, float v) { ores[(c0 + e) * tr + o0 + p0 + i] = v; };
            if constexpr (ONE && FMT == NL4) {
              if (pa && (rp0 & 15u) == 0)
                dot_pass_pa<1>(ring, rp0, rp0, np, np, G, tb, act, sidx, outd);
              else
                dot_pass_n<FMT, 1>((const MOE_LDS uint32_t*)ring, rp0, rp0, np, np, G, tb, act, sidx, outd);
            } else if constexpr (ONE)
              dot_pass_n<FMT, 1>((const MOE_LDS uint32_t*)ring, rp0, rp0, np, np, G, tb, act, sidx, outd);
            else
              dot_pass<FMT>((const MOE_LDS uint32_t*)ring, rp0, rp0, np, np, G, tb, act, sidx, ne, outd,
                            pa && (rp0 & 15u) == 0);
          }
        }
      }
      if (kc + NS < nch) {
        MOE_WAIT_LGKM0;
        issue(slot);
        ++issued;
      }
    }
    if (kt == 0 && ny) wait_vm(0);   // wave 0: the first tile's Y rows (issued after its first chunks)
    lds_barrier();
    // scatter: one thread per (owner entry, row)
    for (int idx = tid; idx < n * nr; idx += kDnThreads) {
      const int i = idx / nr, m = idx - i * nr;
      if (!mown[i]) continue;
      const int d = mdst[i];
      float* y = a.Y + (size_t)d * a.ldy + r0 + m;
      float acc = kt == 0 ? ybuf[omap[i] * nr + m] : *y;
      *y = dst_sum(acc, i, n, d, m, tr, mdst, mw, ores);
    }
    lds_barrier();
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

// One wave per token.
__global__ __launch_bounds__(64) void k_route(const float* __restrict__ logits, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ __align__(16) uint32_t s_scr[3 * 1024 + 128];   // route_scr_words(kMaxE)
  __shared__ int s_ids[32];
  __shared__ float s_w[32];
  __shared__ uint32_t s_bits[32];
  const int t = blockIdx.x;
  issue_logits(logits + (size_t)t * E, E, (MOE_LDS float*)s_scr);
  __builtin_amdgcn_s_waitcnt(MOE_VM(0));
  route_token((MOE_LDS uint32_t*)s_scr, E, k, (MOE_LDS int*)s_ids, (MOE_LDS float*)s_w, (MOE_LDS uint32_t*)s_bits);
  if ((int)threadIdx.x < k) {
    ids[(size_t)t * k + threadIdx.x] = s_ids[threadIdx.x];
    w[(size_t)t * k + threadIdx.x] = s_w[threadIdx.x];
  }
}

// One wave: group the T * k routed entries and write the plan.
__global__ __launch_bounds__(64) void k_plan(const int32_t* __restrict__ ids, const float* __restrict__ w,
                                             const int32_t* __restrict__ dst_of_token, int T, int k,
                                             int E, int entry_base, PlanArgs P) {
  __shared__ int s_plan[kPlanLInts];
  const PlanL p = plan_l((MOE_LDS int*)s_plan);
  const int n = T * k;
  const int i = threadIdx.x;
  if (i < n) {
    p.rid[i] = ids[i];
    p.rw[i] = w[i];
  }
  if (i < T) p.dtok[i] = dst_of_token ? dst_of_token[i] : i;
  __syncthreads();
  group_wave(p, n, k, E, entry_base, P.err);
  __syncthreads();
  publish_plan<64>(p, P);
}

// Over (entry, h block) of the call: two blocks per wave.
__global__ __launch_bounds__(kThreads) void k_swiglu(PlanArgs P, const float* __restrict__ g,
                                                     const float* __restrict__ u, int n_ff, int ld,
                                                     float* h, uint8_t* hq) {
  __shared__ int s_gs[kMaxGrp + 1];
  __shared__ int s_misc[4];
  int r_ng = 0, r_gs = 0;
  if ((int)threadIdx.x == 0) r_ng = *P.n_groups;
  if ((int)threadIdx.x <= P.cap_groups) r_gs = P.grp_start[threadIdx.x];
  if ((int)threadIdx.x == 0) s_misc[3] = r_ng;
  if ((int)threadIdx.x <= P.cap_groups) s_gs[threadIdx.x] = r_gs;
  __syncthreads();
  validate_groups((MOE_LDS int*)s_gs, s_misc[3], P, (MOE_LDS int*)s_misc);
  __syncthreads();
  const int e0 = uni(s_misc[1]), e1 = uni(s_misc[2]);
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

// ------------------------------------------------------------------ weight repack -----------

// Byte offset in a row-major row of the byte at offset p of the same row in planar layout (p even:
// every field of both layouts starts at an even offset and has an even length).
template <int FMT>
__device__ __forceinline__ uint32_t planar_src(uint32_t nblk, uint32_t p) {
  constexpr uint32_t B = block_bytes(FMT), C = code_bytes(FMT), H = head_bytes(FMT), S = B - C;
  if (p < C * nblk) {
    const uint32_t b = p / C;
    return B * b + H + (p - C * b);
  }
  const uint32_t q = p - C * nblk, b = q / S, r = q - S * b;
  return r < H ? B * b + r : B * b + H + C + (r - H);   // the header, then (CB2 / CB3) the sub-scales
}
// The inverse: offset in the planar row of byte p of the row-major row.
template <int FMT>
__device__ __forceinline__ uint32_t rowmajor_src(uint32_t nblk, uint32_t p) {
  constexpr uint32_t B = block_bytes(FMT), C = code_bytes(FMT), H = head_bytes(FMT), S = B - C;
  const uint32_t b = p / B, r = p - B * b;
  if (r < H) return C * nblk + S * b + r;
  if (r >= H + C) return C * nblk + S * b + H + (r - H - C);
  return C * b + (r - H);
}

// One row per workgroup at a time, two bytes per lane: every output half-word is gathered from
// its place in the source row (the row, at most 8.5 KB, stays in cache while its workgroup
// reads it).
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_repack(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                     long rows, int rb, int nblk, int to_planar) {
  const int nh = rb >> 1;
  for (long r = blockIdx.x; r < rows; r += gridDim.x) {
    const uint16_t* s = src + r * nh;
    uint16_t* d = dst + r * nh;
    for (int i = threadIdx.x; i < nh; i += kThreads) {
      const uint32_t p = 2u * (uint32_t)i;
      const uint32_t q = to_planar ? planar_src<FMT>((uint32_t)nblk, p) : rowmajor_src<FMT>((uint32_t)nblk, p);
      d[i] = s[q >> 1];
    }
  }
}

// ------------------------------------------------------------------ prompt path (large T) ---

// The plan of a prompt's T x k entries (T x k up to MOE_MAX_PREFILL_ENTRIES, E up to 1024), by
// one workgroup: per-expert counts (LDS atomics: a count does not depend on their order), the
// groups and their starts by a scan over the experts, then rounds of 256 entries in token-major
// order where each entry's place inside its group is its expert's count so far plus the number
// of same-expert entries before it in the round (a per-expert bitmap of the round, set with LDS
// atomic ORs and read back by popcount): groups ascending by expert, entries ascending by token,
// the same order as the decode path's plan. ent_of[t k + j] = the entry of token t's j-th choice
// (-1 for an expert id out of range, which is dropped with MOE_ERR_EXPERT).
constexpr int kPpThreads = 256;
constexpr int kPpMaxE = 1024;
__global__ __launch_bounds__(kPpThreads) void k_plan_large(const int32_t* __restrict__ ids, const float* __restrict__ w,
                                                           const int32_t* __restrict__ dst_of_token, int T, int k,
                                                           int E, int entry_base, PlanArgs P, int32_t* ent_of) {
  __shared__ int s_cnt[kPpMaxE];     // entries per expert, then the running count in pass 2
  __shared__ int s_start[kPpMaxE];   // first entry of the expert's group (relative)
  __shared__ uint32_t s_bits[kPpMaxE * (kPpThreads / 32)];   // this round's entries per expert
  __shared__ int s_part[kPpThreads];
  __shared__ int s_tot[2];
  const int tid = threadIdx.x, n = T * k;
  for (int e = tid; e < E; e += kPpThreads) s_cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kPpThreads) {
    const int e = ids[i];
    if (e >= 0 && e < E)
      atomicAdd(&s_cnt[e], 1);
    else
      set_err(P.err, MOE_ERR_EXPERT);
  }
  __syncthreads();
  // scan over the experts: each thread a run of 4 (E <= 1024), then the runs' totals
  const int per = (E + kPpThreads - 1) / kPpThreads;
  int c_ent = 0, c_grp = 0;
  for (int q = 0; q < per; ++q) {
    const int e = tid * per + q;
    if (e < E) {
      c_ent += s_cnt[e];
      c_grp += s_cnt[e] > 0;
    }
  }
  s_part[tid] = c_ent | (c_grp << 16);   // at most 65535 entries and 1024 groups
  __syncthreads();
  for (int off = 1; off < kPpThreads; off <<= 1) {   // inclusive scan of the packed pairs
    const int v = tid >= off ? s_part[tid - off] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int b_ent = (tid ? s_part[tid - 1] : 0) & 0xFFFF, b_grp = (tid ? s_part[tid - 1] : 0) >> 16;
  for (int q = 0; q < per; ++q) {
    const int e = tid * per + q;
    if (e < E) {
      s_start[e] = b_ent;
      if (s_cnt[e] > 0) {
        P.grp_expert[b_grp] = e;
        P.grp_start[b_grp] = entry_base + b_ent;
        ++b_grp;
      }
      b_ent += s_cnt[e];
    }
  }
  if (tid == kPpThreads - 1) {
    s_tot[0] = s_part[tid] & 0xFFFF;
    s_tot[1] = s_part[tid] >> 16;
  }
  __syncthreads();
  if (tid == 0) {
    P.grp_start[s_tot[1]] = entry_base + s_tot[0];
    *P.n_groups = s_tot[1];
  }
  for (int e = tid; e < E; e += kPpThreads) s_cnt[e] = 0;
  // pass 2: rounds of kPpThreads entries
  constexpr int kW = kPpThreads / 32;
  for (int r0 = 0; r0 < n; r0 += kPpThreads) {
    for (int x = tid; x < E * kW; x += kPpThreads) s_bits[x] = 0u;
    __syncthreads();
    const int i = r0 + tid;
    const int e = i < n ? ids[i] : -1;
    const bool ok = e >= 0 && e < E;
    if (ok) atomicOr(&s_bits[e * kW + (tid >> 5)], 1u << (tid & 31));
    __syncthreads();
    if (i < n) {
      int pos = -1;
      if (ok) {
        int rank = s_cnt[e];
        for (int q = 0; q < (tid >> 5); ++q) rank += __popc(s_bits[e * kW + q]);
        rank += __popc(s_bits[e * kW + (tid >> 5)] & ((1u << (tid & 31)) - 1u));
        pos = entry_base + s_start[e] + rank;
        const int t = i / k;
        P.ent_src[pos] = t;
        P.ent_dst[pos] = dst_of_token ? dst_of_token[t] : t;
        P.ent_w[pos] = w ? w[i] : 0.0f;
      }
      if (ent_of) ent_of[i] = pos;
    }
    __syncthreads();
    for (int x = tid; x < E; x += kPpThreads) {
      int add = 0;
      for (int q = 0; q < kW; ++q) add += __popc(s_bits[x * kW + q]);
      s_cnt[x] += add;
    }
    __syncthreads();
  }
}

// Grouped GEMM of the prompt path on the matrix cores: for group g (blockIdx.y) and a tile of
// kPfRows rows of one of its matrices (blockIdx.x: gate tiles, then up tiles; or down), the rows'
// dot products with every entry's q8_1 activation row, entries in passes of kPfEnt. Per K chunk
// of kPfK weights the tile's raw rows come into LDS by direct-to-LDS loads, are decoded once into
// int8 codes and per-block float scales (the decode path's decoders), the entries' quants and
// scales are staged beside them, and each wave runs one 16 x 16 output tile with
// v_mfma_i32_16x16x32_i8: one instruction per 32-weight block gives the exact integer sums of
// 16 rows x 16 entries, which are scaled in float32 and added in block order, so every output
// is one fixed sequence of float operations: (d_w f(d_x)) isum (+ m f(s_x) for Q5_1), summed
// block after block. Both operands list their 32 weights in the same slot order, so the integer
// sum is that of the block.
constexpr int kPfRows = 32;            // rows of a workgroup tile (two 16-row MFMA tiles)
constexpr int kPfEnt = 32;             // entries of a pass (two 16-column MFMA tiles)
constexpr int kPfK = 256;              // weights of a K chunk (8 blocks of 32, one of 256): small chunks
                                       // keep the LDS small, so five or six workgroups share a CU
constexpr int kPfBlk = kPfK / 32;
constexpr int kPfCS = kPfK + 16;       // LDS row stride of the int8 codes and quants
constexpr int kPfSS = 36;              // LDS block stride of the per-(block, row / entry) scales: a
                                       // wave's stores (blocks x 4 rows) spread over the banks
constexpr int kPfThreads = 256;
static_assert(kPfSS >= kPfRows && kPfSS >= kPfEnt && kPfSS % 4 == 0, "scale rows fit, float4 reads aligned");
// Raw rows of a chunk, packed: row r's aligned 16-byte pieces at r * kPfP pieces (a chunk's bytes
// plus its start's offset inside a piece), so one direct-to-LDS instruction (64 pieces) covers
// several rows.
template <int FMT>
constexpr int pf_pieces() { return (kPfK / block_weights(FMT) * block_bytes(FMT) + 15) / 16 + 1; }
// LDS of the prompt-path GEMM for format FMT: raw rows, codes and quants, the per-block scales
// (weights and activations; offsets and sum fields for Q5_1 only), the CB grid (CB2 / CB3 only).
template <int FMT>
constexpr int pf_lds() {
  return kPfRows * pf_pieces<FMT>() * 16 + (kPfRows + kPfEnt) * kPfCS + (FMT == Q5_1 ? 4 : 2) * kPfBlk * 4 * kPfSS +
         ((FMT == CB2 || FMT == CB3) ? 4096 : 0) + 64;
}
static_assert(5 * pf_lds<NL4>() <= 160 * 1024, "five NL4 prompt-path workgroups share a CU's LDS");
static_assert(2 * pf_lds<Q8_0>() <= 160 * 1024 && 2 * pf_lds<Q5_1>() <= 160 * 1024 &&
              2 * pf_lds<CB3>() <= 160 * 1024, "two prompt-path workgroups share a CU's LDS");
// The (row, block) unit that decode slot x (0..511) of a chunk takes: each 64-slot wave pass
// covers 8 rows x 8 blocks with the row fastest, so the 8 lanes that store their 32 codes to LDS
// together write 8 different rows (row stride 132 dwords: distinct bank groups) rather than
// blocks 32 bytes apart in one row.
static_assert(kPfRows == 32 && kPfBlk <= 16 && kPfRows * kPfBlk % kPfThreads == 0, "decode slot map");
__device__ __forceinline__ int pf_dec_row(int x) { return 8 * ((x >> 6) & 3) + (x & 7); }
__device__ __forceinline__ int pf_dec_blk(int x) { return 8 * (x >> 8) + ((x >> 3) & 7); }

struct PfArgs {
  LayerArgs A;
  PlanArgs P;
  int nmat;             // 2: gate and up (outputs out0, out1); 1: down (output out0, times ent_w)
  int rows, K, rb;      // rows per matrix, weights per row, bytes per row
  Lay ly;               // row-major field map (the chunk's local blocks)
  const uint8_t* act;   // q8_1 rows: by token (gate / up, through ent_src) or by entry (down)
  int act_by_entry, n_act;
  float* out0;
  float* out1;
  long ld;
};

template <int FMT>
__global__ __launch_bounds__(kPfThreads) void k_pf_gemm(PfArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int kP = pf_pieces<FMT>();
  MOE_LDS uint8_t* raw = (MOE_LDS uint8_t*)smem;
  MOE_LDS uint8_t* codes = raw + kPfRows * kP * 16;
  MOE_LDS uint8_t* quant = codes + kPfRows * kPfCS;
  MOE_LDS float* dws = (MOE_LDS float*)(quant + kPfEnt * kPfCS);   // [blk][row]
  MOE_LDS float* dxs = dws + kPfBlk * kPfSS;                      // [blk][entry]
  MOE_LDS float* mos = dxs + kPfBlk * kPfSS;                      // [blk][row] (Q5_1 offsets)
  MOE_LDS float* sxs = mos + kPfBlk * kPfSS;                      // [blk][entry] (Q5_1 sum fields)
  MOE_LDS uint32_t* grid = (MOE_LDS uint32_t*)(dxs + (FMT == Q5_1 ? 3 : 1) * kPfBlk * kPfSS);   // CB2 / CB3
  MOE_LDS int* misc = (MOE_LDS int*)(grid + ((FMT == CB2 || FMT == CB3) ? 1024 : 0));
  const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
  const int g = (int)blockIdx.y;
  const int tpm = (a.rows + kPfRows - 1) / kPfRows;
  const int mi = (int)blockIdx.x / tpm, r0 = ((int)blockIdx.x - mi * tpm) * kPfRows;
  // the group, checked as every call checks its plan (one thread; the others wait)
  if (tid == 0) {
    int ok = 1, sb = 0, se = 0, e = -1;
    const int ng = *a.P.n_groups;
    if (ng < 0 || ng > a.P.cap_groups) {
      set_err(a.P.err, MOE_ERR_NGROUPS);
      ok = 0;
    } else if (g >= ng) {
      ok = 0;
    } else {
      const int s0 = a.P.grp_start[0];
      sb = a.P.grp_start[g];
      se = a.P.grp_start[g + 1];
      if (s0 < 0 || sb < s0 || se < sb || se - s0 > a.P.cap_entries) {
        set_err(a.P.err, MOE_ERR_ENTRIES);
        ok = 0;
      } else {
        e = a.P.grp_expert[g];
        if (e < 0 || e >= a.A.n_experts) {
          set_err(a.P.err, MOE_ERR_EXPERT);
          ok = 0;
        }
      }
    }
    misc[0] = ok;
    misc[1] = sb;
    misc[2] = se;
    misc[3] = e;
  }
  uint32_t t_nl4[4];
  load_nl4(a.A.nl4, t_nl4);
  if constexpr (FMT == CB2 || FMT == CB3) {
    const uint32_t* src = (const uint32_t*)(FMT == CB2 ? a.A.cb2 : a.A.cb3);
    for (int i = tid; i < 512; i += kPfThreads) grid[i] = src[i];
  }
  __syncthreads();
  if (!uni(misc[0])) return;
  const int sb = uni(misc[1]), se = uni(misc[2]), e = uni(misc[3]);
  const void* const* mats = mi == 0 ? (a.nmat == 2 ? a.A.gate : a.A.down) : a.A.up;
  const uint64_t wp = uni64((uint64_t)(uintptr_t)mats[e]);
  if (!ptr_ok(wp, a.P.err)) return;
  Tables tb;
  tables_init(tb, t_nl4, grid, grid);
  float* out = mi == 0 ? a.out0 : a.out1;
  const int mt = wave & 1, nt = wave >> 1, q = lane >> 4, l16 = lane & 15;
  const int bw = block_weights(FMT), bb = block_bytes(FMT);
  const uint32_t cbytes = (uint32_t)(kPfK / bw * bb);   // raw bytes of a row's chunk
  const int nkc = (a.K + kPfK - 1) / kPfK;
  // the memory traffic of a chunk: its raw rows (direct to LDS) and the entries' q8_1 blocks (to
  // registers, kPfEnt * kPfBlk / kPfThreads blocks per thread), issued together
  constexpr int kQ = kPfEnt * kPfBlk / kPfThreads;
  uint32_t qq[kQ][9];
  long arow[kQ];   // the activation row of this thread's entries in the pass, or -1
  auto issue_chunk = [&](int ep, int ne, int kc) {
    const int nblk = min(kPfBlk, (a.K - kc) / 32);
    const uint32_t nbytes = (uint32_t)(nblk * 32 / bw * bb);
    // piece i of the tile's chunk: row i / kP, piece i % kP of the row's span (from its aligned
    // start); wave w issues the 64-piece instructions w, w + 4, ... (rows past the matrix and
    // pieces past a row's span reload the row's first piece: never read)
    for (int i0 = wave * 64; i0 < kPfRows * kP; i0 += kPfThreads) {
      const int idx = i0 + lane, r = idx / kP, p = idx - r * kP;
      const int rr = min(r0 + min(r, kPfRows - 1), a.rows - 1);
      const uint64_t src = wp + (uint64_t)rr * (uint64_t)a.rb + (uint64_t)(kc / bw * bb);
      const uint32_t need = ((uint32_t)(src & 15u) + nbytes + 15u) >> 4;
      const uint64_t at = (src & ~15ull) + ((r0 + r < a.rows && (uint32_t)p < need) ? 16ull * p : 0ull);
      if (idx < kPfRows * kP)   // (lanes past the tile would write past the raw rows)
        __builtin_amdgcn_global_load_lds((const void*)(uintptr_t)at, (MOE_LDS void*)(raw + i0 * 16), 16, 0,
                                         kAuxStream);
    }
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
      const int x = tid + j * kPfThreads, en = x / kPfBlk, bl = x - en * kPfBlk;
#pragma unroll
      for (int i = 0; i < 9; ++i) qq[j][i] = 0u;
      if (arow[j] >= 0 && bl < nblk) {
        const uint32_t* pq = (const uint32_t*)(a.act + (size_t)arow[j] * (size_t)(a.K / 32) * 36 +
                                               (size_t)(kc / 32 + bl) * 36);
#pragma unroll
        for (int i = 0; i < 9; ++i) qq[j][i] = pq[i];
      }
    }
  };
  for (int ep = sb; ep < se; ep += kPfEnt) {
    const int ne = min(kPfEnt, se - ep);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // the pass's activation rows, read once (gate / up: the entries' tokens, checked)
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
      const int en = (tid + j * kPfThreads) / kPfBlk;
      long row = -1;
      if (en < ne) {
        row = ep + en;
        if (!a.act_by_entry) {
          row = a.P.ent_src[ep + en];
          if (row < 0 || row >= a.n_act) {
            set_err(a.P.err, MOE_ERR_SRC);
            row = -1;
          }
        }
      }
      arow[j] = row;
    }
    __syncthreads();   // the previous pass's reads of LDS are done
    issue_chunk(ep, ne, 0);
    for (int ck = 0; ck < nkc; ++ck) {
      const int kc = ck * kPfK;
      const int nblk = min(kPfBlk, (a.K - kc) / 32);   // blocks of this chunk (K is a multiple of 64)
      __builtin_amdgcn_s_waitcnt(MOE_VM(0));   // this chunk's raw rows and quants have landed
      // (2) the entries' quants into LDS
#pragma unroll
      for (int j = 0; j < kQ; ++j) {
        const int x = tid + j * kPfThreads, en = x / kPfBlk, bl = x - en * kPfBlk;
        MOE_LDS uint32_t* dq = (MOE_LDS uint32_t*)(quant + en * kPfCS + 32 * bl);
        *(MOE_LDS u32x4*)dq = u32x4{qq[j][1], qq[j][2], qq[j][3], qq[j][4]};
        *(MOE_LDS u32x4*)(dq + 4) = u32x4{qq[j][5], qq[j][6], qq[j][7], qq[j][8]};
        dxs[bl * kPfSS + en] = h2f(qq[j][0] & 0xFFFFu);
        if constexpr (FMT == Q5_1) sxs[bl * kPfSS + en] = h2f(qq[j][0] >> 16);
      }
      __syncthreads();
      // (3) decode the raw rows into codes and scales: (row, block) pairs over the threads, the
      //     reads of both of a thread's units first
      {
        constexpr int kD = kPfRows * kPfBlk / kPfThreads;
        URaw<FMT> rr[kD];
        bool dl[kD];
#pragma unroll
        for (int j = 0; j < kD; ++j) {
          const int x = tid + j * kPfThreads, r = pf_dec_row(x), bl = pf_dec_blk(x);
          dl[j] = r0 + r < a.rows && bl < nblk;
          const uint64_t src = wp + (uint64_t)(r0 + r) * (uint64_t)a.rb + (uint64_t)(kc / bw * bb);
          const uint32_t row = (uint32_t)(r * kP * 16) + (uint32_t)(src & 15u);   // from raw
          unit_load<FMT>((const MOE_LDS uint32_t*)raw, row, dl[j] ? bl : 0, a.ly, rr[j]);
        }
#pragma unroll
        for (int j = 0; j < kD; ++j) {
          const int x = tid + j * kPfThreads, r = pf_dec_row(x), bl = pf_dec_blk(x);
          uint32_t c[8];
          float sc, mo;
          unit_decode<FMT>(rr[j], bl, tb, c, sc, mo);
          if (!dl[j]) {
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = 0u;
            sc = 0.0f;
            mo = 0.0f;
          }
          MOE_LDS uint32_t* dc = (MOE_LDS uint32_t*)(codes + r * kPfCS + 32 * bl);
          *(MOE_LDS u32x4*)dc = u32x4{c[0], c[1], c[2], c[3]};
          *(MOE_LDS u32x4*)(dc + 4) = u32x4{c[4], c[5], c[6], c[7]};
          dws[bl * kPfSS + r] = sc;
          if constexpr (FMT == Q5_1) mos[bl * kPfSS + r] = mo;   // (the others have no offset plane)
        }
      }
      __syncthreads();
      // the next chunk's loads go out now (raw is free, the quants are in LDS) and land while
      // this chunk's products run
      if (ck + 1 < nkc) issue_chunk(ep, ne, kc + kPfK);
      // (4) this wave's 16 x 16 tile, block after block
      const MOE_LDS uint8_t* pa = codes + (16 * mt + l16) * kPfCS + 8 * q;
      const MOE_LDS uint8_t* pb = quant + (16 * nt + l16) * kPfCS + 8 * q;
      auto block_products = [&](int bl) {
        const long av = *(const MOE_LDS long*)(pa + 32 * bl);
        const long bv = *(const MOE_LDS long*)(pb + 32 * bl);
        typedef int v4i __attribute__((ext_vector_type(4)));
        const v4i z = {0, 0, 0, 0};
        const v4i d = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, bv, z, 0, 0, 0);
        const f32x4 dw = *(const MOE_LDS f32x4*)(dws + bl * kPfSS + 16 * mt + 4 * q);
        const float dx = dxs[bl * kPfSS + 16 * nt + l16];
        float mw[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        float sx = 0.0f;
        if constexpr (FMT == Q5_1) {
          const f32x4 m4 = *(const MOE_LDS f32x4*)(mos + bl * kPfSS + 16 * mt + 4 * q);
          mw[0] = m4.x; mw[1] = m4.y; mw[2] = m4.z; mw[3] = m4.w;
          sx = sxs[bl * kPfSS + 16 * nt + l16];
        }
        const float dwv[4] = {dw.x, dw.y, dw.z, dw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (FMT == Q5_1) {
            const float prod = (dwv[i] * dx) * (float)d[i] + mw[i] * sx;
            acc[i] = acc[i] + prod;
          } else {
            // one fused multiply-add per block (the products are sums of float roundings either
            // way; this path is held to a tolerance, not to the decode path's bits)
            acc[i] = __builtin_fmaf(dwv[i] * dx, (float)d[i], acc[i]);
          }
        }
      };
      // (a straight-line form of whole chunks took 12 more VGPRs, one workgroup less per CU, and
      // was slower)
      for (int bl = 0; bl < nblk; ++bl) block_products(bl);
      __syncthreads();   // the products' reads of codes and quants are done before they are rewritten
    }
    // outputs: lane holds rows 4 q + i of its row tile, entry l16 of its entry tile
    const int en = 16 * nt + l16;
    if (en < ne) {
      const int ent = ep + en;
      const float wv = a.nmat == 1 ? a.P.ent_w[ent] : 1.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = r0 + 16 * mt + 4 * q + i;
        if (row < a.rows) out[(size_t)ent * (size_t)a.ld + row] = a.nmat == 1 ? wv * acc[i] : acc[i];
      }
    }
  }
}

// SwiGLU + q8_1 of the prompt's entries [grp_start[0], grp_start[n_groups]) (the group table is
// trusted as far as its two ends; they are checked against the capacity).
__global__ __launch_bounds__(kThreads) void k_pf_swiglu(PlanArgs P, const float* __restrict__ g,
                                                        const float* __restrict__ u, int n_ff, long ld,
                                                        float* h, uint8_t* hq) {
  __shared__ int s_e[2];
  if (threadIdx.x == 0) {
    const int ng = *P.n_groups;
    int e0 = 0, e1 = 0;
    if (ng < 0 || ng > P.cap_groups) {
      set_err(P.err, MOE_ERR_NGROUPS);
    } else if (ng > 0) {
      e0 = P.grp_start[0];
      e1 = P.grp_start[ng];
      if (e0 < 0 || e1 < e0 || e1 - e0 > P.cap_entries) {
        set_err(P.err, MOE_ERR_ENTRIES);
        e0 = e1 = 0;
      }
    }
    s_e[0] = e0;
    s_e[1] = e1;
  }
  __syncthreads();
  const int e0 = uni(s_e[0]), e1 = uni(s_e[1]);
  const int nb = n_ff / 32;
  const long total = (long)(e1 - e0) * nb;
  const int half = threadIdx.x >> 5, l32 = threadIdx.x & 31;
  for (long base = (long)blockIdx.x * 8; base < total; base += (long)gridDim.x * 8) {
    const long it = base + half;
    const bool live = it < total;
    const long ai = live ? e0 + it / nb : e0;
    const int b = live ? (int)(it % nb) : 0;
    const float gv = live ? g[ai * ld + 32 * b + l32] : 0.0f;
    const float uv = live ? u[ai * ld + 32 * b + l32] : 0.0f;
    swiglu_q81_lanes(gv, uv, l32, live, hq + (size_t)ai * nb * 36 + (size_t)b * 36,
                     h ? h + ai * ld + 32 * b : nullptr);
  }
}

// Y[dst(t)] += sum over j < k of O[ent_of[t k + j]], j ascending, one thread per output element
// (a prompt's destinations are distinct rows, so no two threads add into one element).
__global__ __launch_bounds__(kThreads) void k_pf_scatter(PlanArgs P, const int32_t* __restrict__ ent_of,
                                                         const int32_t* __restrict__ dst_of_token, int k,
                                                         const float* __restrict__ O, long ldo, int n_embd,
                                                         float* Y, int n_rows, long ldy) {
  __shared__ int s_e[2];
  if (threadIdx.x == 0) {
    const int ng = *P.n_groups;
    int e0 = 0, e1 = 0;
    if (ng > 0 && ng <= P.cap_groups) {
      e0 = P.grp_start[0];
      e1 = P.grp_start[ng];
    }
    s_e[0] = e0;
    s_e[1] = e1;
  }
  __syncthreads();
  const int t = (int)blockIdx.y, c = (int)blockIdx.x * kThreads + (int)threadIdx.x;
  const int e0 = s_e[0], e1 = s_e[1];
  const int dst = dst_of_token ? dst_of_token[t] : t;
  if (dst < 0 || dst >= n_rows) {
    if (c == 0) set_err(P.err, MOE_ERR_DST);
    return;
  }
  if (c >= n_embd) return;
  float acc = Y[(size_t)dst * ldy + c];
  for (int j = 0; j < k; ++j) {
    const int ent = ent_of[t * k + j];
    if (ent < 0) continue;   // a choice the plan dropped
    if (ent < e0 || ent >= e1) {
      if (c == 0) set_err(P.err, MOE_ERR_ENTRIES);
      continue;
    }
    acc = acc + O[(size_t)ent * ldo + c];
  }
  Y[(size_t)dst * ldy + c] = acc;
}

// ------------------------------------------------------------------ streaming read ----------

// The achievable-bandwidth reference for the weight streams above: a plain read of a buffer, every
// lane with eight independent 16-byte non-temporal loads in flight per trip, the blocks striding
// over the whole buffer (so every CU reads an equal share). Block b writes the XOR of the 32-bit
// words it read to out[b], which keeps the loads and lets a caller check them.
constexpr int kSrThreads = 256;
__global__ __launch_bounds__(kSrThreads) void k_stream_read(const u32x4* __restrict__ p, uint64_t n16,
                                                            uint32_t* __restrict__ out) {
  const uint64_t stride = (uint64_t)gridDim.x * kSrThreads;
  uint64_t i = (uint64_t)blockIdx.x * kSrThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(p + i + j * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // the block's XOR: a butterfly over the wave, then one word per wave through LDS
  __shared__ uint32_t wx[kSrThreads / 64];
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m);
  if ((threadIdx.x & 63) == 0) wx[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = wx[0] ^ wx[1] ^ wx[2] ^ wx[3];
}

// ------------------------------------------------------------------ host side ---------------

thread_local std::string t_last_error;


int hip_fail(hipError_t e, const char* what) {
  t_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return MOE_E_HIP;
}

// ------------------------------------------------------------------ static scratch ----------

// Workspace of moe_layer_decode_routed_noalloc, for callers that cannot allocate: one array per
// device, held until the process ends. Host code never uses the array's name as an address (on
// the host it is only a stand-in for the symbol); it asks the runtime for the device address once
// per device and passes that pointer on.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kScratchDevices = 64;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// The current device's address of `scratch` (looked up on the first call on each device).
int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices) {
    t_last_error = "device index beyond the scratch table";
    return MOE_E_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) {
      t_last_error = "hipGetSymbolAddress(scratch) gave a null address";
      return MOE_E_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// A layer's format field: the encoding (moe_fmt) with MOE_LAYOUT_PLANAR optionally OR-ed in.
int base_fmt(int f) { return f & ~MOE_LAYOUT_PLANAR; }
bool is_planar(int f) { return (f & MOE_LAYOUT_PLANAR) != 0; }
bool fmt_ok(int f) { return base_fmt(f) >= Q8_0 && base_fmt(f) <= NL4X; }
// Q5_1 (an offset format: its dot product needs the activations' sum fields) is a down format only
bool fmt_ok_gate_up(int f) { return fmt_ok(f) && base_fmt(f) != Q5_1; }

bool cols_ok(int fmt, int n) {
  fmt = base_fmt(fmt);
  if (n <= 0 || n > MOE_MAX_DIM) return false;
  return (fmt == CB2 || fmt == CB3 || fmt == NL4X) ? n % 256 == 0 : n % 64 == 0;
}

int ilog2(int v) {
  int l = 0;
  while ((1 << (l + 1)) <= v) ++l;
  return l;
}

// Lanes per row: among the allowed L whose wave pass (64 / L rows) keeps a chunk within kChunkCap
// bytes (the widest L always qualifies), the best lane utilisation U / (L ceil(U / L)). Gate/up:
// L <= 32 (a pass holds gate and up rows of rp / 2 h rows), ties to the smaller L (longer items);
// down: ties to the larger L (more, smaller row tiles), except that one whose pass holds a whole
// tile of rows_hint rows is kept over those that need two passes.
Geom make_geom(int fmt_field, int ncols, bool gate_up, int rows_hint = 0) {
  const int fmt = base_fmt(fmt_field);
  Geom G{};
  G.U = ncols / 32;
  G.rb = ncols / block_weights(fmt) * block_bytes(fmt);
  G.ly = make_lay(fmt, ncols / block_weights(fmt), is_planar(fmt_field));
  const int Lmax = gate_up ? 32 : 64;
  int bestL = Lmax;
  double best = -1.0;
  bool best_one = false;
  for (int L = 4; L <= Lmax; L <<= 1) {
    const int rp = 64 / L;
    if (rp * G.rb > kChunkCap && L < Lmax) continue;
    const double util = (double)G.U / (double)(L * ((G.U + L - 1) / L));
    const bool one = rows_hint > 0 && rp >= rows_hint;
    const bool better = gate_up ? util > best + 1e-9
                                : util > best + 1e-9 || (util >= best - 1e-9 && (one || !best_one));
    if (better) {
      best = util;
      bestL = L;
      best_one = one;
    }
  }
  G.L = bestL;
  G.lgL = ilog2(bestL);
  G.upl = (G.U + G.L - 1) / G.L;
  G.rp = 64 / G.L;
  return G;
}

int num_cus();

// The down geometry for this device: its tiles hold ceil(n_embd / CUs) rows (at most kDnTileMax).
Geom down_geom(const moe_layer* L) {
  const int tr = std::min(kDnTileMax, std::max(1, (L->n_embd + num_cus() - 1) / num_cus()));
  return make_geom(L->fmt_down, L->n_ff, false, tr);
}

// Slot size in KB: each span (gate rows, then up rows, each in whole KB) plus alignment slack (its
// head offset and 16-byte tail, and the dwords past the end an unaligned read may touch). Two slots
// per wave (the next item streams in while this one computes) where LDS allows, else one.
Stream gu_stream(const Geom& G, int ns) {
  Stream S;
  S.M = 2 * (((G.rp / 2) * G.rb + 48 + 1023) / 1024);
  S.NS = ns;
  return S;
}
Stream dn_stream(const Geom& G, int rc, int ns) {
  Stream S;
  S.M = (rc * G.rb + 48 + 1023) / 1024;
  S.NS = ns;
  return S;
}

// Down tiling: tr rows of Y per tile, the rows spread evenly over `grid` workgroups (at most
// kDnTileMax; a workgroup then takes several tiles), streamed in chunks of rc rows of one group
// (within kChunkCap bytes where a whole wave pass allows).
void dn_tiling(const Geom& G, int n_embd, int grid, int& tr, int& rc) {
  tr = std::min(kDnTileMax, std::max(1, (n_embd + grid - 1) / std::max(grid, 1)));
  rc = std::min(tr, std::max(G.rp, kChunkCap / G.rb / G.rp * G.rp));
}

struct WsLayout {
  size_t lo, hi, d, s, total;
};

size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

// The call's descriptor, then the q8_1 rows of h in split form (row = entry - e0): the 16-byte low
// halves of every block's quants, the high halves, the float scales.
WsLayout ws_layout(const moe_layer* L, const moe_plan* P) {
  WsLayout w{};
  const size_t blocks = (size_t)P->cap_entries * (L->n_ff / 32);
  w.lo = kDescReserve + kCtrBytes;
  w.hi = w.lo + al256(blocks * 16);
  w.d = w.hi + al256(blocks * 16);
  w.s = w.d + al256(blocks * 4);   // the blocks' sum fields (written only for a Q5_1 down matrix)
  w.total = w.s + al256(blocks * 4);
  return w;
}

int check_layer(const moe_layer* L, bool need_down) {
  if (!L || !L->gate || !L->up || (need_down && !L->down)) return MOE_E_ARG;
  if (!fmt_ok_gate_up(L->fmt_gate_up) || !fmt_ok(L->fmt_down)) return MOE_E_FMT;
  if (L->n_experts <= 0) return MOE_E_ARG;
  if (!cols_ok(L->fmt_gate_up, L->n_embd) || !cols_ok(L->fmt_down, L->n_ff)) return MOE_E_SHAPE;
  const int fg = base_fmt(L->fmt_gate_up), fd = base_fmt(L->fmt_down);
  const bool nl4 = fg == NL4 || fd == NL4 || fg == NL4X || fd == NL4X;
  const bool cb2 = fg == CB2 || fd == CB2;
  const bool cb3 = fg == CB3 || fd == CB3;
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
  static int n = 0;
  if (!n) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

// Workgroups for `items` work items: every item gets its own workgroup up to what the CUs hold
// at once (LDS-limited, 8 per CU at most); beyond that workgroups take several items.
// On request (MOE_ROUTE_VERBOSE set in the environment), one line on stderr per distinct kernel
// choice of a launch: its role, weight format and layout, the kernel instance and its launch shape.
const char* fmt_str(int f) {
  static const char* n[] = {"?", "Q8_0", "NL4", "CB2", "CB3", "Q5_1", "NL4X"};
  return n[(f >= 1 && f <= 6) ? f : 0];
}
void note_choice(const char* role, int fmt_field, const char* kernel, const char* mode, int grid, int threads,
                 int lds, const char* extra) {
  static const bool on = getenv("MOE_ROUTE_VERBOSE") != nullptr;
  if (!on) return;
  static std::mutex mu;
  static std::vector<std::string> seen;
  char line[320];
  snprintf(line, sizeof line, "moe_route: %s %s (%s layout) -> %s<%s, %s>: grid %d x %d threads, %d KB LDS%s%s",
           role, fmt_str(base_fmt(fmt_field)), (fmt_field & MOE_LAYOUT_PLANAR) ? "planar" : "row-major", kernel,
           fmt_str(base_fmt(fmt_field)), mode, grid, threads, (lds + 1023) / 1024, extra[0] ? ", " : "", extra);
  std::lock_guard<std::mutex> g(mu);
  if (std::find(seen.begin(), seen.end(), std::string(line)) != seen.end()) return;
  seen.emplace_back(line);
  fprintf(stderr, "%s\n", line);
}

int grid_for(int items, int lds_bytes, int grid_limit) {
  const int per_cu = std::max(1, std::min(8, kLdsMax / std::max(lds_bytes, 1)));
  int grid = std::min(items, num_cus() * per_cu);
  if (grid_limit) grid = std::min(grid, grid_limit);
  return std::max(1, grid);
}

template <class K>
hipError_t allow_smem(K kern, int bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

hipError_t launch_gu(int fmt, int fmt_down, int mode, bool one, const GuArgs& ga, int grid, int bytes,
                     hipStream_t st) {
  auto go = [&](auto kern) -> hipError_t {
    hipError_t e = allow_smem(kern, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kGuThreads), bytes, st, ga.logits, ga.A.nl4, ga.x, ga.A.gate, ga.A.up,
                       ga.T, ga.E, ga.A.n_embd, ga);
    return hipGetLastError();
  };
#define MOE_LY(F, D) \
  case D:            \
    return go(k_gate_up<F, GU_LAYER, D>);
#define MOE_GU(F)                                                            \
  case F:                                                                    \
    if (mode == GU_LAYER) {                                                  \
      switch (fmt_down) { MOE_LY(F, Q8_0) MOE_LY(F, NL4) MOE_LY(F, CB2) MOE_LY(F, CB3) MOE_LY(F, Q5_1) MOE_LY(F, NL4X) } \
      return hipErrorInvalidValue;                                           \
    }                                                                        \
    if (mode == GU_ROUTED && one) return go(k_gate_up<F, GU_ROUTED, F, false, true>); \
    return mode == GU_COMPOSED ? go(k_gate_up<F, GU_COMPOSED>)               \
           : mode == GU_FUSED  ? go(k_gate_up<F, GU_FUSED>)                  \
                               : go(k_gate_up<F, GU_ROUTED>);
  if (ga.regw && fmt == NL4 && mode != GU_LAYER)
    return mode == GU_COMPOSED ? go(k_gate_up<NL4, GU_COMPOSED, NL4, true>)
           : mode == GU_FUSED  ? go(k_gate_up<NL4, GU_FUSED, NL4, true>)
           : one               ? go(k_gate_up<NL4, GU_ROUTED, NL4, true, true>)
                               : go(k_gate_up<NL4, GU_ROUTED, NL4, true>);
  switch (fmt) {
    MOE_GU(Q8_0)
    MOE_GU(NL4)
    MOE_GU(CB2)
    MOE_GU(CB3)
    MOE_GU(NL4X)
  }
#undef MOE_GU
#undef MOE_LY
  return hipErrorInvalidValue;
}

// Workgroups of the one-launch gate/up kernel (format fmt, down format fmt_down) that one CU holds
// at once with `bytes` of dynamic LDS, as the runtime computes it (registers, LDS, waves); 0 if the
// query fails.
int gu_layer_occupancy(int fmt, int fmt_down, int bytes) {
  int nb = 0;
  auto q = [&](auto kern) {
    if (allow_smem(kern, bytes) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, kGuThreads, (size_t)bytes) != hipSuccess)
      nb = 0;
  };
#define MOE_LQ(F, D) \
  case D:            \
    q(k_gate_up<F, GU_LAYER, D>); break;
#define MOE_GQ(F)                                                                                            \
  case F:                                                                                                    \
    switch (fmt_down) { MOE_LQ(F, Q8_0) MOE_LQ(F, NL4) MOE_LQ(F, CB2) MOE_LQ(F, CB3) MOE_LQ(F, Q5_1) MOE_LQ(F, NL4X) } \
    break;
  switch (fmt) {
    MOE_GQ(Q8_0)
    MOE_GQ(NL4)
    MOE_GQ(CB2)
    MOE_GQ(CB3)
    MOE_GQ(NL4X)
  }
#undef MOE_GQ
#undef MOE_LQ
  return nb;
}

hipError_t launch_dn(int fmt, int mode, bool one, const DnArgs& da, int grid, int bytes, hipStream_t st) {
  auto go = [&](auto kern) -> hipError_t {
    hipError_t e = allow_smem(kern, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kDnThreads), bytes, st, da);
    return hipGetLastError();
  };
#define MOE_DN(F) \
  case F:         \
    if (one && mode == DN_DESC) return go(k_down<F, DN_DESC, true>); \
    return mode == DN_DESC ? go(k_down<F, DN_DESC>) : go(k_down<F, DN_PLAN>);
  switch (fmt) {
    MOE_DN(Q8_0)
    MOE_DN(NL4)
    MOE_DN(CB2)
    MOE_DN(CB3)
    MOE_DN(Q5_1)
    MOE_DN(NL4X)
  }
#undef MOE_DN
  return hipErrorInvalidValue;
}

// LDS the gate/up kernel needs for n_tokens activation rows, its stream and how many of its waves
// stream (all 16 when the slots fit, fewer for long rows), or -1 if it does not fit.
int gu_lds(const moe_layer* L, const moe_plan* P, int n_tokens, int mode, Stream* S, int* sw, int* ring,
           int* actb, int* tailb, int* downb) {
  const Geom G = make_geom(L->fmt_gate_up, L->n_embd, true);
  *actb = act_bytes(n_tokens, G.U);
  if (*actb > kGuActMax) return -1;
  // the prologue uses the ring before the stream: routed, the routing waves' scratch; fused, at
  // least one float row of x; layer mode, after the blocks, the down chunks of kDnWaves waves
  int lg = 0;
  *tailb = 0;
  *downb = 0;
  if (mode == GU_ROUTED || mode == GU_LAYER) {
    lg = std::min(n_tokens, kRtWaves) * route_scr_words(L->n_experts) * 4;
    *tailb = gu_tail_bytes(L->n_experts, n_tokens);
  } else if (mode == GU_FUSED) {
    lg = L->n_embd * 4;
  }
  if (mode == GU_LAYER) {
    const Geom Gd = down_geom(L);
    const bool q51 = base_fmt(L->fmt_down) == Q5_1;
    if (act_bytes_kb(P->cap_entries, Gd.U, q51) > kDnActMax) return -1;
    *downb = ly_down_bytes(P->cap_entries, Gd.U, q51);
    int tr, rc;
    dn_tiling(Gd, L->n_embd, num_cus(), tr, rc);
    lg = std::max(lg, kDnWaves * dn_stream(Gd, rc, 1).M * 1024);
  }
  const int avail = kLdsMax - gu_smem_bytes(0, *actb, *tailb + *downb);
  for (int ns = 2; ns >= 1; --ns) {
    *S = gu_stream(G, ns);
    const int per_wave = S->NS * S->M * 1024;
    *sw = std::min(kGuWaves, avail / per_wave);
    if (*sw >= (ns == 2 ? kGuWaves : 1)) {
      *ring = std::max(*sw * per_wave, lg);
      const int b = gu_smem_bytes(*ring, *actb, *tailb + *downb);
      if (b <= kLdsMax) return b;
    }
  }
  return -1;
}

// LDS of the down kernel for chunks of rc rows: two slots per wave where they fit, else one.
int dn_lds(const moe_layer* L, const moe_plan* P, int rc, Stream* S, int* ring, int* actb) {
  const Geom G = down_geom(L);
  *actb = act_bytes_kb(P->cap_entries, G.U, base_fmt(L->fmt_down) == Q5_1);
  if (*actb > kDnActMax) return -1;
  for (int ns = 2; ns >= 1; --ns) {
    *S = dn_stream(G, rc, ns);
    *ring = kDnWaves * S->NS * S->M * 1024;
    const int b = dn_smem_bytes(*ring, *actb);
    if (b <= kLdsMax) return b;
  }
  return -1;
}

// The gate/up kernel of `mode`.
int run_gate_up(hipStream_t st, const moe_layer* L, const moe_plan* P, int mode, const void* act,
                int n_tokens, float* g, float* u, int ld, uint8_t* ws, const float* logits, int T, int k,
                const int32_t* dst_of_token, int entry_base, int grid_limit, float* Y = nullptr,
                int n_rows = 0, int ldy = 0) {
  const Geom G = make_geom(L->fmt_gate_up, L->n_embd, true);
  int ring = 0, actb = 0, sw = 0, tailb = 0, downb = 0;
  Stream S{};
  const int bytes = gu_lds(L, P, n_tokens, mode, &S, &sw, &ring, &actb, &tailb, &downb);
  if (bytes < 0) return MOE_E_SHAPE;
  GuArgs ga{};
  ga.A = layer_args(L);
  ga.P = plan_args(P);
  ga.G = G;
  ga.S = S;
  ga.n_tokens = n_tokens;
  ga.xq = mode == GU_COMPOSED ? (const uint8_t*)act : nullptr;
  ga.x = mode == GU_COMPOSED ? nullptr : (const float*)act;
  ga.g = g;
  ga.u = u;
  ga.ld = ld;
  if (ws) {
    const WsLayout wl = ws_layout(L, P);
    ga.hq_lo = (uint32_t*)(ws + wl.lo);
    ga.hq_hi = (uint32_t*)(ws + wl.hi);
    ga.hq_d = (float*)(ws + wl.d);
    ga.hq_s = base_fmt(L->fmt_down) == Q5_1 ? (float*)(ws + wl.s) : nullptr;
  }
  ga.desc = ws;
  ga.logits = logits;
  ga.T = T;
  ga.E = L->n_experts;
  ga.k = k;
  ga.dst_of_token = dst_of_token;
  ga.entry_base = entry_base;
  ga.lds_ring = ring;
  ga.lds_act = actb;
  ga.sw = sw;
  // register-direct weights: planar NL4 rows of at most kRegUnits units per lane, every wave of
  // the workgroup streaming (the LDS ring then only serves the prologue), groups of at most
  // kRegSlots entries (n_tokens bounds them; larger groups would decode every unit once per pass)
  ga.regw = base_fmt(L->fmt_gate_up) == NL4 && is_planar(L->fmt_gate_up) && G.upl <= kRegUnits &&
            G.U % 8 == 0 && G.rp * 2 * G.U <= std::min(1024, S.NS * S.M * 1024) && sw == kGuWaves &&
            mode != GU_LAYER && n_tokens <= kRegSlots;
  ga.lds_tail = tailb;
  {
    const uint32_t nbk = (uint32_t)(L->n_ff / 32);
    ga.nb_magic = nbk <= 1 ? 0xFFFFFFFFu : (uint32_t)((1ull << 32) / nbk);
  }
  const int items = P->cap_groups * (L->n_ff / 32);
  // one workgroup more than the blocks where the CUs allow: the last one, which writes the plan
  // and the descriptor, then holds no block of its own
  int grid = grid_for(mode == GU_COMPOSED ? items : items + 1, bytes, grid_limit);
  if (mode == GU_LAYER) {
    // every workgroup waits for all the others: at most what the CUs hold at once (the runtime's
    // occupancy for this kernel: registers, LDS and waves; at least one per CU)
    const Geom Gd = down_geom(L);
    ga.Gd = Gd;
    const int resident =
        num_cus() * std::max(1, gu_layer_occupancy(base_fmt(L->fmt_gate_up), base_fmt(L->fmt_down), bytes));
    grid = std::min(std::min(grid_limit ? grid_limit : num_cus(), resident), kLyMaxGrid);
    // one down tile per CU (a smaller grid takes several each)
    dn_tiling(Gd, L->n_embd, num_cus(), ga.trd, ga.rcd);
    const int md = dn_stream(Gd, ga.rcd, 1).M;
    ga.Sd = dn_stream(Gd, ga.rcd, std::max(1, std::min(3, ring / (kDnWaves * md * 1024))));
    ga.Y = Y;
    ga.n_rows = n_rows;
    ga.ldy = ldy;
    ga.ctr = (uint32_t*)(ws + kCtrOff);
    ga.spin_limit = 1 << 22;
  }
  // a routed one-token window over at most 128 experts takes the kernel compiled for it alone
  const bool one = mode == GU_ROUTED && T == 1 && n_tokens == 1 && L->n_experts <= 128 && L->n_embd <= 4096;
  const hipError_t e = launch_gu(base_fmt(L->fmt_gate_up), base_fmt(L->fmt_down), mode, one, ga, grid, bytes, st);
  {
    static const char* mn[] = {"GU_COMPOSED", "GU_FUSED", "GU_ROUTED", "GU_LAYER"};
    char ex[160];
    snprintf(ex, sizeof ex, "%d streaming waves, %d-row passes, %s%s", sw, G.rp,
             ga.regw ? "weights into registers" : "direct-to-LDS ring", one ? ", one-token instance" : "");
    note_choice("gate/up", L->fmt_gate_up, "k_gate_up", mn[mode & 3], grid, kGuThreads, bytes, ex);
  }
  return e == hipSuccess ? MOE_OK : hip_fail(e, "gate/up kernel");
}

int run_down(hipStream_t st, const moe_layer* L, const moe_plan* P, int mode, const uint8_t* ws,
             const uint8_t* hq, float* Y, int n_rows, int ldy, int grid_limit, int n_tokens = 0) {
  const Geom G = down_geom(L);
  // one tile per CU: every CU streams the same share of the down rows
  int tr, rc;
  dn_tiling(G, L->n_embd, num_cus(), tr, rc);
  int ring = 0, actb = 0;
  Stream S{};
  const int bytes = dn_lds(L, P, rc, &S, &ring, &actb);
  if (bytes < 0) return MOE_E_SHAPE;
  DnArgs da{};
  da.A = layer_args(L);
  da.P = plan_args(P);
  da.G = G;
  da.S = S;
  da.desc = ws;
  da.hq = hq;
  if (ws) {
    const WsLayout wl = ws_layout(L, P);
    da.hq_lo = ws + wl.lo;
    da.hq_hi = ws + wl.hi;
    da.hq_d = ws + wl.d;
    da.hq_s = ws + wl.s;
  }
  da.Y = Y;
  da.n_rows = n_rows;
  da.ldy = ldy;
  da.lds_ring = ring;
  da.lds_act = actb;
  da.tr = tr;
  da.rc = rc;
  da.nsub = (tr + rc - 1) / rc;
  da.ntiles = (L->n_embd + tr - 1) / tr;
  const int tiles = (L->n_embd + tr - 1) / tr;
  const int grid = grid_for(tiles, bytes, grid_limit);
  // a one-token call takes the kernel compiled for it alone
  const bool one = mode == DN_DESC && n_tokens == 1;
  const hipError_t e = launch_dn(base_fmt(L->fmt_down), mode, one, da, grid, bytes, st);
  {
    char ex[96];
    snprintf(ex, sizeof ex, "%d-row tiles, %d-row chunks%s", tr, rc, one ? ", one-token instance" : "");
    note_choice("down", L->fmt_down, "k_down", mode == DN_DESC ? "DN_DESC" : "DN_PLAN", grid, kDnThreads, bytes, ex);
  }
  return e == hipSuccess ? MOE_OK : hip_fail(e, "down kernel");
}

// ------------------------------------------------------------------ prompt path (host) ------

int check_plan_pf(const moe_plan* P) {
  if (!P || !P->n_groups || !P->grp_expert || !P->grp_start || !P->ent_src || !P->ent_dst ||
      !P->ent_w || !P->err)
    return MOE_E_ARG;
  if (P->cap_groups < 1 || P->cap_groups > MOE_MAX_PREFILL_GROUPS || P->cap_entries < 1 ||
      P->cap_entries > MOE_MAX_PREFILL_ENTRIES)
    return MOE_E_ARG;
  return MOE_OK;
}

int run_pf_gemm(hipStream_t st, const moe_layer* L, const moe_plan* P, bool down, const void* act,
                int n_act, float* out0, float* out1, long ld) {
  const int fmt = base_fmt(down ? L->fmt_down : L->fmt_gate_up);
  const int rows = down ? L->n_embd : L->n_ff, K = down ? L->n_ff : L->n_embd;
  PfArgs pa{};
  pa.A = layer_args(L);
  pa.P = plan_args(P);
  pa.nmat = down ? 1 : 2;
  pa.rows = rows;
  pa.K = K;
  pa.rb = K / block_weights(fmt) * block_bytes(fmt);
  pa.ly = make_lay(fmt, K / block_weights(fmt), false);
  pa.act = (const uint8_t*)act;
  pa.act_by_entry = down ? 1 : 0;
  pa.n_act = n_act;
  pa.out0 = out0;
  pa.out1 = out1;
  pa.ld = ld;
  const dim3 grid((unsigned)(pa.nmat * ((rows + kPfRows - 1) / kPfRows)), (unsigned)P->cap_groups);
  auto go = [&](auto kern, int lds) -> hipError_t {
    hipError_t e = allow_smem(kern, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kPfThreads), lds, st, pa);
    return hipGetLastError();
  };
  hipError_t e = hipErrorInvalidValue;
  switch (fmt) {
    case Q8_0: e = go(k_pf_gemm<Q8_0>, pf_lds<Q8_0>()); break;
    case NL4: e = go(k_pf_gemm<NL4>, pf_lds<NL4>()); break;
    case CB2: e = go(k_pf_gemm<CB2>, pf_lds<CB2>()); break;
    case CB3: e = go(k_pf_gemm<CB3>, pf_lds<CB3>()); break;
    case Q5_1: e = go(k_pf_gemm<Q5_1>, pf_lds<Q5_1>()); break;
    case NL4X: e = go(k_pf_gemm<NL4X>, pf_lds<NL4X>()); break;
  }
  return e == hipSuccess ? MOE_OK : hip_fail(e, down ? "prefill down kernel" : "prefill gate/up kernel");
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

int moe_repack(void* stream, int fmt, const void* src, int64_t rows, int cols, void* dst, int to_planar) {
  if (!src || !dst || rows < 0 || (to_planar != 0 && to_planar != 1)) return MOE_E_ARG;
  if (!fmt_ok(fmt) || is_planar(fmt)) return MOE_E_FMT;
  if (!cols_ok(fmt, cols)) return MOE_E_SHAPE;
  if (((uintptr_t)src & 1) || ((uintptr_t)dst & 1)) return MOE_E_ARG;
  const int rb = cols / block_weights(fmt) * block_bytes(fmt);
  const uintptr_t a0 = (uintptr_t)src, b0 = (uintptr_t)dst, n = (uintptr_t)rows * (uintptr_t)rb;
  if (rows && a0 < b0 + n && b0 < a0 + n) return MOE_E_ARG;   // the two must not overlap
  if (rows == 0) return MOE_OK;
  const int grid = (int)std::min<int64_t>(rows, 8192);
  const int nblk = cols / block_weights(fmt);
  const hipStream_t st = (hipStream_t)stream;
  const uint16_t* s = (const uint16_t*)src;
  uint16_t* d = (uint16_t*)dst;
  switch (fmt) {
    case Q8_0: hipLaunchKernelGGL(k_repack<Q8_0>, dim3(grid), dim3(kThreads), 0, st, s, d, (long)rows, rb, nblk, to_planar); break;
    case NL4: hipLaunchKernelGGL(k_repack<NL4>, dim3(grid), dim3(kThreads), 0, st, s, d, (long)rows, rb, nblk, to_planar); break;
    case CB2: hipLaunchKernelGGL(k_repack<CB2>, dim3(grid), dim3(kThreads), 0, st, s, d, (long)rows, rb, nblk, to_planar); break;
    case CB3: hipLaunchKernelGGL(k_repack<CB3>, dim3(grid), dim3(kThreads), 0, st, s, d, (long)rows, rb, nblk, to_planar); break;
    case Q5_1: hipLaunchKernelGGL(k_repack<Q5_1>, dim3(grid), dim3(kThreads), 0, st, s, d, (long)rows, rb, nblk, to_planar); break;
    default: hipLaunchKernelGGL(k_repack<NL4X>, dim3(grid), dim3(kThreads), 0, st, s, d, (long)rows, rb, nblk, to_planar); break;
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_repack");
}

int moe_prefill_plan(void* stream, const int32_t* ids, const float* w, const int32_t* dst_of_token, int T,
                     int k, int E, int entry_base, const moe_plan* P, int32_t* ent_of) {
  int rc = check_plan_pf(P);
  if (rc) return rc;
  if (!ids || T < 0 || k < 1 || E < 1 || E > 1024 || entry_base < 0) return MOE_E_ARG;
  const long n = (long)T * k;
  if (n > P->cap_entries || std::min<long>(n, E) > P->cap_groups || n > MOE_MAX_PREFILL_ENTRIES)
    return MOE_E_ARG;
  hipLaunchKernelGGL(k_plan_large, dim3(1), dim3(kPpThreads), 0, (hipStream_t)stream, ids, w, dst_of_token, T,
                     k, E, entry_base, plan_args(P), ent_of);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_prefill_plan");
}

int moe_prefill_gate_up(void* stream, const moe_layer* L, const moe_plan* P, const void* xq, int n_tokens,
                        float* g, float* u, int ld) {
  int rc = check_layer(L, false);
  if (rc) return rc;
  if ((rc = check_plan_pf(P))) return rc;
  if (is_planar(L->fmt_gate_up)) return MOE_E_FMT;
  if (!xq || !g || !u || ld < L->n_ff || n_tokens < 0) return MOE_E_ARG;
  if ((uintptr_t)xq & 3) return MOE_E_ARG;
  return run_pf_gemm((hipStream_t)stream, L, P, false, xq, n_tokens, g, u, ld);
}

int moe_prefill_swiglu_q8_1(void* stream, const moe_plan* P, const float* g, const float* u, int n_ff, int ld,
                            float* h, void* hq) {
  int rc = check_plan_pf(P);
  if (rc) return rc;
  if (!g || !u || !hq || n_ff <= 0 || n_ff % 32 || n_ff > MOE_MAX_DIM || ld < n_ff) return MOE_E_ARG;
  if ((uintptr_t)hq & 3) return MOE_E_ARG;
  const long total = (long)P->cap_entries * (n_ff / 32);
  const int grid = (int)std::max<long>(1, std::min<long>((total + 7) / 8, 8192));
  hipLaunchKernelGGL(k_pf_swiglu, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, plan_args(P), g, u, n_ff,
                     (long)ld, h, (uint8_t*)hq);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_prefill_swiglu_q8_1");
}

int moe_prefill_down(void* stream, const moe_layer* L, const moe_plan* P, const void* hq, float* O, int ldo) {
  int rc = check_layer(L, true);
  if (rc) return rc;
  if ((rc = check_plan_pf(P))) return rc;
  if (is_planar(L->fmt_down)) return MOE_E_FMT;
  if (!hq || !O || ldo < L->n_embd) return MOE_E_ARG;
  if ((uintptr_t)hq & 3) return MOE_E_ARG;
  return run_pf_gemm((hipStream_t)stream, L, P, true, hq, 0, O, nullptr, ldo);
}

int moe_prefill_scatter(void* stream, const moe_plan* P, const int32_t* ent_of, const int32_t* dst_of_token,
                        int T, int k, const float* O, int ldo, int n_embd, float* Y, int n_rows, int ldy) {
  int rc = check_plan_pf(P);
  if (rc) return rc;
  if (!ent_of || !O || !Y || T < 0 || k < 1 || n_embd <= 0 || ldo < n_embd || ldy < n_embd || n_rows < 0)
    return MOE_E_ARG;
  if (T == 0) return MOE_OK;
  const dim3 grid((unsigned)((n_embd + kThreads - 1) / kThreads), (unsigned)T);
  hipLaunchKernelGGL(k_pf_scatter, grid, dim3(kThreads), 0, (hipStream_t)stream, plan_args(P), ent_of,
                     dst_of_token, k, O, (long)ldo, n_embd, Y, n_rows, (long)ldy);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_prefill_scatter");
}

int moe_route_topk(void* stream, const float* logits, int T, int E, int k, int32_t* ids, float* w) {
  if (!logits || !ids || !w || T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > 32)
    return MOE_E_ARG;
  if (T == 0) return MOE_OK;
  hipLaunchKernelGGL(k_route, dim3(T), dim3(64), 0, (hipStream_t)stream, logits, E, k, ids, w);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e, "moe_route_topk");
}

int moe_build_plan(void* stream, const int32_t* ids, const float* w, const int32_t* dst_of_token,
                   int T, int k, int E, int entry_base, const moe_plan* P) {
  int rc = check_plan(P);
  if (rc) return rc;
  if (!ids || !w || T < 0 || k < 1 || E < 1 || entry_base < 0) return MOE_E_ARG;
  if (T * k > P->cap_entries || T * k > P->cap_groups || T * k > 64) return MOE_E_ARG;
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(64), 0, (hipStream_t)stream, ids, w, dst_of_token, T, k, E,
                     entry_base, plan_args(P));
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
  return run_gate_up((hipStream_t)stream, L, P, GU_COMPOSED, xq, n_tokens, g, u, ld, nullptr, nullptr, 0,
                     0, nullptr, 0, grid_limit);
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
  off[0] = w.lo;
  off[1] = w.hi;
  off[2] = w.d;
  return MOE_OK;
}

int moe_down_scatter(void* stream, const moe_layer* L, const moe_plan* P, const void* hq, float* Y,
                     int n_rows, int ldy, int grid_limit) {
  int rc = check_layer(L, true);
  if (rc) return rc;
  if ((rc = check_plan(P))) return rc;
  if (!hq || !Y || n_rows < 0 || ldy < L->n_embd || grid_limit < 0) return MOE_E_ARG;
  if ((uintptr_t)hq & 3) return MOE_E_ARG;
  return run_down((hipStream_t)stream, L, P, DN_PLAN, nullptr, (const uint8_t*)hq, Y, n_rows, ldy,
                  grid_limit);
}

int moe_layer_gate_up(void* stream, const moe_layer* L, const moe_plan* P, const float* logits, int T,
                      int k, const int32_t* dst_of_token, int entry_base, const float* x, int n_tokens,
                      void* ws, size_t ws_bytes, int grid_limit) {
  int rc = check_layer(L, true);
  if (rc) return rc;
  if ((rc = check_plan(P))) return rc;
  if (!x || n_tokens < 0 || grid_limit < 0) return MOE_E_ARG;
  if ((uintptr_t)x & 15) return MOE_E_ARG;
  if (logits) {
    if (T < 1 || T != n_tokens || k < 1 || k > 32 || k > L->n_experts || L->n_experts > 1024 ||
        entry_base < 0)
      return MOE_E_ARG;
    if (T * k > P->cap_entries || T * k > P->cap_groups || T * k > 64) return MOE_E_ARG;
  }
  const WsLayout wl = ws_layout(L, P);
  if (!ws || ws_bytes < wl.total || ((uintptr_t)ws & 255)) return MOE_E_WS;
  uint8_t* b = (uint8_t*)ws;
  return run_gate_up((hipStream_t)stream, L, P, logits ? GU_ROUTED : GU_FUSED, x, n_tokens, nullptr,
                     nullptr, 0, b, logits, T, k, dst_of_token, entry_base, grid_limit);
}

int moe_layer_down(void* stream, const moe_layer* L, const moe_plan* P, const void* ws, size_t ws_bytes,
                   int n_tokens, float* Y, int n_rows, int ldy, int grid_limit) {
  int rc = check_layer(L, true);
  if (rc) return rc;
  if ((rc = check_plan(P))) return rc;
  if (!Y || n_tokens < 0 || n_rows < 0 || ldy < L->n_embd || grid_limit < 0) return MOE_E_ARG;
  const WsLayout wl = ws_layout(L, P);
  if (!ws || ws_bytes < wl.total || ((uintptr_t)ws & 255)) return MOE_E_WS;
  const uint8_t* b = (const uint8_t*)ws;
  return run_down((hipStream_t)stream, L, P, DN_DESC, b, nullptr, Y, n_rows, ldy, grid_limit, n_tokens);
}

int moe_layer_decode(void* stream, const moe_layer* L, const moe_plan* P, const float* x, int n_tokens,
                     float* Y, int n_rows, int ldy, void* ws, size_t ws_bytes, int grid_limit) {
  if (!Y || n_rows < 0 || (L && ldy < L->n_embd)) return MOE_E_ARG;
  const int rc = moe_layer_gate_up(stream, L, P, nullptr, 0, 0, nullptr, 0, x, n_tokens, ws, ws_bytes,
                                   grid_limit);
  if (rc) return rc;
  return moe_layer_down(stream, L, P, ws, ws_bytes, n_tokens, Y, n_rows, ldy, grid_limit);
}

int moe_layer_step(void* stream, const moe_layer* L, const moe_plan* P, const float* logits, int T, int k,
                   const int32_t* dst_of_token, int entry_base, const float* x, float* Y, int n_rows, int ldy,
                   void* ws, size_t ws_bytes, int grid_limit) {
  int rc = check_layer(L, true);
  if (rc) return rc;
  if ((rc = check_plan(P))) return rc;
  if (!logits || !x || !Y || n_rows < 0 || ldy < L->n_embd || grid_limit < 0) return MOE_E_ARG;
  if ((uintptr_t)x & 15) return MOE_E_ARG;
  if (T < 1 || k < 1 || k > 32 || k > L->n_experts || L->n_experts > 1024 || entry_base < 0) return MOE_E_ARG;
  if (T * k > P->cap_entries || T * k > P->cap_groups || T * k > 64) return MOE_E_ARG;
  const WsLayout wl = ws_layout(L, P);
  if (!ws || ws_bytes < wl.total || ((uintptr_t)ws & 255)) return MOE_E_WS;
  return run_gate_up((hipStream_t)stream, L, P, GU_LAYER, x, T, nullptr, nullptr, 0, (uint8_t*)ws, logits, T,
                     k, dst_of_token, entry_base, grid_limit, Y, n_rows, ldy);
}

int moe_layer_decode_routed(void* stream, const moe_layer* L, const moe_plan* P, const float* logits,
                            int T, int k, const int32_t* dst_of_token, int entry_base, const float* x,
                            float* Y, int n_rows, int ldy, void* ws, size_t ws_bytes, int grid_limit) {
  if (!logits || !Y || n_rows < 0 || (L && ldy < L->n_embd)) return MOE_E_ARG;
  const int rc = moe_layer_gate_up(stream, L, P, logits, T, k, dst_of_token, entry_base, x, T, ws,
                                   ws_bytes, grid_limit);
  if (rc) return rc;
  return moe_layer_down(stream, L, P, ws, ws_bytes, T, Y, n_rows, ldy, grid_limit);
}

int moe_layer_decode_routed_noalloc(void* stream, const moe_layer* L, const moe_plan* P, const float* logits,
                                    int T, int k, const int32_t* dst_of_token, int entry_base, const float* x,
                                    float* Y, int n_rows, int ldy, int grid_limit) {
  int rc = check_layer(L, true);
  if (rc) return rc;
  if ((rc = check_plan(P))) return rc;
  // the size check needs no device: an oversize layer is rejected before anything is enqueued
  const size_t need = ws_layout(L, P).total;
  if (need > kScratchBytes) {
    t_last_error = "moe_layer_decode_routed_noalloc: the layer needs " + std::to_string(need) +
                   " bytes of workspace, more than the " + std::to_string(kScratchBytes) + " of the static scratch";
    return MOE_E_WS;
  }
  void* ws = nullptr;
  if ((rc = scratch_ptr(&ws))) return rc;
  return moe_layer_decode_routed(stream, L, P, logits, T, k, dst_of_token, entry_base, x, Y, n_rows, ldy, ws,
                                 kScratchBytes, grid_limit);
}

int moe_stream_read(void* stream, const void* buf, uint64_t bytes, uint32_t* out, int grid) {
  if (!buf || !out || grid < 1 || grid > 65535 || bytes == 0 || (bytes & 15) ||
      ((uintptr_t)buf & 15))
    return MOE_E_ARG;
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(kSrThreads), 0, (hipStream_t)stream, (const u32x4*)buf,
                     bytes >> 4, out);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e, "stream read kernel");
}

}  // extern "C"
