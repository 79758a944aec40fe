// Shared device helpers of the qmoe HIP library (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qmoe.h"

namespace qmoe {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef uint16_t s2u_t __attribute__((ext_vector_type(2)));

enum { ACT_F16 = 0, ACT_BF16 = 1 };

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}
__device__ __forceinline__ float bf16_to_f32(uint32_t bits) {
  return __builtin_bit_cast(float, bits << 16);
}
template <int ACT>
__device__ __forceinline__ float act_to_f32(uint32_t bits) {
  if constexpr (ACT == ACT_F16) return f16_to_f32(bits);
  else return bf16_to_f32(bits);
}
// fp32 -> fp16, round to nearest even (hardware conversion; fp16 denormals kept).
// The empty asm keeps the fp32 value opaque: otherwise a preceding multiply is
// folded into a mixed-precision fma with a +0 addend, which turns a -0
// product into +0.
__device__ __forceinline__ uint16_t f32_to_f16(float v) {
  asm("" : "+v"(v));
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}
// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
// Two fp32 values -> two fp16 (HALF) or bf16 values in one word (a in the
// low half), each rounded to nearest even from its fp32 value by the packed
// hardware conversion.  The empty asm keeps the compiler from fusing a
// producing multiply into a mixed-precision conversion that would round once.
template <bool HALF>
__device__ __forceinline__ uint32_t f32x2_to_16(float a, float b) {
  asm("" : "+v"(a), "+v"(b));
  if constexpr (HALF) return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, h2_t));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, b2_t));
}
__device__ __forceinline__ void store_out(void* out, int dtype, int64_t i, float v) {
  if (dtype == QMOE_F32) ((float*)out)[i] = v;
  else if (dtype == QMOE_F16) ((uint16_t*)out)[i] = f32_to_f16(v);
  else ((uint16_t*)out)[i] = f32_to_bf16(v);
}
template <int OUT>
__device__ __forceinline__ void store_out_t(void* out, int64_t i, float v) {
  if constexpr (OUT == QMOE_F32) ((float*)out)[i] = v;
  else if constexpr (OUT == QMOE_F16) ((uint16_t*)out)[i] = f32_to_f16(v);
  else ((uint16_t*)out)[i] = f32_to_bf16(v);
}

// silu(z) = z / (1 + e^-z) with the hardware exponential and reciprocal
// (each within about an ulp) instead of an IEEE division sequence
__device__ __forceinline__ float silu_f32(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float sigmoid_f32(float z) { return 1.0f / (1.0f + expf(-z)); }
// Element i of an f32 / f16 / bf16 array.
__device__ __forceinline__ float load_act(const void* p, int dtype, int64_t i) {
  if (dtype == QMOE_F32) return ((const float*)p)[i];
  if (dtype == QMOE_F16) return f16_to_f32(((const uint16_t*)p)[i]);
  return bf16_to_f32(((const uint16_t*)p)[i]);
}

// Workgroup barrier that orders LDS only.  __syncthreads() also orders global
// memory, which on gfx9 means waiting for every outstanding vector-memory load
// (vmcnt(0)) -- including prefetches meant to stay in flight across the
// barrier.  Here only LDS traffic (lgkmcnt) is drained before s_barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- LDS-DMA
typedef __attribute__((address_space(3))) void lds_void_t;

// LDS-DMA issue.  Written as inline asm so that the compiler, which cannot
// tell which LDS region a DMA writes, does not drain every outstanding load
// (vmcnt(0)) before each LDS read; the kernels wait for their own transfers
// explicitly.  Extra loads the compiler does not count can only make its own
// waits stricter (loads complete in order).  M0 carries the wave's LDS base;
// lane i writes 16 (or 4) bytes at M0 + i * 16 (or 4).
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_void_t*)p; }
__device__ __forceinline__ void dma_buf16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" :: "s"(lds), "v"(voff), "s"(r)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_glb16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" :: "s"(lds), "v"(src) : "memory", "m0");
}
__device__ __forceinline__ void dma_glb4(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" :: "s"(lds), "v"(src) : "memory", "m0");
}
// The same with a wave-uniform base address in SGPRs and a 32-bit per-lane
// byte offset (one VGPR instead of a 64-bit address per lane).
__device__ __forceinline__ void dma_glb16_s(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" :: "s"(lds), "v"(voff), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_glb4_s(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" :: "s"(lds), "v"(voff), "s"(base)
               : "memory", "m0");
}

// A wave-uniform pointer as one SGPR pair (for operands that must be scalar).
template <typename T>
__device__ __forceinline__ T* sgpr_ptr(T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// s_waitcnt vmcnt(N) leaving the other counters alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// (x & mask) | magic as one v_and_or_b32.  The constants become opaque
// register values (empty asm, no instruction), so the compiler selects the
// three-operand instruction itself instead of an AND and an OR with literal
// operands.  Not written as inline asm: the hazard checks do not see into
// an asm statement, and a matrix instruction that reads its result too early,
// or whose operand it overwrites too soon, then computes with wrong values.
__device__ __forceinline__ uint32_t and_or_b32(uint32_t x, uint32_t mask, uint32_t magic) {
  asm("" : "+s"(mask));
  asm("" : "+v"(magic));
  return (x & mask) | magic;
}

// Byte permute: result byte i = byte sel_i of the 8-byte value {hi:lo}
// (selector 0..3 -> lo, 4..7 -> hi, 12 -> 0x00).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// ---------------------------------------------------------------- MXFP4

// E8M0 block scale 2^(e - 127) as fp32 (e = 0: the subnormal 2^-127; e = 0xFF:
// NaN).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  const uint32_t bits = e == 0 ? 0x00400000u : (e == 255 ? 0x7FC00000u : e << 23);
  return __builtin_bit_cast(float, bits);
}

// Eight E2M1 codes of one tiled word (element i in nibble i, the on-disk byte
// order) -> four packed pairs (2j, 2j+1) in k order, fp16 (ACT_F16) or bf16,
// each value times s: the hardware conversion turns byte j into elements 2j
// (low nibble) and 2j+1.  Exact when every code times s is zero or a normal
// number of the format: always for s = 1 (every E2M1 value is representable
// in both), and for fp16 when s = 2^-13 .. 2^13.
template <int ACT>
__device__ __forceinline__ u4_t fp4x8_pairs_scaled(uint32_t q, float s) {
  if constexpr (ACT == ACT_F16)
    return u4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, s, 0)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, s, 1)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, s, 2)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, s, 3))};
  else
    return u4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 0)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 1)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 2)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 3))};
}
template <int ACT>
__device__ __forceinline__ u4_t fp4x8_pairs(uint32_t q) {
  return fp4x8_pairs_scaled<ACT>(q, 1.0f);
}

// Four small unsigned integers (bytes holding 0..15) -> two packed fp16
// pairs (bytes 0, 1 and 2, 3), exactly.  Read as E4M3 such a byte is c * 2^-9
// (0..7 are the subnormals m * 2^-9, 8..15 the first normal binade
// (8 + m) * 2^-9), so the hardware conversion scaled by 2^9 yields c: one
// instruction per pair instead of a magic-number splice and a subtraction.
template <bool HI>
__device__ __forceinline__ uint32_t u8x2_small_f16(uint32_t t) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(t, 512.0f, HI));
}

// ---------------------------------------------------------------- FP8 E4M3

// Four E4M3 codes (byte i = element i) -> two packed pairs of fp16 (ACT_F16)
// or bf16 values, elements (0, 1) and (2, 3), with the hardware conversion
// at scale 1.  Exact: an E4M3 value has 4 significant bits and its exponent
// range (2^-9 .. 448) lies inside both formats'; 0x7F / 0xFF give NaN.
template <int ACT>
__device__ __forceinline__ u2_t fp8x4_pairs(uint32_t q) {
  if constexpr (ACT == ACT_F16)
    return u2_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q, 1.0f, false)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(q, 1.0f, true))};
  else
    return u2_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, false)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, true))};
}

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x32_{f16,bf16}: D[16x16] += A[16x32] * B[32x16].  Lane l
// supplies row (l % 16) of A and column (l % 16) of B, eight k-values each for
// the k-slot group (l / 16); D element (4 * (l / 16) + r, l % 16) is acc[r].
__device__ __forceinline__ f4_t mfma(h8_t a, h8_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4_t mfma(b8_t a, b8_t b, f4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int ACT> struct ActT;
template <> struct ActT<ACT_F16> { typedef h8_t v8; typedef h2_t v2; };
template <> struct ActT<ACT_BF16> { typedef b8_t v8; typedef b2_t v2; };

template <int ACT>
__device__ __forceinline__ typename ActT<ACT>::v8 as_v8(u4_t u) {
  return __builtin_bit_cast(typename ActT<ACT>::v8, u);
}

// 2-element dot products with fp32 accumulation (v_dot2_f32_{f16,bf16}).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c, int act) {
  if (act == ACT_F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, a), __builtin_bit_cast(b2_t, b), c, false);
}
template <int ACT>
__device__ __forceinline__ float dot2t(uint32_t a, uint32_t b, float c) {
  if constexpr (ACT == ACT_F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, a), __builtin_bit_cast(b2_t, b), c, false);
}

// Work item of block b in a tiled launch.  Blocks are dealt to the 8 XCDs
// round-robin; tile t goes to XCD t % 8, and each XCD runs its tiles'
// n_nt column tiles back to back, so a tile's activation rows stay in one L2
// and every XCD walks the tiles in list order (a plan lists its partial
// tiles last, so a launch ends on its smallest tiles).  False: no work.
__device__ __forceinline__ bool tile_of_block(int b, int n_tiles, int n_nt, int& mt, int& nt) {
  const int x = b & 7, j = b >> 3, q = j / n_nt;
  mt = x + 8 * q;
  nt = j - q * n_nt;
  return mt < n_tiles;
}

// Plan buffer layout (int32 words), see qmoe_moe_plan in qmoe.h.  The tile
// array is sized for the smallest tile height (16), so the layout does not
// depend on bm.
struct PlanLayout {
  int64_t counts, offsets, sorted, tiles, inv, total;
};
__host__ __device__ inline int64_t plan_max_tiles(int64_t P, int E, int bm) {
  return (P < E ? P : E) + P / bm;
}
__host__ __device__ inline PlanLayout plan_layout(int64_t P, int E) {
  PlanLayout L;
  L.counts = 8;
  L.offsets = L.counts + E;
  L.sorted = L.offsets + E + 1;
  L.tiles = (L.sorted + P + 3) & ~(int64_t)3;
  L.inv = L.tiles + 4 * plan_max_tiles(P, E, 16);
  L.total = L.inv + P;
  return L;
}

// Chunk histograms of the plan build follow the layout (pairs per chunk).
constexpr int PLAN_CHUNK = 1024;
__host__ __device__ inline int64_t plan_scratch_words(int64_t P, int E) {
  return ((P + PLAN_CHUNK - 1) / PLAN_CHUNK) * (int64_t)E;
}

// Work-balancing area of a plan for the int4 gathered matmul (plans of at
// least SK_MIN_PAIRS pairs): SK_SLOTS tickets, then SK_SLOTS fp32 partial
// tiles of 80 x 256 accumulators, one per K part of a unit that the matmul
// splits across workgroups.  The plan build zeroes the tickets, header word
// 7 records SK_SLOTS, and every split unit leaves its ticket at zero.
constexpr int SK_SLOTS = 512;
constexpr int SK_PART_FLOATS = 80 * 256;
constexpr int64_t SK_MIN_PAIRS = 2048;
__host__ __device__ inline int64_t plan_sk_offset(int64_t P, int E) {
  return (plan_layout(P, E).total + plan_scratch_words(P, E) + 63) & ~(int64_t)63;
}
__host__ __device__ inline int64_t plan_words(int64_t P, int E) {
  if (P < SK_MIN_PAIRS) return plan_layout(P, E).total + plan_scratch_words(P, E);
  return plan_sk_offset(P, E) + SK_SLOTS + (int64_t)SK_SLOTS * SK_PART_FLOATS;
}

// Whether a plan buffer's header names the call it is used with (tile
// height, tokens, top-k, experts: words 3..6).  A plan built for another
// call has other offsets and tile heights; kernels given one do no work
// rather than read past their arrays.
__device__ __forceinline__ bool plan_matches(const int32_t* plan, int bm, int64_t t, int topk, int E) {
  return plan[3] == bm && plan[4] == (int32_t)t && plan[5] == topk && plan[6] == E;
}

}  // namespace qmoe
