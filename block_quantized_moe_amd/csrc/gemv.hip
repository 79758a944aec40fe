// Decode GEMV for a handful of tokens routed to their top-k experts.
//
// The Everything Bagel 2 page's expert-indexed int4 GEMV reads the expert id
// on the device to pick a slab of the stacked [nExperts, outDim, inDim/8]
// weights; the DSV4 campaign page adds a small-batch qgemv and a "sum-folded"
// q2_K down projection that fuses the GEMV with the top-k weighted sum.
//
// Two kernels, both bandwidth bound (every weight byte is read once per call):
//  * gemv_rows_kernel (STORE / SWIGLU): one workgroup per (distinct expert,
//    block of output rows).  A workgroup whose slot repeats an earlier slot's
//    expert exits; the first one serves every token routed to that expert, so
//    the weights stream once.  Lanes split K in 32-value chunks (a row of
//    K = 2048 is one 16-byte load per lane), activations sit in registers, and
//    dot2 instructions accumulate in fp32; a butterfly over the lanes of a row
//    finishes each dot product.
//  * gemv_combine_kernel (WEIGHTED_COMBINE): one workgroup per block of output
//    rows; its four waves share out the distinct experts, each wave loads its
//    tokens' activations once and walks the block's rows, keeps per-token
//    partial sums in LDS, and the waves' sums are added in a fixed order, so
//    the result is bit-reproducible.
// Integer codes are fed to the dot products exactly (as fp16 / bf16 values
// with a known offset) and the per-block scale and bias are applied to the
// fp32 partial sums.
#include <type_traits>

#include "common.h"

namespace qmoe {

constexpr int GV_MAXT = 4;  // tokens per pass over the weights
constexpr int GV_MAX_K = 8192;  // longest reduction: 4 chunks of 32 per lane
// Unit passes of gemv_rows_kernel whose weight loads are issued together: two
// when the batch still leaves room for several waves per SIMD (one token per
// pass, or formats with at most 16 code bytes per chunk), else one (always
// one with four chunks per lane).
__host__ __device__ constexpr int gr_load(int fmt, int mt, int cpl) {
  return cpl > 2 ? 1 : (mt == 1 || fmt == QMOE_MXFP4 || fmt == QMOE_IQ2_XXS || fmt == QMOE_INT4) ? 2 : 1;
}

struct GemvArgs {
  const void* qs;
  const void* aux;
  const void* scales;
  const void* biases;
  const void* d;
  const void* dmin;
  const uint8_t* grid;
  const uint8_t* signs;
  int64_t N, K;
  int group;
  int E, topk, nslots;
  const uint16_t* a;
  const int32_t* ids;
  const float* topk_w;
  void* out;
  int out_dtype;
  int lpr;        // lanes per row (a power of two, at most 64)
  int chunks;     // 32-value chunks per row (K / 32); lane li takes li, li + lpr, ... below it
  int units_per_wg;
};

// Activations of one 32-value chunk: 16 packed pairs plus the sums of its two
// 16-value halves (in fp32).
struct XChunk {
  uint32_t p[16];
  float s0, s1;
};

// The half sums are formed only for the formats whose arithmetic uses them
// (int4 bias, Q2_K mins): forming them makes the kernel wait for the
// activations before it issues its weight loads.
template <int FMT>
__host__ __device__ constexpr bool needs_x_sums() {
  return FMT == QMOE_INT4 || FMT == QMOE_Q2_K || FMT == QMOE_Q4_K || FMT == QMOE_Q6_K;
}

template <int ACT, bool SUMS>
__device__ __forceinline__ void load_x(const uint16_t* src, XChunk& x) {
  const u4_t* v = (const u4_t*)src;
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u4_t q = v[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x.p[4 * i + j] = q[j];
      if constexpr (SUMS) {
        const float a = act_to_f32<ACT>(q[j] & 0xFFFFu) + act_to_f32<ACT>(q[j] >> 16);
        if (i < 2) s0 += a; else s1 += a;
      }
    }
  }
  x.s0 = s0;
  x.s1 = s1;
}

template <int ACT> struct Magic;
template <> struct Magic<ACT_F16> { static constexpr uint32_t bits = 0x64006400u; static constexpr float v = 1024.f; static constexpr uint32_t byte = 0x64646464u; };
template <> struct Magic<ACT_BF16> { static constexpr uint32_t bits = 0x43004300u; static constexpr float v = 128.f; static constexpr uint32_t byte = 0x43434343u; };

// Exact conversion of four signed bytes to two packed pairs (fp16 or bf16).
template <int ACT>
__device__ __forceinline__ void i8x4_pairs(uint32_t w, uint32_t& p0, uint32_t& p1) {
  uint32_t o[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float lo = (float)(int8_t)((w >> (16 * h)) & 0xFFu);
    const float hi = (float)(int8_t)((w >> (16 * h + 8)) & 0xFFu);
    if constexpr (ACT == ACT_F16) o[h] = (uint32_t)f32_to_f16(lo) | ((uint32_t)f32_to_f16(hi) << 16);
    else o[h] = (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
  }
  p0 = o[0];
  p1 = o[1];
}

// The weight bytes of one 32-value chunk (global row R, chunk c), as loaded:
// codes and the per-block metadata, unpacked later by chunk_math.  Loading
// and arithmetic are separate so a kernel can put the loads of several rows
// in flight before the first dot product.
struct ChunkRaw {
  u4_t q0, q1;
  u4_t q2, q3;  // Q6_K: the codes' top bit pairs
  uint32_t m0, m1, m2, m3;
};

template <int FMT>
__device__ __forceinline__ ChunkRaw chunk_load(const GemvArgs& g, int64_t R, int64_t c) {
  const int64_t K = g.K;
  ChunkRaw w;
  if constexpr (FMT == QMOE_INT4) {
    // Tiled layout: chunk c of row R is lane groups 2(c&1), 2(c&1)+1 of tile (R/16, c/2).
    const int64_t rb = R >> 4, rr = R & 15;
    const uint32_t* tile = (const uint32_t*)g.qs + (rb * (K / 64) + (c >> 1)) * 128;
    const u2_t qa = *(const u2_t*)(tile + (32 * (c & 1) + rr) * 2);
    const u2_t qb = *(const u2_t*)(tile + (32 * (c & 1) + 16 + rr) * 2);
    w.q0 = u4_t{qa[0], qa[1], qb[0], qb[1]};
    w.m0 = ((const uint32_t*)g.scales)[(rb * (K / g.group) + (32 * c) / g.group) * 16 + rr];
  } else if constexpr (FMT == QMOE_Q8_0) {
    // tiled layout: chunks 2(c&1), 2(c&1)+1 of k tile c/2, 16 bytes each per row
    const int64_t rb = R >> 4, rr = R & 15;
    const int8_t* base = (const int8_t*)g.qs + (((rb * (K / 64) + (c >> 1)) * 4 + 2 * (c & 1)) * 16 + rr) * 16;
    w.q0 = *(const u4_t*)base;
    w.q1 = *(const u4_t*)(base + 256);
    w.m0 = ((const uint16_t*)g.scales)[(rb * (K / 32) + c) * 16 + rr];
  } else if constexpr (FMT == QMOE_FP8) {
    // codes tiled like Q8_0: chunks 2(c&1), 2(c&1)+1 of k tile c/2; one
    // fp32 scale per 128 x 128 block
    const int64_t rb = R >> 4, rr = R & 15;
    const uint8_t* base = (const uint8_t*)g.qs + (((rb * (K / 64) + (c >> 1)) * 4 + 2 * (c & 1)) * 16 + rr) * 16;
    w.q0 = *(const u4_t*)base;
    w.q1 = *(const u4_t*)(base + 256);
    w.m0 = __builtin_bit_cast(uint32_t, ((const float*)g.scales)[(R >> 7) * (K >> 7) + (c >> 2)]);
  } else if constexpr (FMT == QMOE_MXFP4) {
    // tiled layout: chunk c is block c&1 of k tile c/2, 16 bytes per row
    const int64_t rb = R >> 4, rr = R & 15;
    w.q0 = *(const u4_t*)((const uint32_t*)g.qs + (((rb * (K / 64) + (c >> 1)) * 2 + (c & 1)) * 16 + rr) * 4);
    w.m0 = ((const uint8_t*)g.scales)[(rb * (K / 32) + c) * 16 + rr];
  } else if constexpr (FMT == QMOE_Q2_K) {
    // tiled layout: t = (R/16) * (K/256) + super-block, row r = R % 16
    const int64_t t = (R >> 4) * (K / 256) + c / 8, r = R & 15;
    const int cc = (int)(c & 7);
    const uint8_t* qb = (const uint8_t*)g.qs + ((t * 2 + (cc >> 2)) * 16 + r) * 32;
    w.q0 = *(const u4_t*)qb;
    w.q1 = *(const u4_t*)(qb + 16);
    w.m0 = ((const uint8_t*)g.scales)[(t * 16 + r) * 16 + 2 * cc];
    w.m1 = ((const uint8_t*)g.scales)[(t * 16 + r) * 16 + 2 * cc + 1];
    w.m2 = ((const uint16_t*)g.d)[t * 16 + r];
    w.m3 = ((const uint16_t*)g.dmin)[t * 16 + r];
  } else if constexpr (FMT == QMOE_Q4_K) {
    // chunk c = sub-block j = c%8 of super-block c/8: bytes 0..31 of quarter
    // j/2 of row r, low nibbles for even j, high for odd
    const int64_t t = (R >> 4) * (K / 256) + c / 8, r = R & 15;
    const int j = (int)(c & 7);
    const uint8_t* qb = (const uint8_t*)g.qs + ((t * 4 + (j >> 1)) * 16 + r) * 32;
    w.q0 = *(const u4_t*)qb;
    w.q1 = *(const u4_t*)(qb + 16);
    const uint8_t* sm = (const uint8_t*)g.scales + (t * 16 + r) * 16;
    w.m0 = sm[j];
    w.m1 = sm[8 + j];
    w.m2 = ((const uint16_t*)g.d)[t * 16 + r];
    w.m3 = ((const uint16_t*)g.dmin)[t * 16 + r];
  } else if constexpr (FMT == QMOE_Q6_K) {
    // chunk c = sub-blocks 2j, 2j+1 (j = c%8) of super-block c/8: low bits as
    // Q4_K's codes, top bit pairs from bytes 0..31 of half j/4 at bits 2 (j%4)
    const int64_t t = (R >> 4) * (K / 256) + c / 8, r = R & 15;
    const int j = (int)(c & 7);
    const uint8_t* qb = (const uint8_t*)g.qs + ((t * 4 + (j >> 1)) * 16 + r) * 32;
    const uint8_t* hb = (const uint8_t*)g.aux + ((t * 2 + (j >> 2)) * 16 + r) * 32;
    w.q0 = *(const u4_t*)qb;
    w.q1 = *(const u4_t*)(qb + 16);
    w.q2 = *(const u4_t*)hb;
    w.q3 = *(const u4_t*)(hb + 16);
    const uint8_t* sc = (const uint8_t*)g.scales + (t * 16 + r) * 16;
    w.m0 = sc[2 * j];
    w.m1 = sc[2 * j + 1];
    w.m2 = ((const uint16_t*)g.d)[t * 16 + r];
  } else {  // IQ2_XXS: chunk c is group c%8 of super-block c/8 (tiled layout)
    const int64_t t = (R >> 4) * (K / 256) + c / 8, r = R & 15;
    const int G = (int)(c & 7);
    const u2_t ia = *(const u2_t*)((const uint32_t*)g.qs + ((t * 8 + G) * 16 + r) * 2);
    w.m0 = ia[0];
    w.m1 = ia[1];
    w.m2 = ((const uint16_t*)g.d)[t * 16 + r];
  }
  return w;
}

// Dot products of one loaded chunk (chunk c) with the activations of nt
// tokens; results added to res[].
template <int FMT, int ACT, int MT>
__device__ __forceinline__ void chunk_math(const GemvArgs& g, const ChunkRaw& w, int64_t c, const XChunk* x,
                                           int nt, float* res, const uint32_t* lut_grid,
                                           const uint32_t* lut_sign) {
  if constexpr (FMT == QMOE_INT4) {
    const float s = f16_to_f32(w.m0 & 0xFFFFu);
    const float b = f16_to_f32(w.m0 >> 16);
    uint32_t cp[16];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) cp[4 * q + i] = ((w.q0[q] >> (4 * i)) & 0x000F000Fu) | Magic<ACT>::bits;
    const float cb = b - Magic<ACT>::v * s;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t < nt) {
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) p = dot2t<ACT>(x[t].p[i], cp[i], p);
        res[t] += s * p + cb * (x[t].s0 + x[t].s1);
      }
    }
  } else if constexpr (FMT == QMOE_Q8_0 || FMT == QMOE_FP8 || FMT == QMOE_MXFP4) {
    uint32_t cp[16];
    float dd;
    if constexpr (FMT == QMOE_Q8_0) {
      dd = f16_to_f32(w.m0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        i8x4_pairs<ACT>(w.q0[q], cp[2 * q], cp[2 * q + 1]);
        i8x4_pairs<ACT>(w.q1[q], cp[8 + 2 * q], cp[8 + 2 * q + 1]);
      }
    } else if constexpr (FMT == QMOE_FP8) {
      dd = __builtin_bit_cast(float, w.m0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u2_t p0 = fp8x4_pairs<ACT>(w.q0[q]), p1 = fp8x4_pairs<ACT>(w.q1[q]);
        cp[2 * q] = p0[0];
        cp[2 * q + 1] = p0[1];
        cp[8 + 2 * q] = p1[0];
        cp[8 + 2 * q + 1] = p1[1];
      }
    } else {
      dd = e8m0_to_f32(w.m0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u4_t p = fp4x8_pairs<ACT>(w.q0[q]);
#pragma unroll
        for (int i = 0; i < 4; ++i) cp[4 * q + i] = p[i];
      }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t < nt) {
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) p = dot2t<ACT>(x[t].p[i], cp[i], p);
        res[t] += dd * p;
      }
    }
  } else if constexpr (FMT == QMOE_Q2_K) {
    const int cc = (int)(c & 7);
    const uint32_t shift = 2u * (uint32_t)(cc & 3);
    const uint32_t sc0 = w.m0, sc1 = w.m1;
    const float d = f16_to_f32(w.m2);
    const float dm = f16_to_f32(w.m3);
    const float dl0 = d * (float)(sc0 & 15u), ml0 = dm * (float)(sc0 >> 4);
    const float dl1 = d * (float)(sc1 & 15u), ml1 = dm * (float)(sc1 >> 4);
    uint32_t cp[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t t0 = (w.q0[q] >> shift) & 0x03030303u;
      const uint32_t t1 = (w.q1[q] >> shift) & 0x03030303u;
      cp[2 * q] = perm_b32(Magic<ACT>::byte, t0, 0x04010400u) & 0xFF03FF03u;
      cp[2 * q + 1] = perm_b32(Magic<ACT>::byte, t0, 0x04030402u) & 0xFF03FF03u;
      cp[8 + 2 * q] = perm_b32(Magic<ACT>::byte, t1, 0x04010400u) & 0xFF03FF03u;
      cp[8 + 2 * q + 1] = perm_b32(Magic<ACT>::byte, t1, 0x04030402u) & 0xFF03FF03u;
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t < nt) {
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p0 = dot2t<ACT>(x[t].p[i], cp[i], p0);
          p1 = dot2t<ACT>(x[t].p[8 + i], cp[8 + i], p1);
        }
        res[t] += dl0 * (p0 - Magic<ACT>::v * x[t].s0) - ml0 * x[t].s0 +
                  dl1 * (p1 - Magic<ACT>::v * x[t].s1) - ml1 * x[t].s1;
      }
    }
  } else if constexpr (FMT == QMOE_Q4_K) {
    // value = d sc q - dmin m over the whole chunk (one sub-block)
    const uint32_t shift = 4u * (uint32_t)(c & 1);
    const float dl = f16_to_f32(w.m2) * (float)w.m0;
    const float ml = f16_to_f32(w.m3) * (float)w.m1;
    uint32_t cp[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t t0 = (w.q0[q] >> shift) & 0x0F0F0F0Fu;
      const uint32_t t1 = (w.q1[q] >> shift) & 0x0F0F0F0Fu;
      cp[2 * q] = perm_b32(Magic<ACT>::byte, t0, 0x04010400u);
      cp[2 * q + 1] = perm_b32(Magic<ACT>::byte, t0, 0x04030402u);
      cp[8 + 2 * q] = perm_b32(Magic<ACT>::byte, t1, 0x04010400u);
      cp[8 + 2 * q + 1] = perm_b32(Magic<ACT>::byte, t1, 0x04030402u);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t < nt) {
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) p = dot2t<ACT>(x[t].p[i], cp[i], p);
        const float xs = x[t].s0 + x[t].s1;
        res[t] += dl * (p - Magic<ACT>::v * xs) - ml * xs;
      }
    }
  } else if constexpr (FMT == QMOE_Q6_K) {
    // value = d sc (q - 32) per 16-value half, each half with its own scale
    const uint32_t sn = 4u * (uint32_t)(c & 1), sh = 2u * (uint32_t)(c & 3);
    const float d = f16_to_f32(w.m2);
    const float d0 = d * (float)(int8_t)w.m0, d1 = d * (float)(int8_t)w.m1;
    uint32_t cp[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t t0 = ((w.q0[q] >> sn) & 0x0F0F0F0Fu) | (((w.q2[q] >> sh) & 0x03030303u) << 4);
      const uint32_t t1 = ((w.q1[q] >> sn) & 0x0F0F0F0Fu) | (((w.q3[q] >> sh) & 0x03030303u) << 4);
      cp[2 * q] = perm_b32(Magic<ACT>::byte, t0, 0x04010400u);
      cp[2 * q + 1] = perm_b32(Magic<ACT>::byte, t0, 0x04030402u);
      cp[8 + 2 * q] = perm_b32(Magic<ACT>::byte, t1, 0x04010400u);
      cp[8 + 2 * q + 1] = perm_b32(Magic<ACT>::byte, t1, 0x04030402u);
    }
    constexpr float off = Magic<ACT>::v + 32.0f;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t < nt) {
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p0 = dot2t<ACT>(x[t].p[i], cp[i], p0);
          p1 = dot2t<ACT>(x[t].p[8 + i], cp[8 + i], p1);
        }
        res[t] += d0 * (p0 - off * x[t].s0) + d1 * (p1 - off * x[t].s1);
      }
    }
  } else {  // IQ2_XXS
    const uint32_t idx = w.m0;
    const uint32_t aux = w.m1;
    const float db = f16_to_f32(w.m2) * (0.5f + (float)(aux >> 28)) * 0.25f;
    uint32_t cp[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u4_t row = *(const u4_t*)(lut_grid + 4 * ((idx >> (8 * j)) & 0xFFu));
      const u4_t msk = *(const u4_t*)(lut_sign + 4 * ((aux >> (7 * j)) & 0x7Fu));
#pragma unroll
      for (int i = 0; i < 4; ++i) cp[4 * j + i] = row[i] ^ msk[i];
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t < nt) {
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) p = dot2t<ACT>(x[t].p[i], cp[i], p);
        res[t] += db * p;
      }
    }
  }
}

template <int FMT, int ACT, int MT>
__device__ __forceinline__ void chunk_dot(const GemvArgs& g, int64_t R, int64_t c, const XChunk* x,
                                          int nt, float* res, const uint32_t* lut_grid,
                                          const uint32_t* lut_sign) {
  chunk_math<FMT, ACT, MT>(g, chunk_load<FMT>(g, R, c), c, x, nt, res, lut_grid, lut_sign);
}

template <int ACT>
__device__ __forceinline__ void build_iq2_luts(const uint8_t* grid, const uint8_t* signs,
                                               uint32_t* lut_grid, uint32_t* lut_sign) {
  const int tid = threadIdx.x;
  {
    const u2_t b = *(const u2_t*)(grid + 8 * tid);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = b[i >> 1] >> (16 * (i & 1));
      const float lo = (float)(w & 0xFFu), hi = (float)((w >> 8) & 0xFFu);
      uint32_t packed;
      if constexpr (ACT == ACT_F16) packed = (uint32_t)f32_to_f16(lo) | ((uint32_t)f32_to_f16(hi) << 16);
      else packed = (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
      lut_grid[4 * tid + i] = packed;
    }
  }
  if (tid < 128) {
    const uint32_t m = signs[tid];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lut_sign[4 * tid + i] = (((m >> (2 * i)) & 1u) << 15) | (((m >> (2 * i + 1)) & 1u) << 31);
  }
}

// Butterfly sum over the `lpr` lanes that share a row.
__device__ __forceinline__ float row_reduce(float v, int lpr) {
  for (int off = lpr >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// STORE / SWIGLU.  grid = (row blocks, slots).
template <int FMT, int ACT, int EPI, int CPL, int MT>
__global__ __launch_bounds__(256) void gemv_rows_kernel(GemvArgs g) {
  constexpr bool IQ2 = (FMT == QMOE_IQ2_XXS);
  __shared__ __attribute__((aligned(16))) uint32_t lut_grid[IQ2 ? 256 * 4 : 4];
  __shared__ __attribute__((aligned(16))) uint32_t lut_sign[IQ2 ? 128 * 4 : 4];
  __shared__ int list[QMOE_MAX_GEMV_BATCH * QMOE_MAX_TOPK];
  __shared__ int nlist, dup;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = blockIdx.y;
  const int e = g.ids[slot];
  if (e < 0 || e >= g.E) return;
  if (tid == 0) { nlist = 0; dup = 0; }
  if constexpr (IQ2) build_iq2_luts<ACT>(g.grid, g.signs, lut_grid, lut_sign);
  __syncthreads();
  for (int p = tid; p < g.nslots; p += 256) {
    if (g.ids[p] == e) {
      if (p < slot) dup = 1;
      else list[atomicAdd(&nlist, 1)] = p;
    }
  }
  __syncthreads();
  if (dup) return;
  const int n = nlist;

  const int lpr = g.lpr;
  const int rpw = 64 / lpr;                 // row units per wave pass
  const int sub = lane / lpr, li = lane % lpr;
  constexpr bool swiglu = (EPI == QMOE_EPI_SWIGLU);
  const int64_t Nunits = swiglu ? g.N / 2 : g.N;
  const int64_t u0 = (int64_t)blockIdx.x * g.units_per_wg;

  for (int tb = 0; tb < n; tb += MT) {
    const int nt = min(MT, n - tb);
    XChunk x[MT][CPL];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t < nt) {
        const int s2 = list[tb + t];
        const uint16_t* xr = g.a + (int64_t)(s2 / g.topk) * g.K;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          load_x<ACT, needs_x_sums<FMT>()>(xr + 32 * (int64_t)min(li + c * lpr, g.chunks - 1), x[t][c]);
      }
    }
    // GR_LOAD unit passes at a time (units_per_wg is a multiple of
    // GR_LOAD * 4 * rpw): every weight load of the batch is issued before the
    // first dot product
    constexpr int NR = swiglu ? 2 : 1;  // weight rows per unit (gate, up)
    constexpr int GR_LOAD = gr_load(FMT, MT, CPL);
    for (int ub0 = wave * rpw; ub0 < g.units_per_wg; ub0 += GR_LOAD * 4 * rpw) {
      ChunkRaw wr[GR_LOAD][NR][CPL];
#pragma unroll
      for (int i = 0; i < GR_LOAD; ++i) {
        const int64_t unit = u0 + ub0 + i * 4 * rpw + sub;
        const int64_t Rg = (int64_t)e * g.N + (unit < Nunits ? unit : 0);
#pragma unroll
        for (int h = 0; h < NR; ++h)
#pragma unroll
          for (int c = 0; c < CPL; ++c) wr[i][h][c] = chunk_load<FMT>(g, Rg + h * (g.N / 2), min(li + c * lpr, g.chunks - 1));
      }
#pragma unroll
      for (int i = 0; i < GR_LOAD; ++i) {
        const int64_t unit = u0 + ub0 + i * 4 * rpw + sub;
        const bool valid = unit < Nunits;
        float r0[MT], r1[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) { r0[t] = 0.f; r1[t] = 0.f; }
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          if (li + c * lpr >= g.chunks) continue;  // lanes past the row's last chunk
          XChunk xc[MT];
#pragma unroll
          for (int t = 0; t < MT; ++t) xc[t] = x[t][c];
          chunk_math<FMT, ACT, MT>(g, wr[i][0][c], li + c * lpr, xc, nt, r0, lut_grid, lut_sign);
          if constexpr (swiglu) chunk_math<FMT, ACT, MT>(g, wr[i][NR - 1][c], li + c * lpr, xc, nt, r1, lut_grid, lut_sign);
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          if (t < nt) {
            const float y0 = row_reduce(r0[t], lpr);
            const float y1 = swiglu ? row_reduce(r1[t], lpr) : 0.f;
            if (valid && li == 0) {
              const int s2 = list[tb + t];
              if (swiglu) store_out(g.out, g.out_dtype, (int64_t)s2 * Nunits + unit, silu_f32(y0) * y1);
              else store_out(g.out, g.out_dtype, (int64_t)s2 * Nunits + unit, y0);
            }
          }
        }
      }
    }
  }
}

// WEIGHTED_COMBINE (sum-folded down projection).  grid = row blocks of
// GC_ITERS wave passes (GC_ITERS * 64 / lpr rows).  A wave takes distinct
// experts; for each it loads the activation chunks of up to MT of the tokens
// routed there once and then walks the block's rows with them (the row loop
// is unrolled, so the weight loads of several rows are in flight together).
// Per-token partial sums sit in LDS per wave and are added in wave order, so
// the result is bit-reproducible.
constexpr int GC_ITERS = 8;
// row passes whose weight loads are issued together (one with four chunks per lane)
__host__ __device__ constexpr int gc_load(int cpl) { return cpl > 2 ? 1 : 4; }
constexpr int GC_ROWS = GC_ITERS * 4;  // rows per block at most (lpr >= 16)

template <int FMT, int ACT, int CPL, int MT>
__global__ __launch_bounds__(256) void gemv_combine_kernel(GemvArgs g) {
  constexpr bool IQ2 = (FMT == QMOE_IQ2_XXS);
  __shared__ __attribute__((aligned(16))) uint32_t lut_grid[IQ2 ? 256 * 4 : 4];
  __shared__ __attribute__((aligned(16))) uint32_t lut_sign[IQ2 ? 128 * 4 : 4];
  __shared__ int sid[QMOE_MAX_GEMV_BATCH * QMOE_MAX_TOPK];
  __shared__ int minslot[QMOE_MAX_EXPERTS];
  __shared__ int dlist[QMOE_MAX_GEMV_BATCH * QMOE_MAX_TOPK];
  __shared__ int ndist;
  __shared__ float part[4][QMOE_MAX_GEMV_BATCH][GC_ROWS];  // [wave][token][row in block]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = g.nslots;
  if constexpr (IQ2) build_iq2_luts<ACT>(g.grid, g.signs, lut_grid, lut_sign);
  for (int p = tid; p < P; p += 256) sid[p] = g.ids[p];
  for (int i = tid; i < 4 * QMOE_MAX_GEMV_BATCH * GC_ROWS; i += 256) (&part[0][0][0])[i] = 0.f;
  for (int i = tid; i < g.E; i += 256) minslot[i] = P;
  __syncthreads();
  // the first slot of each expert: the smallest slot index naming it
  for (int p = tid; p < P; p += 256) {
    const int e = sid[p];
    if (e >= 0 && e < g.E) atomicMin(&minslot[e], p);
  }
  __syncthreads();
  if (wave == 0) {  // ordered compaction of first occurrences, 64 slots per ballot (P <= 512)
    int base = 0;
    for (int p0 = 0; p0 < P; p0 += 64) {
      const int p = p0 + lane;
      const int e = p < P ? sid[p] : -1;
      const bool f = e >= 0 && e < g.E && minslot[e] == p;
      const uint64_t m = __ballot(f);
      if (f) dlist[base + __popcll(m & ((1ull << lane) - 1ull))] = p;
      base += __popcll(m);
    }
    if (lane == 0) ndist = base;
  }
  __syncthreads();

  const int lpr = g.lpr;
  const int rpw = 64 / lpr;
  const int sub = lane / lpr, li = lane % lpr;
  const int rows_blk = GC_ITERS * rpw;
  const int64_t n0 = (int64_t)blockIdx.x * rows_blk;

  for (int di = wave; di < ndist; di += 4) {
    const int e = sid[dlist[di]];
    // tokens routed to e, in slot order, MT at a time
    int pos = dlist[di];
    while (pos < P) {
      int sl[MT];
      int nt = 0;
      while (pos < P && nt < MT) {
        if (sid[pos] == e) sl[nt++] = pos;
        ++pos;
      }
      if (nt == 0) break;
      XChunk xc[CPL][MT];
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int t = 0; t < MT; ++t)
          if (t < nt)
            load_x<ACT, needs_x_sums<FMT>()>(g.a + (int64_t)sl[t] * g.K + 32 * (int64_t)min(li + c * lpr, g.chunks - 1),
                                             xc[c][t]);
      constexpr int GC_LOAD = gc_load(CPL);
#pragma unroll
      for (int i0 = 0; i0 < GC_ITERS; i0 += GC_LOAD) {
        // the weight chunks of GC_LOAD row passes, all loads issued first
        ChunkRaw wr[GC_LOAD][CPL];
#pragma unroll
        for (int i = 0; i < GC_LOAD; ++i) {
          const int64_t row = n0 + (i0 + i) * rpw + sub;
          const int64_t Rg = (int64_t)e * g.N + (row < g.N ? row : g.N - 1);
#pragma unroll
          for (int c = 0; c < CPL; ++c) wr[i][c] = chunk_load<FMT>(g, Rg, min(li + c * lpr, g.chunks - 1));
        }
#pragma unroll
        for (int i = 0; i < GC_LOAD; ++i) {
          float r[MT];
#pragma unroll
          for (int t = 0; t < MT; ++t) r[t] = 0.f;
#pragma unroll
          for (int c = 0; c < CPL; ++c)
            if (li + c * lpr < g.chunks) chunk_math<FMT, ACT, MT>(g, wr[i][c], li + c * lpr, xc[c], nt, r, lut_grid, lut_sign);
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            if (t < nt) {
              const float y = row_reduce(r[t], lpr);
              if (li == 0) {
                const int s2 = sl[t];
                part[wave][s2 / g.topk][(i0 + i) * rpw + sub] += g.topk_w[s2] * y;
              }
            }
          }
        }
      }
    }
  }
  __syncthreads();
  const int btok = P / g.topk;
  for (int i = tid; i < btok * rows_blk; i += 256) {
    const int b = i / rows_blk, r = i % rows_blk;
    const int64_t n = n0 + r;
    if (n < g.N) {
      const float v = ((part[0][b][r] + part[1][b][r]) + part[2][b][r]) + part[3][b][r];
      store_out(g.out, g.out_dtype, (int64_t)b * g.N + n, v);
    }
  }
}

// ---------------------------------------------------------------- int4, tiled
//
// On the tiled int4 layout (16 rows x 64 k per contiguous 512-byte run) the
// product of one expert with the few tokens routed to it runs on the matrix
// cores: A = activations of up to 16 tokens (token m in lanes m, m+16, m+32,
// m+48), B = the tile's exact integer codes C + q (C = 128 as bf16, 1024 as
// fp16) in the tile's own k order, so lane l's 8-byte slice of the run is
// exactly its B operand.  A second product against ones gives each token's
// activation sum X over the tile, and per tile
//     y[m][n] += s[n] * P[m][n] + (b[n] - C * s[n]) * X[m],
// so scale and bias enter once per group, in fp32 (group >= 64 here).  More
// than 16 tokens on one expert are taken in further passes; the weights stay
// in registers between passes.

template <int ACT> struct One;
template <> struct One<ACT_F16> { static constexpr uint32_t bits = 0x3C003C00u; };
template <> struct One<ACT_BF16> { static constexpr uint32_t bits = 0x3F803F80u; };

// The eight codes of one word (elements 0..7) as four packed pairs.
template <int ACT>
__device__ __forceinline__ u4_t int4_codes(uint32_t q) {
  const uint32_t magic = Magic<ACT>::bits;
  u4_t c;
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = and_or_b32(q >> (4 * i), 0x000F000Fu, magic);
  return c;
}

// One tile's contribution for NB row blocks: acc[b] += s * P + cb * X.  With
// R1 only row 0 of the product (accumulator element 0 of lanes 0..15) is kept.
template <int ACT, int NB, bool R1 = false>
__device__ __forceinline__ void int4_tile(const u4_t& x0, const u4_t& x1, const u2_t (&w)[NB],
                                          const uint32_t (&sb)[NB], f4_t (&acc)[NB]) {
  const u4_t ones = u4_t{One<ACT>::bits, One<ACT>::bits, One<ACT>::bits, One<ACT>::bits};
  const f4_t z = f4_t{0.f, 0.f, 0.f, 0.f};
  f4_t X = mfma(as_v8<ACT>(x0), as_v8<ACT>(ones), z);
  X = mfma(as_v8<ACT>(x1), as_v8<ACT>(ones), X);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    f4_t P = mfma(as_v8<ACT>(x0), as_v8<ACT>(int4_codes<ACT>(w[b][0])), z);
    P = mfma(as_v8<ACT>(x1), as_v8<ACT>(int4_codes<ACT>(w[b][1])), P);
    const float s = f16_to_f32(sb[b] & 0xFFFFu);
    const float cb = __builtin_fmaf(-Magic<ACT>::v, s, f16_to_f32(sb[b] >> 16));
#pragma unroll
    for (int i = 0; i < (R1 ? 1 : 4); ++i) acc[b][i] = __builtin_fmaf(cb, X[i], __builtin_fmaf(s, P[i], acc[b][i]));
  }
}

// Buffer resource over [base, base + bytes): loads past the end return 0
// without touching memory.  base must be wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t OOB = 0x80000000u;  // a buffer offset that is always out of range

// Slot ids of a call held in registers: lane l keeps slot 64c + l of chunk c
// (-1 past the end), so the per-expert token lists below are ballots with no
// memory traffic.  At most QMOE_MAX_GEMV_BATCH * QMOE_MAX_TOPK = 512 slots.
constexpr int GV_CH = (QMOE_MAX_GEMV_BATCH * QMOE_MAX_TOPK) / 64;

typedef int SlotIds[GV_CH];

// Compile-time loop: f(std::integral_constant<int, c>) for c = C .. N-1, so
// every register-array index below is a constant from the start.
template <int C, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (C < N) {
    f(std::integral_constant<int, C>{});
    static_for<C + 1, N>(f);
  }
}

__device__ __forceinline__ void load_slot_ids(const int32_t* ids, int P, SlotIds& s) {
  const int lane = threadIdx.x & 63;
  static_for<0, GV_CH>([&](auto ci) {
    constexpr int c = decltype(ci)::value;
    const int p = 64 * c + lane;
    s[c] = ids[p < P ? p : 0];
    if (p >= P) s[c] = -1;
  });
}

// Expert of slot p (p wave-uniform, p < P), as a wave-uniform value.
__device__ __forceinline__ int slot_expert(const SlotIds& s, int p) {
  int v = s[0];
  static_for<1, GV_CH>([&](auto ci) {
    constexpr int c = decltype(ci)::value;
    if ((p >> 6) == c) v = s[c];
  });
  return __builtin_amdgcn_readlane(v, p & 63);
}

// Slot of the j-th occurrence (in slot order) of expert e, or -1; *count
// receives the number of occurrences.  Wave-wide.
__device__ __forceinline__ int nth_slot(const SlotIds& s, int P, int e, int j, int* count) {
  int base = 0, res = -1;
  static_for<0, GV_CH>([&](auto ci) {
    constexpr int c = decltype(ci)::value;
    if (64 * c < P) {
      const uint64_t m = __ballot(s[c] == e);
      const int cnt = __popcll(m);
      if (j >= base && j < base + cnt) {
        uint64_t mm = m;
        for (int i = base; i < j; ++i) mm &= mm - 1;
        res = 64 * c + __ffsll((unsigned long long)mm) - 1;
      }
      base += cnt;
    }
  });
  *count = base;
  return res;
}

// Decode kernels that put a call's whole weight stream in flight at once.  A
// workgroup owns one item and its waves split K into runs of GS_TPW tiles;
// each wave issues every load of its run (weight words, scale|bias words and,
// by LDS-DMA, the activation rows it needs) before computing, so a wave costs
// about one memory latency and the grid covers the chip.
//   STORE / SWIGLU: item = (slot p, 16-unit block).  An item whose slot
//     repeats an earlier slot's expert exits at once; the first one serves
//     every token routed to that expert, `rows` tokens per pass.
//   WEIGHTED_COMBINE: item = (token b, 16-row block); wave (j, c) computes the
//     expert of slot b * topk + j over K run c, and the top-k weighted sum is
//     formed in slot order (bit-reproducible).
constexpr int GS_TPW = 8;                     // tiles per wave
constexpr int GS_ROW = GS_TPW * 64 * 2 + 16;  // bytes per staged activation row (padded)
constexpr int GS_MAX_ROWS = 4;                // tokens per pass (STORE / SWIGLU)

__host__ __device__ constexpr int64_t gs_lds_bytes(int waves, int rows, int nb, bool cmb) {
  return (int64_t)waves * rows * GS_ROW + (cmb ? (int64_t)waves * 64 : (int64_t)(waves - 1) * nb * 1024);
}

template <int ACT, int EPI>
__global__ __launch_bounds__(1024) void gemv_int4_split_kernel(GemvArgs g, int rows) {
  constexpr bool CMB = (EPI == QMOE_EPI_WEIGHTED_COMBINE);
  constexpr int NB = (EPI == QMOE_EPI_SWIGLU) ? 2 : 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t gs_dyn[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = blockDim.x >> 6;
  const int r = lane & 15, lg = lane >> 4;
  const int P = g.nslots;
  const int gsh = __builtin_ctz((unsigned)g.group) - 6;
  const int64_t K = g.K;
  const int T = (int)(K >> 6), G = T >> gsh;
  const int CW = (T + GS_TPW - 1) / GS_TPW;  // waves per K
  const int64_t Nunits = (EPI == QMOE_EPI_SWIGLU) ? g.N / 2 : g.N;
  const int nub = (int)(Nunits / 16);
  uint8_t* const red = gs_dyn + (int64_t)W * rows * GS_ROW;

  const int item = blockIdx.x;
  const int ub = item % nub;
  int kc, e, slot_c = 0, nt = 1, sl = 0;
  SlotIds sid;
  if constexpr (CMB) {
    const int j = wave / CW;
    kc = wave - j * CW;
    slot_c = (item / nub) * g.topk + j;
    e = __builtin_amdgcn_readfirstlane(g.ids[slot_c]);
  } else {
    load_slot_ids(g.ids, P, sid);
    const int slot = item / nub;
    e = slot_expert(sid, slot);
    int c;
    if (e < 0 || e >= g.E || nth_slot(sid, P, e, 0, &c) != slot) return;  // uniform over the workgroup
    kc = wave;
    sl = nth_slot(sid, P, e, r, &nt);
  }
  const bool ok = e >= 0 && e < g.E;
  const int kt0 = kc * GS_TPW;
  const int64_t arows = CMB ? P : P / g.topk;
  // Combine: the token's k expert ids and weights, read by wave 0's lanes
  // now (in flight with the weights) rather than one dependent load pair
  // per slot after the reduction.
  int cmb_id = -1;
  float cmb_w = 0.f;
  if constexpr (CMB) {
    if (wave == 0 && lane < g.topk) {
      const int p = (item / nub) * g.topk + lane;
      cmb_id = g.ids[p];
      cmb_w = g.topk_w[p];
    }
  }
  const __amdgpu_buffer_rsrc_t xrs = rsrc(g.a, (uint32_t)(arows * K * 2));

  // Activation rows pass .. pass + n - 1 of this wave's K run: lane i loads
  // 16 bytes of each row into registers (rows past n load nothing), and
  // put_rows() writes them to this wave's LDS rows, where the MFMA operand
  // layout is read back.  Loads into registers, not LDS-DMA, so that every
  // wait is the compiler's own, in issue order with the weight loads.
  u4_t xv[GS_MAX_ROWS];
  auto load_rows = [&](int n) {
#pragma unroll
    for (int i = 0; i < GS_MAX_ROWS; ++i) {
      const int src = CMB ? slot_c : __builtin_amdgcn_readlane(sl, i < n ? i : 0) / g.topk;
      const uint32_t off = i < n ? (uint32_t)(((int64_t)src * K + kt0 * 64) * 2) + lane * 16 : OOB;
      xv[i] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0));
      if (CMB) break;
    }
  };
  auto put_rows = [&](int n) {
    uint8_t* const base = gs_dyn + (int64_t)wave * rows * GS_ROW + lane * 16;
#pragma unroll
    for (int i = 0; i < GS_MAX_ROWS; ++i) {
      if (i < n) *(u4_t*)(base + i * GS_ROW) = xv[i];
      if (CMB) break;
    }
  };
  int nrows = CMB ? 1 : min(nt, rows);
  load_rows(nrows);

  u2_t w[GS_TPW][NB];
  uint32_t sb[GS_TPW][NB];
  __amdgpu_buffer_rsrc_t wr[NB], sr[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t rb = ((int64_t)(ok ? e : 0) * g.N + (b ? Nunits : 0) + ub * 16) >> 4;
    wr[b] = rsrc((const uint32_t*)g.qs + rb * T * 128, ok ? (uint32_t)(T * 512) : 0u);
    sr[b] = rsrc((const uint32_t*)g.scales + rb * G * 16, ok ? (uint32_t)(G * 64) : 0u);
  }
  // Tile by tile, so that the first tiles are computed while the rest land.
  // The empty asm statements keep this order (the scheduler would otherwise
  // group the loads by kind, and the first tile would wait for the last load).
#pragma unroll
  for (int t = 0; t < GS_TPW; ++t) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      w[t][b] = __builtin_bit_cast(u2_t, __builtin_amdgcn_raw_buffer_load_b64(wr[b], (uint32_t)(lane * 8 + (kt0 + t) * 512), 0, 0));
      sb[t][b] = __builtin_amdgcn_raw_buffer_load_b32(sr[b], (uint32_t)(r * 4 + ((kt0 + t) >> gsh) * 64), 0, 0);
    }
    asm volatile("" ::: "memory");
  }
  put_rows(nrows);

  // One pass: the products of the staged rows, reduced over the waves and
  // stored (slot rows pass .. pass + nrows - 1 of the expert).
  auto run_pass = [&]() {
    const uint8_t* xr = gs_dyn + (int64_t)wave * rows * GS_ROW + (r < nrows ? r : 0) * GS_ROW + 32 * lg;
    f4_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f4_t{0.f, 0.f, 0.f, 0.f};
    auto tiles = [&](auto r1) {
#pragma unroll
      for (int t = 0; t < GS_TPW; ++t) {
        if (kt0 + t < T) {
          const u4_t x0 = *(const u4_t*)(xr + t * 128);
          const u4_t x1 = *(const u4_t*)(xr + t * 128 + 16);
          int4_tile<ACT, NB, decltype(r1)::value>(x0, x1, w[t], sb[t], acc);
        }
      }
    };
    // one token (always, for the combine): only row 0 of each product is used
    if (CMB || nrows == 1) tiles(std::true_type{});
    else tiles(std::false_type{});
    // keep the decoding inside each pass (hoisted out of the pass loop below,
    // it would hold every tile's codes in registers)
#pragma unroll
    for (int t = 0; t < GS_TPW; ++t)
#pragma unroll
      for (int b = 0; b < NB; ++b) asm volatile("" : "+v"(w[t][b]), "+v"(sb[t][b]));
    if constexpr (CMB) {
      // row 0 of the product is the slot's result; lanes 0..15 hold it
      float* y = (float*)red;  // [W][16]
      if (lane < 16) y[wave * 16 + lane] = acc[0][0];
      lds_barrier();
      if (threadIdx.x < 16) {
        const int b = item / nub;
        float v = 0.f;
        for (int j = 0; j < g.topk; ++j) {
          const int ej = __builtin_amdgcn_readlane(cmb_id, j);
          if (ej < 0 || ej >= g.E) continue;
          float yj = 0.f;
          for (int c = 0; c < CW; ++c) yj += y[(j * CW + c) * 16 + threadIdx.x];
          v = __builtin_fmaf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cmb_w), j)), yj, v);
        }
        store_out(g.out, g.out_dtype, (int64_t)b * g.N + ub * 16 + threadIdx.x, v);
      }
    } else {
      f4_t* rd = (f4_t*)red;  // [W - 1][NB][64]
      if (wave > 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) rd[((wave - 1) * NB + b) * 64 + lane] = acc[b];
      }
      lds_barrier();
      if (wave == 0) {
        for (int v = 1; v < W; ++v)
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[b] += rd[((v - 1) * NB + b) * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * lg + i;
          const int sm = __shfl(sl, m);
          if (m < nrows) {
            const float v = (EPI == QMOE_EPI_SWIGLU) ? silu_f32(acc[0][i]) * acc[NB - 1][i] : acc[0][i];
            store_out(g.out, g.out_dtype, (int64_t)sm * Nunits + ub * 16 + r, v);
          }
        }
      }
    }
  };
  run_pass();
  if constexpr (!CMB) {
    // more tokens on this expert than one pass holds (rare): restage and rerun
    for (int pass = rows; pass < nt; pass += rows) {
      lds_barrier();  // red[] and the staged rows are reused
      int c;
      sl = nth_slot(sid, P, e, pass + r, &c);
      nrows = min(nt - pass, rows);
      load_rows(nrows);
      put_rows(nrows);
      run_pass();
    }
  }
}

// Waves per workgroup of the split kernel (0: it does not take the call).
static int gs_waves(const GemvArgs& g, int epi) {
  const int cw = (int)((g.K / 64 + GS_TPW - 1) / GS_TPW);
  const int w = epi == QMOE_EPI_WEIGHTED_COMBINE ? g.topk * cw : cw;
  return w <= 16 ? w : 0;
}

// Whether the tiled int4 kernels take this call (else the generic ones do).
static bool int4_tiled_ok(const GemvArgs& g, int epi) {
  if (g.group < 64 || g.K > 4096 || gs_waves(g, epi) == 0) return false;
  return g.N % (epi == QMOE_EPI_SWIGLU ? 32 : 16) == 0;
}

template <int ACT, int EPI>
static int launch_gemv_split(const GemvArgs& g, int waves, hipStream_t s) {
  // the dynamic LDS limit is raised once per process (a function-local static
  // is initialised once, also when several threads launch)
  static const hipError_t attr = hipFuncSetAttribute((const void*)gemv_int4_split_kernel<ACT, EPI>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return QMOE_ERR_LAUNCH;
  constexpr bool CMB = EPI == QMOE_EPI_WEIGHTED_COMBINE;
  const int64_t units = EPI == QMOE_EPI_SWIGLU ? g.N / 2 : g.N;
  const int64_t tokens = g.nslots / g.topk;
  const int rows = CMB ? 1 : (int)(tokens < GS_MAX_ROWS ? tokens : GS_MAX_ROWS);
  const dim3 grid((unsigned)((units / 16) * (CMB ? tokens : g.nslots)));
  const size_t lds = (size_t)gs_lds_bytes(waves, rows, EPI == QMOE_EPI_SWIGLU ? 2 : 1, CMB);
  hipLaunchKernelGGL((gemv_int4_split_kernel<ACT, EPI>), grid, dim3(waves * 64), lds, s, g, rows);
  return QMOE_OK;
}

template <int ACT>
static int launch_gemv_int4_tiled(const GemvArgs& g, int epi, hipStream_t s) {
  const int w = gs_waves(g, epi);
  if (epi == QMOE_EPI_WEIGHTED_COMBINE) return launch_gemv_split<ACT, QMOE_EPI_WEIGHTED_COMBINE>(g, w, s);
  if (epi == QMOE_EPI_SWIGLU) return launch_gemv_split<ACT, QMOE_EPI_SWIGLU>(g, w, s);
  return launch_gemv_split<ACT, QMOE_EPI_STORE>(g, w, s);
}

template <int FMT, int ACT, int CPL, int MT>
static void launch_gemv_facm(const GemvArgs& g, int epi, int64_t units_total, hipStream_t s) {
  if (epi == QMOE_EPI_WEIGHTED_COMBINE) {
    const int rows_blk = GC_ITERS * (64 / g.lpr);
    const dim3 grid((unsigned)((g.N + rows_blk - 1) / rows_blk));
    hipLaunchKernelGGL((gemv_combine_kernel<FMT, ACT, CPL, MT>), grid, dim3(256), 0, s, g);
  } else {
    const dim3 grid((unsigned)((units_total + g.units_per_wg - 1) / g.units_per_wg), (unsigned)g.nslots);
    if (epi == QMOE_EPI_SWIGLU)
      hipLaunchKernelGGL((gemv_rows_kernel<FMT, ACT, QMOE_EPI_SWIGLU, CPL, MT>), grid, dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((gemv_rows_kernel<FMT, ACT, QMOE_EPI_STORE, CPL, MT>), grid, dim3(256), 0, s, g);
  }
}

// One token per call (b = 1): the kernels hold one token's activations per
// pass instead of GV_MAXT, which frees registers for more waves per SIMD.  A
// token that names one expert twice still works, in two passes.  Four chunks
// per lane (K above 4096) always take one token per pass.
template <int FMT, int ACT, int CPL>
static void launch_gemv_fac(const GemvArgs& g, int epi, int64_t units_total, hipStream_t s) {
  if (g.nslots == g.topk || CPL > 2) launch_gemv_facm<FMT, ACT, CPL, 1>(g, epi, units_total, s);
  else launch_gemv_facm<FMT, ACT, CPL, GV_MAXT>(g, epi, units_total, s);
}

template <int FMT>
static void launch_gemv_f(const GemvArgs& g, int act, int cpl, int epi, int64_t units, hipStream_t s) {
  if (act == QMOE_F16) {
    if (cpl == 1) launch_gemv_fac<FMT, ACT_F16, 1>(g, epi, units, s);
    else if (cpl == 2) launch_gemv_fac<FMT, ACT_F16, 2>(g, epi, units, s);
    else launch_gemv_fac<FMT, ACT_F16, 4>(g, epi, units, s);
  } else {
    if (cpl == 1) launch_gemv_fac<FMT, ACT_BF16, 1>(g, epi, units, s);
    else if (cpl == 2) launch_gemv_fac<FMT, ACT_BF16, 2>(g, epi, units, s);
    else launch_gemv_fac<FMT, ACT_BF16, 4>(g, epi, units, s);
  }
}

int64_t gemv_max_k() { return GV_MAX_K; }

// Host launcher for qmoe_moe_gemv (arguments already validated: K a multiple
// of 32, at most GV_MAX_K).  A row's K / 32 chunks are spread over lpr lanes
// (a power of two), CPL chunks per lane; lanes whose chunk index lies past
// the row's last chunk load a valid chunk and skip its arithmetic.
int launch_gemv(const qmoe_weights* w, const void* a, int act, int64_t b, const int32_t* ids,
                 const float* topk_w, int topk, int epi, void* out, int out_dtype, hipStream_t s) {
  GemvArgs g;
  g.qs = w->qs; g.aux = w->aux; g.scales = w->scales; g.biases = w->biases;
  g.d = w->d; g.dmin = w->dmin; g.grid = w->grid; g.signs = w->signs;
  g.N = w->n; g.K = w->k; g.group = w->group;
  g.E = w->n_experts; g.topk = topk; g.nslots = (int)(b * topk);
  g.a = (const uint16_t*)a; g.ids = ids; g.topk_w = topk_w;
  g.out = out; g.out_dtype = out_dtype;
  const int64_t chunks = w->k / 32;
  g.chunks = (int)chunks;
  const int cpl = chunks <= 64 ? 1 : chunks <= 128 ? 2 : 4;
  int lpr = 64;
  if (cpl == 1)
    for (lpr = 1; lpr < chunks; lpr <<= 1) {}
  // the sum-folded kernel keeps at most 4 rows per wave pass
  if (epi == QMOE_EPI_WEIGHTED_COMBINE && lpr < 16) lpr = 16;
  g.lpr = lpr;
  const int rpw = 64 / g.lpr;
  const int64_t units = (epi == QMOE_EPI_SWIGLU) ? w->n / 2 : w->n;
  // Enough workgroups to keep several waves per SIMD waiting on memory: aim
  // for about 4096 in total (measured: 512 left the MXFP4 decode 15-20% slower).
  // The rows kernel takes gr_load passes of 4 * rpw units at a time.
  const int mt = (g.nslots == topk || cpl > 2) ? 1 : GV_MAXT;
  const int64_t step = gr_load(w->fmt, mt, cpl) * 4 * rpw;
  int64_t upw = (units * g.nslots) / 4096;
  if (upw < step) upw = step;
  upw = (upw + step - 1) / step * step;
  if (upw > 64) upw = 64 > step ? 64 : step;
  g.units_per_wg = (int)upw;
  if (w->fmt == QMOE_INT4 && (chunks & (chunks - 1)) == 0 && int4_tiled_ok(g, epi)) {
    return act == QMOE_F16 ? launch_gemv_int4_tiled<ACT_F16>(g, epi, s) : launch_gemv_int4_tiled<ACT_BF16>(g, epi, s);
  }
  switch (w->fmt) {
    case QMOE_Q8_0: launch_gemv_f<QMOE_Q8_0>(g, act, cpl, epi, units, s); break;
    case QMOE_Q2_K: launch_gemv_f<QMOE_Q2_K>(g, act, cpl, epi, units, s); break;
    case QMOE_Q4_K: launch_gemv_f<QMOE_Q4_K>(g, act, cpl, epi, units, s); break;
    case QMOE_Q6_K: launch_gemv_f<QMOE_Q6_K>(g, act, cpl, epi, units, s); break;
    case QMOE_IQ2_XXS: launch_gemv_f<QMOE_IQ2_XXS>(g, act, cpl, epi, units, s); break;
    case QMOE_MXFP4: launch_gemv_f<QMOE_MXFP4>(g, act, cpl, epi, units, s); break;
    case QMOE_FP8: launch_gemv_f<QMOE_FP8>(g, act, cpl, epi, units, s); break;
    default: launch_gemv_f<QMOE_INT4>(g, act, cpl, epi, units, s); break;
  }
  return QMOE_OK;
}

}  // namespace qmoe
