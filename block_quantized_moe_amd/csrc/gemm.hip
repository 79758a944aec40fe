// Prefill matmul over quantised weights: the gathered MoE tile GEMM and the
// dense qmm share one kernel.
//
// What is computed: for each tile of (up to 80) rows routed to one expert
// and a slice of that expert's output rows, y = A . W[e]^T with fp32
// accumulation, followed by an epilogue (store, SwiGLU, top-k weighted
// scatter-add, or accumulate).  The DSV4 campaign page's tiled MoE prefill
// GEMM (map0 work queue, 64-slot iq2_xxs gate/up tile, q2_K SoA down twin)
// and the metaltile shim page's mt_qmm_mma / mt_moe_gather_qmm kernels are the
// prior art; the tiling here is built for CDNA4 instead.
//
// Layout on gfx950:
//  * 256 threads = 4 waves.  A workgroup owns one (row tile, column tile) and
//    each wave owns 64 weight rows as four 16-column MFMA blocks (SwiGLU: two
//    blocks of gate rows and the two matching blocks of up rows, so
//    silu(g)*u is lane-local).  One B fragment feeds every 16-row block of the
//    tile; one A fragment feeds the wave's four column blocks.
//  * K advances in 64-wide tiles.  The activation tile (80 x 64) is gathered
//    by routed row straight into LDS, double buffered, one barrier per tile.
//    The weight bytes each lane needs are loaded straight into registers two
//    tiles ahead (ping-pong buffers), so the HBM stream has two tiles of every
//    wave in flight.
//  * Within a 64-wide K tile, lane group g (lanes 16g..16g+15) owns the 16
//    contiguous k-values [16g, 16g+16); MFMA step s consumes values
//    16g+8s..16g+8s+7 of every lane group (the A fragments are read from LDS
//    with the same permutation, so the contraction is unchanged).  Formats
//    whose scale changes every 32 values with bf16 activations use the plain
//    k order instead (MFMA step s = values 32s..32s+31).
//  * fp16 activations: weights are dequantised to fp16 in registers (one or
//    two fp16 roundings per weight) and fed to v_mfma_f32_16x16x32_f16.
//  * bf16 activations: the MFMA consumes the integer codes, which are exact in
//    bf16, and the scales are applied to fp32 partial sums, so no weight is
//    rounded to bf16's 8-bit significand.  For int4 the per-group term
//    s*sum(x*(128+q)) is applied per tile, and the bias term
//    sum_g (b_g - 128 s_g) * X_g (X_g = sum of the activations of group g,
//    computed by an MFMA against ones) is added at the end by three MFMAs
//    over the groups with hi/lo bf16 splits of X and of the bias.
#include <atomic>
#include <type_traits>

#include "common.h"

namespace qmoe {

constexpr int BM = 80;        // rows per tile (at most; plan tiles must not be taller)
constexpr int BK = 64;        // k per LDS tile
constexpr int LDA = BK + 8;   // LDS row stride in halves (144 B, conflict-free b128 reads)
constexpr int MB = BM / 16;   // 16-row MFMA blocks per tile
constexpr int NB = 4;         // 16-column blocks per wave
constexpr int BN = 4 * NB * 16;  // weight rows per workgroup (256)
constexpr int XG_MAX = 64;    // int4 groups per row kept for the bf16 bias term
constexpr int LDX = XG_MAX + 4;

enum { AM_GATHER = 0, AM_SORTED = 1, AM_DENSE = 2 };

struct GemmArgs {
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
  int amode;
  const uint16_t* a;
  int64_t a_bytes;  // size of the activation buffer (byte offsets must stay below 2^31)
  const int32_t* plan;
  int E, topk, bm;
  int64_t P, t;
  int64_t M;  // dense rows
  const float* topk_w;
  void* out;
  int out_dtype;
  int64_t ldo;
  int n_ntiles;
  int n_blocks;
  int stage_out;  // int4 ring kernel: 2-byte output through LDS in whole rows (16-byte aligned rows)
  int sk_slots_xcd;      // int4 ring kernel: resident workgroups per XCD (0: no split units)
  int32_t* sk_tickets;   // the plan's work-balancing area
  float* sk_part;
};

// Which k order a (format, activation) path uses inside a 64-wide tile.
template <int FMT, int ACT>
struct KOrder {
  // true: lane group g owns k in [16g, 16g+16); false: MFMA step s covers [32s, 32s+32)
  static constexpr bool chunk =
      !(FMT == QMOE_MXFP4 ||
        (ACT == ACT_BF16 && (FMT == QMOE_Q8_0 || FMT == QMOE_IQ2_XXS || FMT == QMOE_Q4_K || FMT == QMOE_Q6_K)));
};

// Raw weight bytes one lane needs for one 64-wide K tile of one output row.
struct Raw {
  u4_t v;        // codes
  u4_t v2;       // Q6_K: the codes' top bit pairs
  uint32_t x0;   // scale / idx word
  uint32_t x1;   // bias / aux word
  uint32_t x2;   // d / second idx word
  uint32_t x3;   // dmin / second aux word
  uint32_t x4;   // second d
};

// ------------------------------------------------------------------ loads

template <int FMT, int ACT>
__device__ __forceinline__ Raw load_raw(const GemmArgs& g, int64_t R, int64_t k0, int lg) {
  Raw r;
  const int64_t K = g.K;
  if constexpr (FMT == QMOE_INT4) {
    // tiled layout: the 16 rows of block R/16 and one 64-wide k tile form one
    // 512-byte run, lane 16*lg + r holding row r's values 16*lg .. +15
    const int64_t rb = R >> 4, rr = R & 15;
    const u2_t q = *(const u2_t*)((const uint32_t*)g.qs + ((rb * (K / 64) + k0 / 64) * 64 + 16 * lg + rr) * 2);
    r.v[0] = q[0];
    r.v[1] = q[1];
    // scale in the low half, bias in the high half (the other fields stay unused)
    r.x0 = ((const uint32_t*)g.scales)[(rb * (K / g.group) + k0 / g.group) * 16 + rr];
  } else if constexpr (FMT == QMOE_Q8_0) {
    // tiled layout: the 16 rows x 64 k of one tile are one 1 KB run, chunk c
    // (16 values) of row r at byte 256c + 16r
    const int64_t rb = R >> 4, rr = R & 15;
    const int8_t* tile = (const int8_t*)g.qs + (rb * (K / 64) + k0 / 64) * 1024 + 16 * rr;
    const uint16_t* sc = (const uint16_t*)g.scales + (rb * (K / 32) + k0 / 32) * 16 + rr;
    if constexpr (KOrder<FMT, ACT>::chunk) {
      r.v = *(const u4_t*)(tile + 256 * lg);
      r.x0 = sc[16 * (lg >> 1)];
    } else {
      // values 8lg .. 8lg+7 and 32+8lg .. 32+8lg+7 of the tile
      const u2_t q0 = *(const u2_t*)(tile + 256 * (lg >> 1) + 8 * (lg & 1));
      const u2_t q1 = *(const u2_t*)(tile + 256 * (2 + (lg >> 1)) + 8 * (lg & 1));
      r.v = u4_t{q0[0], q0[1], q1[0], q1[1]};
      r.x0 = sc[0];
      r.x2 = sc[16];
    }
  } else if constexpr (FMT == QMOE_MXFP4) {
    // tiled layout: block j of the tile is 16 rows x 16 B; lane group lg
    // takes word lg (elements 8lg .. 8lg+7) of both blocks, a wave reading
    // 256 contiguous bytes per block
    const int64_t rb = R >> 4, rr = R & 15;
    const uint32_t* tile = (const uint32_t*)g.qs + (rb * (K / 64) + k0 / 64) * 128 + 4 * rr + lg;
    r.v[0] = tile[0];
    r.v[1] = tile[64];
    const uint8_t* e = (const uint8_t*)g.scales + (rb * (K / 32) + k0 / 32) * 16 + rr;
    r.x0 = e[0];
    r.x2 = e[16];
  } else if constexpr (FMT == QMOE_FP8) {
    // codes tiled like Q8_0 (chunk c of row r at byte 256c + 16r of the 1 KB
    // tile); the tile lies inside one 128 x 128 scale block
    const int64_t rb = R >> 4, rr = R & 15;
    r.v = *(const u4_t*)((const uint8_t*)g.qs + (rb * (K / 64) + k0 / 64) * 1024 + 16 * rr + 256 * lg);
    r.x0 = __builtin_bit_cast(uint32_t, ((const float*)g.scales)[(R >> 7) * (K >> 7) + (k0 >> 7)]);
  } else if constexpr (FMT == QMOE_Q2_K) {
    // tiled layout: t = 16-row block * K/256 + super-block; a wave's loads of
    // one 16-row block read contiguous runs
    const int64_t t = (R >> 4) * (K / 256) + k0 / 256, rr = R & 15;
    const int e0 = (int)(k0 & 255) + 16 * lg;
    const int h = e0 >> 7, cb = e0 & 31;  // code bytes 32h + cb .. +15
    r.v = *(const u4_t*)((const uint8_t*)g.qs + ((t * 2 + h) * 16 + rr) * 32 + cb);
    r.x0 = ((const uint8_t*)g.scales)[(t * 16 + rr) * 16 + (e0 >> 4)];
    r.x1 = 2u * (uint32_t)((e0 & 127) >> 5);  // bit shift of this lane's codes
    r.x2 = ((const uint16_t*)g.d)[t * 16 + rr];
    r.x3 = ((const uint16_t*)g.dmin)[t * 16 + rr];
  } else if constexpr (FMT == QMOE_Q4_K) {
    // tiled layout: the 64-wide tile is quarter h of the super-block, 32 code
    // bytes per row (element 64h + i in the low nibble of byte i, 64h + 32 + i
    // in the high); scales then mins of the 8 sub-blocks as bytes
    const int64_t t = (R >> 4) * (K / 256) + k0 / 256, rr = R & 15;
    const int h = (int)(k0 & 255) >> 6;
    const uint8_t* cq = (const uint8_t*)g.qs + ((t * 4 + h) * 16 + rr) * 32;
    const uint8_t* sm = (const uint8_t*)g.scales + (t * 16 + rr) * 16;
    if constexpr (KOrder<FMT, ACT>::chunk) {
      // values 16 lg .. +15: bytes 16 (lg & 1) .. +15, high nibbles for lg >= 2
      r.v = *(const u4_t*)(cq + 16 * (lg & 1));
      r.x1 = 4u * (uint32_t)(lg >> 1);
      const int j = 2 * h + (lg >> 1);
      r.x0 = (uint32_t)sm[j] | ((uint32_t)sm[8 + j] << 8);
    } else {
      // MFMA step s: values 32 s + 8 lg .. +7 = low (s = 0) or high (s = 1)
      // nibbles of bytes 8 lg .. +7; sub-blocks 2h and 2h + 1
      const u2_t q = *(const u2_t*)(cq + 8 * lg);
      r.v[0] = q[0];
      r.v[1] = q[1];
      r.x0 = (uint32_t)sm[2 * h] | ((uint32_t)sm[2 * h + 1] << 8) | ((uint32_t)sm[8 + 2 * h] << 16) |
             ((uint32_t)sm[9 + 2 * h] << 24);
    }
    r.x2 = ((const uint16_t*)g.d)[t * 16 + rr];
    r.x3 = ((const uint16_t*)g.dmin)[t * 16 + rr];
  } else if constexpr (FMT == QMOE_Q6_K) {
    // tiled layout: low 4 bits as Q4_K's codes; top bit pairs of element
    // 128 n + 32 p + i at byte i of half n, bits 2p (the tile is quarter h, so
    // n = h / 2 and p = 2 (h % 2) + (0 or 1)); int8 scales of 16-value sub-blocks
    const int64_t t = (R >> 4) * (K / 256) + k0 / 256, rr = R & 15;
    const int h = (int)(k0 & 255) >> 6;
    const uint8_t* cq = (const uint8_t*)g.qs + ((t * 4 + h) * 16 + rr) * 32;
    const uint8_t* ch = (const uint8_t*)g.aux + ((t * 2 + (h >> 1)) * 16 + rr) * 32;
    const int8_t* sc = (const int8_t*)g.scales + (t * 16 + rr) * 16;
    if constexpr (KOrder<FMT, ACT>::chunk) {
      r.v = *(const u4_t*)(cq + 16 * (lg & 1));
      r.v2 = *(const u4_t*)(ch + 16 * (lg & 1));
      r.x1 = (4u * (uint32_t)(lg >> 1)) | ((2u * (uint32_t)(2 * (h & 1) + (lg >> 1))) << 8);
      r.x0 = (uint32_t)(uint8_t)sc[4 * h + lg];  // sub-block of values 16 lg .. +15
    } else {
      // step s: values 32 s + 8 lg .. +7: nibbles of bytes 8 lg .. +7 (high
      // for s = 1), top bits of bytes 8 lg .. +7 at bits 4 (h % 2) + 2 s;
      // the four scales of sub-blocks 4h .. 4h + 3
      const u2_t q = *(const u2_t*)(cq + 8 * lg);
      const u2_t p = *(const u2_t*)(ch + 8 * lg);
      r.v = u4_t{q[0], q[1], p[0], p[1]};
      r.x1 = 4u * (uint32_t)(h & 1);
      r.x0 = *(const uint32_t*)(sc + 4 * h);
    }
    r.x2 = ((const uint16_t*)g.d)[t * 16 + rr];
  } else {  // IQ2_XXS, tiled: (index word, aux word) pairs by group and row
    const int64_t t = (R >> 4) * (K / 256) + k0 / 256, rr = R & 15;
    const uint32_t* ia = (const uint32_t*)g.qs + (t * 8 * 16 + rr) * 2;
    if constexpr (KOrder<FMT, ACT>::chunk) {
      const int G = ((int)(k0 & 255) + 16 * lg) >> 5;
      const u2_t p = *(const u2_t*)(ia + G * 32);
      r.x0 = p[0];
      r.x1 = p[1];
    } else {
      const int G = (int)(k0 & 255) >> 5;
      const u2_t p0 = *(const u2_t*)(ia + G * 32);
      const u2_t p1 = *(const u2_t*)(ia + (G + 1) * 32);
      r.x0 = p0[0];
      r.x1 = p0[1];
      r.x2 = p1[0];
      r.x3 = p1[1];
    }
    r.x4 = ((const uint16_t*)g.d)[t * 16 + rr];
  }
  return r;
}

// ------------------------------------------------------------------ B fragments

// Two byte codes -> two halves holding (magic byte : code byte): perm selectors.
constexpr uint32_t SEL_B01 = 0x04010400u;  // [b0, m, b1, m]
constexpr uint32_t SEL_B23 = 0x04030402u;  // [b2, m, b3, m]

// fp16 path: dequantised weights for MFMA steps 0 and 1 of a lane (chunk order
// k = 16g + 8s + i).  lg = lane group (only the IQ2_XXS octet choice needs it).
template <int FMT>
__device__ __forceinline__ void frag_f16(const Raw& r, int lg, const uint32_t* lut_grid,
                                         const uint32_t* lut_sign, u4_t& o0, u4_t& o1) {
  if constexpr (FMT == QMOE_INT4) {
    const h2_t s2 = h2_t{__builtin_bit_cast(_Float16, (uint16_t)r.x0), __builtin_bit_cast(_Float16, (uint16_t)r.x0)};
    const h2_t b2 = h2_t{__builtin_bit_cast(_Float16, (uint16_t)(r.x0 >> 16)), __builtin_bit_cast(_Float16, (uint16_t)(r.x0 >> 16))};
    const h2_t off = h2_t{(_Float16)1024.0f, (_Float16)1024.0f};
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t q = r.v[w];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t p = ((q >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
        const h2_t c = __builtin_bit_cast(h2_t, p) - off;
        const uint32_t v = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(c, s2, b2));
        if (w == 0) o0[i] = v; else o1[i] = v;
      }
    }
  } else if constexpr (FMT == QMOE_Q8_0) {
    const _Float16 dh = __builtin_bit_cast(_Float16, (uint16_t)r.x0);
    const h2_t d2 = h2_t{dh, dh};
    const h2_t off = h2_t{(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t u = r.v[w] ^ 0x80808080u;
      const h2_t lo = __builtin_bit_cast(h2_t, perm_b32(0x64646464u, u, SEL_B01)) - off;
      const h2_t hi = __builtin_bit_cast(h2_t, perm_b32(0x64646464u, u, SEL_B23)) - off;
      const uint32_t vl = __builtin_bit_cast(uint32_t, lo * d2);
      const uint32_t vh = __builtin_bit_cast(uint32_t, hi * d2);
      if (w < 2) { o0[2 * w] = vl; o0[2 * w + 1] = vh; }
      else { o1[2 * (w - 2)] = vl; o1[2 * (w - 2) + 1] = vh; }
    }
  } else if constexpr (FMT == QMOE_Q2_K) {
    const uint32_t sc = r.x0;
    const float d = f16_to_f32(r.x2), dm = f16_to_f32(r.x3);
    const _Float16 dl = (_Float16)(d * (float)(sc & 15u));
    const _Float16 ml = (_Float16)(-(dm * (float)(sc >> 4)));
    const h2_t dl2 = h2_t{dl, dl}, ml2 = h2_t{ml, ml};
    const uint32_t shift = r.x1;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t t = (r.v[w] >> shift) & 0x03030303u;
      const h2_t lo = __builtin_bit_cast(h2_t, u8x2_small_f16<false>(t));
      const h2_t hi = __builtin_bit_cast(h2_t, u8x2_small_f16<true>(t));
      const uint32_t vl = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(lo, dl2, ml2));
      const uint32_t vh = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(hi, dl2, ml2));
      if (w < 2) { o0[2 * w] = vl; o0[2 * w + 1] = vh; }
      else { o1[2 * (w - 2)] = vl; o1[2 * (w - 2) + 1] = vh; }
    }
  } else if constexpr (FMT == QMOE_Q4_K) {
    const float d = f16_to_f32(r.x2), dm = f16_to_f32(r.x3);
    const _Float16 dl = (_Float16)(d * (float)(r.x0 & 255u));
    const _Float16 ml = (_Float16)(-(dm * (float)((r.x0 >> 8) & 255u)));
    const h2_t dl2 = h2_t{dl, dl}, ml2 = h2_t{ml, ml};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t t = (r.v[w] >> r.x1) & 0x0F0F0F0Fu;
      const h2_t lo = __builtin_bit_cast(h2_t, u8x2_small_f16<false>(t));
      const h2_t hi = __builtin_bit_cast(h2_t, u8x2_small_f16<true>(t));
      const uint32_t vl = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(lo, dl2, ml2));
      const uint32_t vh = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(hi, dl2, ml2));
      if (w < 2) { o0[2 * w] = vl; o0[2 * w + 1] = vh; }
      else { o1[2 * (w - 2)] = vl; o1[2 * (w - 2) + 1] = vh; }
    }
  } else if constexpr (FMT == QMOE_Q6_K) {
    const _Float16 dl = (_Float16)(f16_to_f32(r.x2) * (float)(int8_t)(r.x0 & 255u));
    const h2_t dl2 = h2_t{dl, dl};
    const h2_t off = h2_t{(_Float16)1056.0f, (_Float16)1056.0f};  // 1024 + 32
    const uint32_t sn = r.x1 & 255u, sh = (r.x1 >> 8) & 255u;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t t = ((r.v[w] >> sn) & 0x0F0F0F0Fu) | (((r.v2[w] >> sh) & 0x03030303u) << 4);
      const h2_t lo = __builtin_bit_cast(h2_t, perm_b32(0x64646464u, t, SEL_B01)) - off;
      const h2_t hi = __builtin_bit_cast(h2_t, perm_b32(0x64646464u, t, SEL_B23)) - off;
      const uint32_t vl = __builtin_bit_cast(uint32_t, lo * dl2);
      const uint32_t vh = __builtin_bit_cast(uint32_t, hi * dl2);
      if (w < 2) { o0[2 * w] = vl; o0[2 * w + 1] = vh; }
      else { o1[2 * (w - 2)] = vl; o1[2 * (w - 2) + 1] = vh; }
    }
  } else {  // IQ2_XXS: octets j0, j0+1 of the group, j0 = 2 * (lg & 1)
    const uint32_t idx = r.x0, aux = r.x1;
    // d (0.5 + s) / 4: the second factor is exact in fp32, so the product
    // rounds once, to fp16
    const float bs = __builtin_fmaf((float)(aux >> 28), 0.25f, 0.125f);
    const _Float16 dbh = (_Float16)(f16_to_f32(r.x4) * bs);
    const h2_t db2 = h2_t{dbh, dbh};
    const int j0 = 2 * (lg & 1);
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const int j = j0 + o;
      const uint32_t gi = __builtin_amdgcn_ubfe(idx, 8 * j, 8);
      const uint32_t si = __builtin_amdgcn_ubfe(aux, 7 * j, 7);
      const u4_t row = *(const u4_t*)(lut_grid + 4 * gi);
      const u4_t msk = *(const u4_t*)(lut_sign + 4 * si);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const h2_t m = __builtin_bit_cast(h2_t, row[i] ^ msk[i]) * db2;
        if (o == 0) o0[i] = __builtin_bit_cast(uint32_t, m);
        else o1[i] = __builtin_bit_cast(uint32_t, m);
      }
    }
  }
}

// bf16 helpers: round-to-nearest-even fp32 -> bf16 bits, and a hi/lo split.
__device__ __forceinline__ uint32_t bf16_rne_bits(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ void split_hi_lo(float v, uint32_t& hi, uint32_t& lo) {
  hi = bf16_rne_bits(v);
  lo = bf16_rne_bits(v - __builtin_bit_cast(float, hi << 16));
}

// ------------------------------------------------------------------ kernel

// Per-workgroup context handed from the kernel prologue to the tile body.
struct TileCtx {
  uint16_t* As;          // [2][BM * LDA]
  const int* rows_a;
  const int* rows_o;
  const float* wts;
  float* xg;             // [BM * LDX] (bf16 int4 only)
  const uint32_t* lut_grid;
  const uint32_t* lut_sign;
  int tid, lane, wave, lg, lr;
  int nrows, mbn;
  int64_t ncol[NB];
  bool nvalid[NB];
  int64_t Rb[NB];
};

// The K loop and epilogue of a tile of at most MBV 16-row blocks (c.mbn of
// them hold rows).  FOLD (MXFP4 with fp16 activations only): every block
// scale of the workgroup's weight rows is known to lie in 2^-13 .. 2^13.
template <int FMT, int ACT, int EPI, int MBV, bool FOLD = false>
__device__ __forceinline__ void qmm_body(const GemmArgs& g, const TileCtx& c) {
  constexpr bool INT4_BF16 = (ACT == ACT_BF16 && FMT == QMOE_INT4);
  const int tid = c.tid, wave = c.wave, lg = c.lg, lr = c.lr;
  constexpr int ACHV = (MBV * 16 * 8 + 255) / 256;  // 16-byte activation chunks per thread

  f4_t acc[MBV][NB];
#pragma unroll
  for (int m = 0; m < MBV; ++m)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[m][b] = f4_t{0, 0, 0, 0};

  const int KT = (int)(g.K / BK);
  const uint16_t* __restrict__ A = g.a;

  // ---- activation staging: rows 0 .. 16*MBV-1 of the tile, 8 chunks of 16 B each.
  // Buffer loads with a byte offset per chunk; rows without data get an
  // offset past the end of the buffer, which the hardware returns as zeros, so
  // the staging has no branches (and the vmcnt bookkeeping stays exact).
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)A, (short)0, (int)g.a_bytes, 0x00020000);
  uint32_t aoff[ACHV];
#pragma unroll
  for (int i = 0; i < ACHV; ++i) {
    const int ch = tid + 256 * i;
    const int r = ch >> 3, part = ch & 7;
    const int src = (r < 16 * c.mbn) ? c.rows_a[r] : -1;
    aoff[i] = src >= 0 ? (uint32_t)(src * g.K * 2 + 16 * part) : 0x80000000u;
  }
  u4_t astage[ACHV];
  auto load_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < ACHV; ++i)
      astage[i] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(arsrc, aoff[i] + (uint32_t)kt * (BK * 2), 0, 0));
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ACHV; ++i) {
      const int ch = tid + 256 * i;
      const int r = ch >> 3, part = ch & 7;
      if (r < 16 * MBV) *(u4_t*)(&c.As[buf * BM * LDA + r * LDA + 8 * part]) = astage[i];
    }
  };

  // ---- one K tile of MFMA work from LDS buffer `buf` and raw weights `rw`
  auto compute = [&](int kt, int buf, const Raw (&rw)[NB]) {
    const uint16_t* Ab = c.As + buf * BM * LDA;
    if constexpr (FMT == QMOE_MXFP4) {
      // plain k order, either activation type: step s = one 32-value block;
      // the E2M1 code values enter the MFMA exactly and the block's
      // power-of-two scale multiplies the partial sum.  The tile's A
      // fragments are read from LDS once into registers and serve all four
      // column blocks (reading them once per block made the kernel
      // LDS-bound).
      typedef typename ActT<ACT>::v8 V8;
      V8 af[MBV][2];
#pragma unroll
      for (int m = 0; m < MBV; ++m) {
        if (m >= c.mbn) break;
        const uint16_t* ar = Ab + (16 * m + lr) * LDA + 8 * lg;
        af[m][0] = __builtin_bit_cast(V8, *(const u4_t*)ar);
        af[m][1] = __builtin_bit_cast(V8, *(const u4_t*)(ar + 32));
      }
      if constexpr (FOLD) {
        // each E2M1 value times its block scale is an exact fp16 normal
        // number (0.5 * 2^-13 .. 6 * 2^13): the scale goes into the B operand
        // through the conversion and the MFMAs accumulate directly, with no
        // fp32 scaling per block
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const h8_t b0 = __builtin_bit_cast(h8_t, fp4x8_pairs_scaled<ACT>(rw[b].v[0], e8m0_to_f32(rw[b].x0)));
          const h8_t b1 = __builtin_bit_cast(h8_t, fp4x8_pairs_scaled<ACT>(rw[b].v[1], e8m0_to_f32(rw[b].x2)));
#pragma unroll
          for (int m = 0; m < MBV; ++m) {
            if (m >= c.mbn) break;
            acc[m][b] = mfma(af[m][0], b0, acc[m][b]);
            acc[m][b] = mfma(af[m][1], b1, acc[m][b]);
          }
        }
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const u4_t cc[2] = {fp4x8_pairs<ACT>(rw[b].v[0]), fp4x8_pairs<ACT>(rw[b].v[1])};
          const float d0 = e8m0_to_f32(rw[b].x0), d1 = e8m0_to_f32(rw[b].x2);
#pragma unroll
          for (int m = 0; m < MBV; ++m) {
            if (m >= c.mbn) break;
            const f4_t t0 = mfma(af[m][0], __builtin_bit_cast(V8, cc[0]), f4_t{0, 0, 0, 0});
            const f4_t t1 = mfma(af[m][1], __builtin_bit_cast(V8, cc[1]), f4_t{0, 0, 0, 0});
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[m][b][r] = __builtin_fmaf(d1, t1[r], __builtin_fmaf(d0, t0[r], acc[m][b][r]));
          }
        }
      }
    } else if constexpr (FMT == QMOE_FP8) {
      // chunk order, either activation type: the E4M3 values enter the MFMA
      // exactly and the block scale multiplies the tile's fp32 partial sum.
      // Column blocks two at a time (A fragments read from LDS once per
      // pair), which keeps the converted operands within the register budget.
      typedef typename ActT<ACT>::v8 V8;
#pragma unroll
      for (int hp = 0; hp < NB; hp += 2) {
        u4_t cc[2][2];
        float sc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const u2_t p0 = fp8x4_pairs<ACT>(rw[hp + j].v[2 * st]);
            const u2_t p1 = fp8x4_pairs<ACT>(rw[hp + j].v[2 * st + 1]);
            cc[j][st] = u4_t{p0[0], p0[1], p1[0], p1[1]};
          }
          sc[j] = __builtin_bit_cast(float, rw[hp + j].x0);
        }
#pragma unroll
        for (int m = 0; m < MBV; ++m) {
          if (m >= c.mbn) break;
          const uint16_t* ar = Ab + (16 * m + lr) * LDA + 16 * lg;
          const V8 a0 = __builtin_bit_cast(V8, *(const u4_t*)ar);
          const V8 a1 = __builtin_bit_cast(V8, *(const u4_t*)(ar + 8));
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            f4_t t = mfma(a0, __builtin_bit_cast(V8, cc[j][0]), f4_t{0, 0, 0, 0});
            t = mfma(a1, __builtin_bit_cast(V8, cc[j][1]), t);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[m][hp + j][r] = __builtin_fmaf(sc[j], t[r], acc[m][hp + j][r]);
          }
        }
      }
    } else if constexpr (ACT == ACT_F16) {
      u4_t bf[NB][2];
#pragma unroll
      for (int b = 0; b < NB; ++b) frag_f16<FMT>(rw[b], lg, c.lut_grid, c.lut_sign, bf[b][0], bf[b][1]);
#pragma unroll
      for (int m = 0; m < MBV; ++m) {
        if (m >= c.mbn) break;
        const uint16_t* ar = Ab + (16 * m + lr) * LDA + 16 * lg;
        const h8_t a0 = __builtin_bit_cast(h8_t, *(const u4_t*)ar);
        const h8_t a1 = __builtin_bit_cast(h8_t, *(const u4_t*)(ar + 8));
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          acc[m][b] = mfma(a0, __builtin_bit_cast(h8_t, bf[b][0]), acc[m][b]);
          acc[m][b] = mfma(a1, __builtin_bit_cast(h8_t, bf[b][1]), acc[m][b]);
        }
      }
    } else if constexpr (FMT == QMOE_INT4) {
      // codes (128+q) as bf16 pairs; the tile lies inside one group.  The
      // column blocks are taken two at a time (the A fragments are read from
      // LDS once per pair) to keep the live registers within two waves/SIMD.
      const b8_t ones = __builtin_bit_cast(b8_t, u4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
      const int tiles_per_group = g.group / BK;
      const int gi = kt / tiles_per_group;
      const bool first_of_group = (kt % tiles_per_group) == 0;
#pragma unroll
      for (int hp = 0; hp < NB; hp += 2) {
        u4_t c0[2], c1[2];
        float s[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            c0[j][i] = ((rw[hp + j].v[0] >> (4 * i)) & 0x000F000Fu) | 0x43004300u;
            c1[j][i] = ((rw[hp + j].v[1] >> (4 * i)) & 0x000F000Fu) | 0x43004300u;
          }
          s[j] = f16_to_f32(rw[hp + j].x0);
        }
#pragma unroll
        for (int m = 0; m < MBV; ++m) {
          if (m >= c.mbn) break;
          const uint16_t* ar = Ab + (16 * m + lr) * LDA + 16 * lg;
          const b8_t a0 = __builtin_bit_cast(b8_t, *(const u4_t*)ar);
          const b8_t a1 = __builtin_bit_cast(b8_t, *(const u4_t*)(ar + 8));
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            f4_t t = mfma(a0, __builtin_bit_cast(b8_t, c0[j]), f4_t{0, 0, 0, 0});
            t = mfma(a1, __builtin_bit_cast(b8_t, c1[j]), t);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[m][hp + j][r] = __builtin_fmaf(s[j], t[r], acc[m][hp + j][r]);
          }
          if (hp == 0 && (m & 3) == wave) {  // this wave records the row sums of block m
            f4_t xs = mfma(a0, ones, f4_t{0, 0, 0, 0});
            xs = mfma(a1, ones, xs);
            if (lr < 4) {
              float* dst = &c.xg[(16 * m + 4 * lg + lr) * LDX + gi];
              const float val = xs[lr];
              *dst = first_of_group ? val : *dst + val;
            }
          }
        }
      }
    } else if constexpr (FMT == QMOE_Q8_0) {
      // plain k order: step s = one 32-value block; codes converted exactly
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        u4_t cc[2];
        const float d0 = f16_to_f32(rw[b].x0), d1 = f16_to_f32(rw[b].x2);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t w = rw[b].v[2 * st + (i >> 1)];
            const int sh = 16 * (i & 1);
            const float lo = (float)(int8_t)((w >> sh) & 0xFFu);
            const float hi = (float)(int8_t)((w >> (sh + 8)) & 0xFFu);
            cc[st][i] = (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
          }
        }
#pragma unroll
        for (int m = 0; m < MBV; ++m) {
          if (m >= c.mbn) break;
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const b8_t a = __builtin_bit_cast(b8_t, *(const u4_t*)(Ab + (16 * m + lr) * LDA + 32 * st + 8 * lg));
            const f4_t t = mfma(a, __builtin_bit_cast(b8_t, cc[st]), f4_t{0, 0, 0, 0});
            const float ds = st ? d1 : d0;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[m][b][r] = __builtin_fmaf(ds, t[r], acc[m][b][r]);
          }
        }
      }
    } else if constexpr (FMT == QMOE_IQ2_XXS) {
      // plain k order: step s = one 32-value group, octet lg of it
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        u4_t cc[2];
        float dsc[2];
        const float d = f16_to_f32(rw[b].x4);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const uint32_t idx = st ? rw[b].x2 : rw[b].x0;
          const uint32_t aux = st ? rw[b].x3 : rw[b].x1;
          dsc[st] = d * (0.5f + (float)(aux >> 28)) * 0.25f;
          const uint32_t gi = (idx >> (8 * lg)) & 0xFFu;
          const uint32_t si = (aux >> (7 * lg)) & 0x7Fu;
          const u4_t row = *(const u4_t*)(c.lut_grid + 4 * gi);
          const u4_t msk = *(const u4_t*)(c.lut_sign + 4 * si);
          cc[st] = row ^ msk;
        }
#pragma unroll
        for (int m = 0; m < MBV; ++m) {
          if (m >= c.mbn) break;
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const b8_t a = __builtin_bit_cast(b8_t, *(const u4_t*)(Ab + (16 * m + lr) * LDA + 32 * st + 8 * lg));
            const f4_t t = mfma(a, __builtin_bit_cast(b8_t, cc[st]), f4_t{0, 0, 0, 0});
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[m][b][r] = __builtin_fmaf(dsc[st], t[r], acc[m][b][r]);
          }
        }
      }
    } else if constexpr (FMT == QMOE_Q4_K) {
      // plain k order: step s = sub-block 2h + s of the tile's quarter h.  The
      // codes enter as exact bf16 (128 + q); sum a*(d sc q - dmin m) over the
      // step is d sc * T - (128 d sc + dmin m) * X with T the MFMA of the
      // codes and X the step's activation sums (an MFMA with ones)
      const b8_t ones = __builtin_bit_cast(b8_t, u4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
      u4_t cc[NB][2];
      float dsc[NB][2], cx[NB][2];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float d = f16_to_f32(rw[b].x2), dm = f16_to_f32(rw[b].x3);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const uint32_t t0 = (rw[b].v[0] >> (4 * st)) & 0x0F0F0F0Fu, t1 = (rw[b].v[1] >> (4 * st)) & 0x0F0F0F0Fu;
          cc[b][st] = u4_t{perm_b32(0x43434343u, t0, SEL_B01), perm_b32(0x43434343u, t0, SEL_B23),
                           perm_b32(0x43434343u, t1, SEL_B01), perm_b32(0x43434343u, t1, SEL_B23)};
          dsc[b][st] = d * (float)((rw[b].x0 >> (8 * st)) & 255u);
          cx[b][st] = 128.0f * dsc[b][st] + dm * (float)((rw[b].x0 >> (16 + 8 * st)) & 255u);
        }
      }
#pragma unroll
      for (int m = 0; m < MBV; ++m) {
        if (m >= c.mbn) break;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const b8_t a = __builtin_bit_cast(b8_t, *(const u4_t*)(Ab + (16 * m + lr) * LDA + 32 * st + 8 * lg));
          const f4_t tx = mfma(a, ones, f4_t{0, 0, 0, 0});
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const f4_t tq = mfma(a, __builtin_bit_cast(b8_t, cc[b][st]), f4_t{0, 0, 0, 0});
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[m][b][r] = __builtin_fmaf(dsc[b][st], tq[r], __builtin_fmaf(-cx[b][st], tx[r], acc[m][b][r]));
          }
        }
      }
    } else if constexpr (FMT == QMOE_Q6_K) {
      // plain k order: step s covers sub-blocks 4h + 2s (lane groups 0-1) and
      // 4h + 2s + 1 (lane groups 2-3), each with its own scale, so each half
      // goes through its own MFMA (the other lanes' operands zero).  Codes
      // (128 + q) are exact in bf16 (q < 64); sum a*d sc (q - 32) over a half
      // is d sc * (T - 160 X).
      const b8_t ones = __builtin_bit_cast(b8_t, u4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
      const b8_t zero8 = __builtin_bit_cast(b8_t, u4_t{0u, 0u, 0u, 0u});
      const bool first_half = lg < 2;
      u4_t cc[NB][2];
      float ds[NB][4];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float d = f16_to_f32(rw[b].x2);
#pragma unroll
        for (int j = 0; j < 4; ++j) ds[b][j] = d * (float)(int8_t)((rw[b].x0 >> (8 * j)) & 255u);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const uint32_t sh = rw[b].x1 + 2u * (uint32_t)st;
          const uint32_t t0 = ((rw[b].v[0] >> (4 * st)) & 0x0F0F0F0Fu) | (((rw[b].v[2] >> sh) & 0x03030303u) << 4);
          const uint32_t t1 = ((rw[b].v[1] >> (4 * st)) & 0x0F0F0F0Fu) | (((rw[b].v[3] >> sh) & 0x03030303u) << 4);
          cc[b][st] = u4_t{perm_b32(0x43434343u, t0, SEL_B01), perm_b32(0x43434343u, t0, SEL_B23),
                           perm_b32(0x43434343u, t1, SEL_B01), perm_b32(0x43434343u, t1, SEL_B23)};
        }
      }
      const b8_t ones_a = first_half ? ones : zero8, ones_b = first_half ? zero8 : ones;
#pragma unroll
      for (int m = 0; m < MBV; ++m) {
        if (m >= c.mbn) break;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const b8_t a = __builtin_bit_cast(b8_t, *(const u4_t*)(Ab + (16 * m + lr) * LDA + 32 * st + 8 * lg));
          const f4_t xa = mfma(a, ones_a, f4_t{0, 0, 0, 0});
          const f4_t xb = mfma(a, ones_b, f4_t{0, 0, 0, 0});
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const b8_t cv = __builtin_bit_cast(b8_t, cc[b][st]);
            const f4_t ta = mfma(a, first_half ? cv : zero8, f4_t{0, 0, 0, 0});
            const f4_t tb = mfma(a, first_half ? zero8 : cv, f4_t{0, 0, 0, 0});
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[m][b][r] += ds[b][2 * st] * (ta[r] - 160.0f * xa[r]) + ds[b][2 * st + 1] * (tb[r] - 160.0f * xb[r]);
          }
        }
      }
    } else {  // Q2_K with bf16: codes a*q and mins m, d and dmin on the partial sums
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        u4_t cq[2], cm;
        const float a = (float)(rw[b].x0 & 15u);
        const float mn = (float)(rw[b].x0 >> 4);
        const float dd = f16_to_f32(rw[b].x2), dm = f16_to_f32(rw[b].x3);
        const uint32_t mb16 = __builtin_bit_cast(uint32_t, mn) >> 16;
        cm = u4_t{mb16 | (mb16 << 16), mb16 | (mb16 << 16), mb16 | (mb16 << 16), mb16 | (mb16 << 16)};
        const uint32_t shift = rw[b].x1;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t t = (rw[b].v[w] >> shift) & 0x03030303u;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float lo = a * (float)((t >> (16 * h)) & 0xFFu);
            const float hi = a * (float)((t >> (16 * h + 8)) & 0xFFu);
            cq[w >> 1][2 * (w & 1) + h] = (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
          }
        }
#pragma unroll
        for (int m = 0; m < MBV; ++m) {
          if (m >= c.mbn) break;
          const uint16_t* ar = Ab + (16 * m + lr) * LDA + 16 * lg;
          const b8_t a0 = __builtin_bit_cast(b8_t, *(const u4_t*)ar);
          const b8_t a1 = __builtin_bit_cast(b8_t, *(const u4_t*)(ar + 8));
          f4_t tq = mfma(a0, __builtin_bit_cast(b8_t, cq[0]), f4_t{0, 0, 0, 0});
          tq = mfma(a1, __builtin_bit_cast(b8_t, cq[1]), tq);
          f4_t tm = mfma(a0, __builtin_bit_cast(b8_t, cm), f4_t{0, 0, 0, 0});
          tm = mfma(a1, __builtin_bit_cast(b8_t, cm), tm);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[m][b][r] = __builtin_fmaf(dd, tq[r], __builtin_fmaf(-dm, tm[r], acc[m][b][r]));
        }
      }
    }
  };

  // Two tiles per trip: ra holds tile kt, rb tile kt + 1; each is refilled with
  // the tile two ahead right after it is consumed.  Activation loads run one
  // tile ahead through registers.  Past the last tile the prefetches re-read
  // the last tile (an L2 hit), so the loop body has no branches around loads
  // and the barriers (LDS-only) never wait for the weight stream.
  const int last = KT - 1;
  Raw ra[NB], rb[NB];
  load_a(0);
#pragma unroll
  for (int b = 0; b < NB; ++b) ra[b] = load_raw<FMT, ACT>(g, c.Rb[b], 0, lg);
#pragma unroll
  for (int b = 0; b < NB; ++b) rb[b] = load_raw<FMT, ACT>(g, c.Rb[b], (int64_t)min(1, last) * BK, lg);
  store_a(0);
  load_a(min(1, last));
  for (int kt = 0; kt < KT; kt += 2) {
    lds_barrier();
    compute(kt, 0, ra);
#pragma unroll
    for (int b = 0; b < NB; ++b) ra[b] = load_raw<FMT, ACT>(g, c.Rb[b], (int64_t)min(kt + 2, last) * BK, lg);
    store_a(1);
    load_a(min(kt + 2, last));
    lds_barrier();
    if (kt + 1 < KT) compute(kt + 1, 1, rb);
#pragma unroll
    for (int b = 0; b < NB; ++b) rb[b] = load_raw<FMT, ACT>(g, c.Rb[b], (int64_t)min(kt + 3, last) * BK, lg);
    store_a(0);
    load_a(min(kt + 3, last));
  }

  // ---------------------------------------------------------------- bf16 int4 bias term
  if constexpr (INT4_BF16) {
    lds_barrier();  // row sums of every block are in xg
    const int G = (int)(g.K / g.group);
    for (int c0 = 0; c0 < G; c0 += 32) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        // B operand: (bias - 128 scale) of groups c0 + 8 lg .. + 8 of this lane's row, hi/lo bf16
        u4_t bh, bl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t h2[2], l2[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int gg = c0 + 8 * lg + 2 * i + q;
            float cb = 0.f;
            if (gg < G) {
              const uint32_t sbv = ((const uint32_t*)g.scales)[((c.Rb[b] >> 4) * G + gg) * 16 + (c.Rb[b] & 15)];
              cb = f16_to_f32(sbv >> 16) - 128.0f * f16_to_f32(sbv & 0xFFFFu);
            }
            split_hi_lo(cb, h2[q], l2[q]);
          }
          bh[i] = h2[0] | (h2[1] << 16);
          bl[i] = l2[0] | (l2[1] << 16);
        }
#pragma unroll
        for (int m = 0; m < MBV; ++m) {
          if (m >= c.mbn) break;
          const float* xr = &c.xg[(16 * m + lr) * LDX + c0 + 8 * lg];
          u4_t xh, xl;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t h2[2], l2[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const int gg = c0 + 8 * lg + 2 * i + q;
              split_hi_lo(gg < G ? xr[2 * i + q] : 0.f, h2[q], l2[q]);
            }
            xh[i] = h2[0] | (h2[1] << 16);
            xl[i] = l2[0] | (l2[1] << 16);
          }
          const b8_t XH = __builtin_bit_cast(b8_t, xh), XL = __builtin_bit_cast(b8_t, xl);
          acc[m][b] = mfma(XH, __builtin_bit_cast(b8_t, bh), acc[m][b]);
          acc[m][b] = mfma(XH, __builtin_bit_cast(b8_t, bl), acc[m][b]);
          acc[m][b] = mfma(XL, __builtin_bit_cast(b8_t, bh), acc[m][b]);
        }
      }
    }
  }

  // ---------------------------------------------------------------- epilogue
  if constexpr (EPI == QMOE_EPI_STORE || EPI == QMOE_EPI_SWIGLU) {
    // 2-byte outputs leave through the (now idle) activation tile as rows of
    // 128 output columns, then 16-byte pieces per thread, so each output row
    // is written whole and contiguous.  SwiGLU's 128 columns take one pass;
    // STORE's 256 take two (waves 0-1, then waves 2-3).
    if (g.stage_out) {
      constexpr bool swiglu = (EPI == QMOE_EPI_SWIGLU);
      constexpr int HW = 128;            // output columns per pass
      constexpr int LROW = 2 * HW + 16;  // LDS row stride in bytes
      static_assert(BM * LROW <= 2 * BM * LDA * 2, "a pass fits in the activation tile");
      const bool half = (g.out_dtype == QMOE_F16);
      uint8_t* stg = (uint8_t*)c.As;
      const int64_t nlim = swiglu ? g.N / 2 : g.N;
      const int64_t col0 = swiglu ? c.ncol[0] - 32 * wave - lr : c.ncol[0] - 64 * wave - lr;  // first column of the workgroup
#pragma unroll
      for (int h = 0; h < (swiglu ? 1 : 2); ++h) {
        __syncthreads();  // the K loop (or the previous pass) is done with the tile
        // two values per packed conversion: the wave's column blocks in pairs
        auto stage_rows = [&](auto half_c) {
          constexpr bool HALF = decltype(half_c)::value;
#pragma unroll
          for (int m = 0; m < MBV; ++m) {
            if (m >= c.mbn) break;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              uint16_t* dst = (uint16_t*)(stg + (16 * m + 4 * lg + r) * LROW);
              if constexpr (swiglu) {
                const uint32_t p = f32x2_to_16<HALF>(silu_f32(acc[m][0][r]) * acc[m][2][r],
                                                   silu_f32(acc[m][1][r]) * acc[m][3][r]);
                dst[32 * wave + lr] = (uint16_t)p;
                dst[32 * wave + 16 + lr] = (uint16_t)(p >> 16);
              } else {
#pragma unroll
                for (int b = 0; b < NB; b += 2) {
                  const uint32_t p = f32x2_to_16<HALF>(acc[m][b][r], acc[m][b + 1][r]);
                  dst[64 * (wave & 1) + 16 * b + lr] = (uint16_t)p;
                  dst[64 * (wave & 1) + 16 * (b + 1) + lr] = (uint16_t)(p >> 16);
                }
              }
            }
          }
        };
        if (swiglu || (wave >> 1) == h) {
          if (half) stage_rows(std::true_type{});
          else stage_rows(std::false_type{});
        }
        __syncthreads();
        for (int i = tid; i < c.nrows * (HW / 8); i += 256) {
          const int r = i / (HW / 8), cc = i - r * (HW / 8);
          const int64_t col = col0 + HW * h + 8 * cc;
          if (col < nlim)
            *(u4_t*)((uint16_t*)g.out + (int64_t)c.rows_o[r] * g.ldo + col) = *(const u4_t*)(stg + r * LROW + 16 * cc);
        }
      }
      return;
    }
  }
#pragma unroll
  for (int m = 0; m < MBV; ++m) {
    if (m >= c.mbn) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * m + 4 * lg + r;
      if (row >= c.nrows) continue;
      const int64_t orow = c.rows_o[row];
      if constexpr (EPI == QMOE_EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (c.nvalid[j]) store_out(g.out, g.out_dtype, orow * g.ldo + c.ncol[j], silu_f32(acc[m][j][r]) * acc[m][2 + j][r]);
      } else if constexpr (EPI == QMOE_EPI_STORE) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if (c.nvalid[b]) store_out(g.out, g.out_dtype, orow * g.ldo + c.ncol[b], acc[m][b][r]);
      } else if constexpr (EPI == QMOE_EPI_WEIGHTED_COMBINE) {
        const float w = c.wts[row];
        float* o = (float*)g.out + orow * g.ldo;
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if (c.nvalid[b]) atomicAdd(o + c.ncol[b], w * acc[m][b][r]);
      } else {  // ACCUMULATE
        float* o = (float*)g.out + orow * g.ldo;
#pragma unroll
        for (int b = 0; b < NB; ++b)
          if (c.nvalid[b]) o[c.ncol[b]] += acc[m][b][r];
      }
    }
  }
}

// MXFP4: whether every E8M0 exponent of this lane's weight rows, over all of
// K, lies in 114 .. 140 (scales 2^-13 .. 2^13), read from the 16-byte scale
// vectors of the lane's 16-row blocks (lane l checks vectors l, l + 64, ...).
// A block whose rows do not start on a 16-row boundary (clamped tail rows)
// answers false.
__device__ __forceinline__ bool mxfp4_foldable(const GemmArgs& g, const TileCtx& c) {
  const int64_t KB = g.K / 32;  // scale vectors per 16-row block
  bool ok = true;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t base = c.Rb[b] - c.lr;
    if (base & 15) {
      ok = false;
      continue;
    }
    const u4_t* run = (const u4_t*)((const uint8_t*)g.scales + (base >> 4) * KB * 16);
    for (int64_t i = c.lane; i < KB; i += 64) {
      const u4_t v = run[i];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) ok = ok && ((v[q] >> (8 * j)) & 0xFFu) - 114u <= 26u;
    }
  }
  return ok;
}

template <int FMT, int ACT, int EPI>
__global__ __launch_bounds__(256, 2) void qmm_kernel(GemmArgs g) {
  constexpr bool INT4_BF16 = (ACT == ACT_BF16 && FMT == QMOE_INT4);
  constexpr bool IQ2 = (FMT == QMOE_IQ2_XXS);

  __shared__ __attribute__((aligned(16))) uint16_t As[2 * BM * LDA];
  __shared__ int rows_a[BM];
  __shared__ int rows_o[BM];
  __shared__ float wts[BM];
  __shared__ __attribute__((aligned(16))) float xg[INT4_BF16 ? BM * LDX : 4];
  __shared__ __attribute__((aligned(16))) uint32_t lut_grid[IQ2 ? 256 * 4 : 4];
  __shared__ __attribute__((aligned(16))) uint32_t lut_sign[IQ2 ? 128 * 4 : 4];

  TileCtx c;
  c.tid = threadIdx.x;
  c.lane = c.tid & 63;
  c.wave = c.tid >> 6;
  c.lg = c.lane >> 4;
  c.lr = c.lane & 15;
  const int tid = c.tid;

  // The grid is sized for the most tiles a plan can have; blocks past the
  // plan's tiles have no work.
  // A plan whose header names another call gives no tiles.
  const int n_tiles = (g.amode == AM_DENSE) ? (int)((g.M + BM - 1) / BM)
                      : plan_matches(g.plan, g.bm, g.t, g.topk, g.E) ? g.plan[1] : 0;
  int mt, nt;
  if (!tile_of_block(blockIdx.x, n_tiles, g.n_ntiles, mt, nt)) return;

  int expert, row0, nrows;
  if (g.amode == AM_DENSE) {
    expert = 0;
    row0 = mt * BM;
    if (row0 >= g.M) return;
    nrows = (int)min<int64_t>(BM, g.M - row0);
    if (tid < BM) {
      rows_a[tid] = tid < nrows ? row0 + tid : -1;
      rows_o[tid] = row0 + tid;
      wts[tid] = 0.f;
    }
  } else {
    const PlanLayout L = plan_layout(g.P, g.E);
    const int32_t* tl = g.plan + L.tiles + 4 * (int64_t)mt;
    expert = tl[0];
    row0 = tl[1];
    nrows = min(tl[2], BM);
    if (expert < 0 || expert >= g.E) return;
    if (tid < BM) {
      int ra = -1, ro = 0;
      float wt = 0.f;
      if (tid < nrows) {
        const int pair = g.plan[L.sorted + row0 + tid];
        ra = (g.amode == AM_GATHER) ? pair / g.topk : row0 + tid;
        ro = (EPI == QMOE_EPI_WEIGHTED_COMBINE) ? pair / g.topk : row0 + tid;
        if (EPI == QMOE_EPI_WEIGHTED_COMBINE) wt = g.topk_w[pair];
      }
      rows_a[tid] = ra;
      rows_o[tid] = ro;
      wts[tid] = wt;
    }
  }
  if constexpr (IQ2) {
    // grid rows as 8 halves (fp16, or bf16 -- both exact for byte magnitudes)
    {
      const int r = tid;  // 256 rows
      const u2_t b = *(const u2_t*)(g.grid + 8 * r);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = b[i >> 1] >> (16 * (i & 1));
        float lo = (float)(w & 0xFFu), hi = (float)((w >> 8) & 0xFFu);
        uint32_t packed;
        if constexpr (ACT == ACT_F16) packed = (uint32_t)f32_to_f16(lo) | ((uint32_t)f32_to_f16(hi) << 16);
        else packed = (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
        lut_grid[4 * r + i] = packed;
      }
    }
    if (tid < 128) {
      const uint32_t m = g.signs[tid];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        lut_sign[4 * tid + i] = (((m >> (2 * i)) & 1u) << 15) | (((m >> (2 * i + 1)) & 1u) << 31);
    }
  }
  __syncthreads();

  c.As = As;
  c.rows_a = rows_a;
  c.rows_o = rows_o;
  c.wts = wts;
  c.xg = xg;
  c.lut_grid = lut_grid;
  c.lut_sign = lut_sign;
  c.nrows = nrows;

  // Weight rows of this lane for its NB column blocks.
  constexpr bool swiglu = (EPI == QMOE_EPI_SWIGLU);
  const int64_t Nh = g.N / 2;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    int64_t wrow;
    if (swiglu) {
      const int64_t j = (int64_t)nt * (BN / 2) + 32 * c.wave + 16 * (b & 1) + c.lr;
      c.ncol[b] = j;
      c.nvalid[b] = j < Nh;
      const int64_t jc = j < Nh ? j : Nh - 1;
      wrow = (b < 2) ? jc : Nh + jc;
    } else {
      const int64_t n = (int64_t)nt * BN + 64 * c.wave + 16 * b + c.lr;
      c.ncol[b] = n;
      c.nvalid[b] = n < g.N;
      wrow = n < g.N ? n : g.N - 1;
    }
    c.Rb[b] = (int64_t)expert * g.N + wrow;
  }

  c.mbn = (nrows + 15) >> 4;  // valid 16-row blocks
  if constexpr (FMT == QMOE_MXFP4 && ACT == ACT_F16) {
    if (__syncthreads_and(mxfp4_foldable(g, c))) {
      qmm_body<FMT, ACT, EPI, MB, true>(g, c);
      return;
    }
  }
  qmm_body<FMT, ACT, EPI, MB>(g, c);
}

// ------------------------------------------------------------------ int4: LDS ring
//
// int4 on the tiled layout streams both operands through a 3-stage LDS ring
// with direct-to-LDS loads (buffer/global_load ... lds), so two K tiles of
// weights and gathered activations are in flight while a third is computed,
// without holding them in registers.  A workgroup is 8 waves over 80 routed
// rows x 256 weight rows; each wave owns two 16-row weight blocks (SwiGLU: a
// gate block and the matching up block) for all 80 rows, which keeps a wave
// within 128 registers, so two workgroups (four waves per SIMD) share a CU.
// Per K tile: ten 16-byte loads of gathered activation chunks spread over the
// waves (rows past the tile read as zero), and per wave one load of its two
// weight runs (512 bytes each) and one of packed scale|bias words.  LDS-DMA
// completion is tracked by vmcnt, which the compiler does not see for these
// loads, so the waits are explicit: before tile kt is read, only tile kt+1's
// loads may still be outstanding.  One LDS-only barrier per tile publishes the
// activation chunks of all waves and frees the stage the next loads overwrite.
//
// Activation rows are stored unpadded with the 16-byte chunks of row r
// permuted by c ^ ((r ^ (r >> 3)) & 7), so the rows an MFMA fragment read
// touches land in distinct 16-byte bank groups whether the LDS serves 8 or 16
// lanes of a 16-byte read per cycle.

constexpr int RW = 8;                      // waves per workgroup
constexpr int RNB = 2;                     // 16-row weight blocks per wave
constexpr int RS = 3;                      // ring stages
constexpr int R_ACH = BM * 8;              // activation chunks per stage (640)
constexpr int R_A = R_ACH * 16;            // 10240 B
// then per wave the weight codes of its RNB blocks (1 KB; FP8 and Q8_0: 2 KB)
// and the scale / metadata region (256 bytes; Q4_K 512, FP8 none), so a stage
// is 20480 bytes for int4 (see ring_body)
constexpr int XG4 = 32;                    // int4 groups per row kept for the bf16 bias term

// Chunk swizzle of the activation rows in a ring stage (rows 128 bytes
// apart share banks every 8 rows).  It depends on r % 16 only, so the rows
// of MFMA sub-tile m sit at a constant offset (2048 m bytes) from those of
// sub-tile 0 and the reads use immediate offsets.
__device__ __forceinline__ int ring_swz(int r) { return ((r & 15) ^ ((r >> 3) & 1)) & 7; }
__device__ __forceinline__ int ring_slot(int r, int c) { return r * 8 + (c ^ ring_swz(r)); }


// Workgroup barrier for the ring: drains this wave's LDS instructions
// (lgkmcnt) but not its vector-memory loads, which include the ring's own
// LDS-DMA transfers (their completion is waited for explicitly, per tile).  A
// release fence would wait for every outstanding load.  The empty asm
// statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The work of workgroup b of the int4 ring kernel.  Workgroup b runs on XCD
// x = b & 7 as the j-th of that XCD (b = 8j + x) and XCD x owns tiles x,
// x + 8, ...: its units are (tile, column block) pairs u = q * n_nt + nt of
// tile x + 8q.  With sx workgroups resident per XCD, the units past the
// XCD's last whole round (at most a quarter round of them) would take one
// more round by themselves; each is split instead into SK_PARTS parts along
// K (when every part keeps at least 4 K tiles), dealt after the whole units
// so they go to the workgroup slots that free first.  Returns false when b
// has no work.
constexpr int SK_PARTS = 4;
struct Work {
  int mt, nt, kb, ke;
  int part;   // K part of a split unit (-1: a whole unit)
  int pslot;  // the part's partial-tile slot (the unit's parts are pslot - part .. + SK_PARTS - 1)
  int tslot;  // the unit's ticket
};
__device__ __forceinline__ bool work_of_block(int b, int n_tiles, int n_nt, int KT, int sx, Work& w) {
  const int x = b & 7, j = b >> 3;
  const int nq = n_tiles > x ? (n_tiles - x + 7) >> 3 : 0;
  const int ux = nq * n_nt;
  int R = 0;
  if (sx > 0 && sx <= 64 && ux > sx && KT >= 4 * SK_PARTS) {
    R = ux % sx;
    if (R * SK_PARTS > sx) R = 0;
  }
  int u;
  w.kb = 0;
  w.ke = KT;
  w.part = -1;
  w.pslot = w.tslot = 0;
  if (j < ux - R) {
    u = j;
  } else {
    const int i = j - (ux - R);  // part i % SK_PARTS of split unit i / SK_PARTS
    if (i >= R * SK_PARTS) return false;
    u = ux - R + i / SK_PARTS;
    w.part = i % SK_PARTS;
    w.kb = w.part * KT / SK_PARTS;
    w.ke = (w.part + 1) * KT / SK_PARTS;
    w.pslot = 64 * x + i;
    w.tslot = 16 * x + i / SK_PARTS;
  }
  const int q = u / n_nt;
  w.mt = x + 8 * q;
  w.nt = u - q * n_nt;
  return true;
}

// The ring kernel's body for int4 (either activation type) and for IQ2_XXS
// and Q2_K with fp16 activations.  IQ2_XXS on the tiled layout has one
// contiguous 256-byte run per 16-row block and K tile (two 32-value groups of
// (index word, aux word) pairs) and one fp16 d per row and 256-value
// super-block; the magnitudes and sign masks are expanded into LDS tables
// once per workgroup, as in the generic kernel.  Q2_K keeps a 16-row block's
// codes of one super-block as two contiguous 512-byte halves (16 rows x 32
// bytes, four 2-bit fields per byte), each holding two K tiles; the tile
// reads its half (the odd tile of a pair fetches it again, from L2) and the
// row's four scale|min bytes, d and dmin.
template <int FMT, int ACT, int EPI>
__device__ __forceinline__ void ring_body(const GemmArgs& g) {
  constexpr bool BF = (ACT == ACT_BF16);
  constexpr bool IQ2 = (FMT == QMOE_IQ2_XXS);
  constexpr bool Q2K = (FMT == QMOE_Q2_K);
  constexpr bool MX = (FMT == QMOE_MXFP4);
  constexpr bool Q4K = (FMT == QMOE_Q4_K);
  constexpr bool Q6K = (FMT == QMOE_Q6_K);
  constexpr bool F8 = (FMT == QMOE_FP8);
  constexpr bool Q8 = (FMT == QMOE_Q8_0);
  static_assert(FMT == QMOE_INT4 || ((IQ2 || Q2K || MX || Q4K || Q6K || F8 || Q8) && !BF),
                "ring formats: int4, and IQ2_XXS, Q2_K, MXFP4, Q4_K, Q6_K, FP8, Q8_0 with fp16 activations");
  // weight codes per wave and stage (FP8: two 1 KB blocks), then metadata: one
  // 64-lane dword load (Q4_K: two; FP8: none, its block scales are
  // wave-uniform and come by scalar loads).  NMETA + 1 loads per wave and
  // tile besides the activation chunks.
  constexpr int BW = (F8 || Q8) ? 2048 : 1024;
  constexpr int RBB = RW * BW;
  constexpr int NMETA = Q4K ? 2 : 1;
  constexpr int SBW = F8 ? 0 : 256 * NMETA;
  constexpr int STAGE = R_A + RBB + RW * SBW;
  // Q8_0's 28 KB stages fit two workgroups per CU only as two stages (one
  // tile in flight while one is computed); the others keep three
  constexpr int NST = Q8 ? 2 : RS;
  __shared__ __attribute__((aligned(16))) uint8_t ring[NST * STAGE];
  __shared__ int rows_a[BM];
  __shared__ int rows_o[BM];
  __shared__ float wts[BM];
  __shared__ __attribute__((aligned(16))) float xg[BF ? XG4 * BM : 4];  // [group][row] activation sums
  __shared__ __attribute__((aligned(16))) uint32_t lut_grid[IQ2 ? 256 * 4 : 4];
  __shared__ uint32_t lut_sbit[IQ2 ? 128 : 1];  // sign byte in both halves
  // Q6_K: the top-bit halves of two tile pairs (slot p & 1 holds pair p's
  // 512 bytes per 16-row block, per wave), outside the ring stages
  __shared__ __attribute__((aligned(16))) uint8_t qh_ring[Q6K ? 2 * RW * 1024 : 16];
  __shared__ int sk_arrival;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lg = lane >> 4, lr = lane & 15;

  // The grid is sized for the most tiles a plan can have; blocks past the
  // plan's tiles have no work.
  // A plan whose header names another call gives no tiles.
  const int n_tiles = (g.amode == AM_DENSE) ? (int)((g.M + BM - 1) / BM)
                      : plan_matches(g.plan, g.bm, g.t, g.topk, g.E) ? g.plan[1] : 0;
  const int KT = (int)(g.K >> 6);
  const bool split_ok = g.amode != AM_DENSE && g.sk_tickets != nullptr && g.plan[7] == SK_SLOTS;
  Work wk;
  if (!work_of_block(blockIdx.x, n_tiles, g.n_ntiles, KT, split_ok ? g.sk_slots_xcd : 0, wk)) return;
  const int mt = wk.mt, nt = wk.nt;

  int expert, nrows;
  if (g.amode == AM_DENSE) {
    expert = 0;
    const int64_t row0 = (int64_t)mt * BM;
    nrows = (int)min<int64_t>(BM, g.M - row0);
    if (tid < BM) {
      rows_a[tid] = tid < nrows ? (int)(row0 + tid) : -1;
      rows_o[tid] = (int)(row0 + tid);
      wts[tid] = 0.f;
    }
  } else {
    const PlanLayout L = plan_layout(g.P, g.E);
    const int32_t* tl = g.plan + L.tiles + 4 * (int64_t)mt;
    expert = tl[0];
    const int row0 = tl[1];
    nrows = min(tl[2], BM);
    if (expert < 0 || expert >= g.E) return;
    if (tid < BM) {
      int ra = -1, ro = 0;
      float wt = 0.f;
      if (tid < nrows) {
        const int pair = g.plan[L.sorted + row0 + tid];
        ra = (g.amode == AM_GATHER) ? pair / g.topk : row0 + tid;
        ro = (EPI == QMOE_EPI_WEIGHTED_COMBINE) ? pair / g.topk : row0 + tid;
        if (EPI == QMOE_EPI_WEIGHTED_COMBINE) wt = g.topk_w[pair];
      }
      rows_a[tid] = ra;
      rows_o[tid] = ro;
      wts[tid] = wt;
    }
  }
  if constexpr (IQ2) {
    if (tid < 256) {  // grid row tid as 8 fp16 magnitudes
      const u2_t b = *(const u2_t*)(g.grid + 8 * tid);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = b[i >> 1] >> (16 * (i & 1));
        lut_grid[4 * tid + i] = (uint32_t)f32_to_f16((float)(w & 0xFFu)) | ((uint32_t)f32_to_f16((float)((w >> 8) & 0xFFu)) << 16);
      }
    } else if (tid < 384) {
      const uint32_t m = g.signs[tid - 256];
      lut_sbit[tid - 256] = m | (m << 16);
    }
  }
  __syncthreads();
  const int mbn = (nrows + 15) >> 4;

  // The wave's two 16-row weight blocks: all rows of a block are valid or
  // none are (N is a multiple of 16, and of 32 with SwiGLU); invalid blocks
  // read a valid block and are not stored.
  constexpr bool swiglu = (EPI == QMOE_EPI_SWIGLU);
  const int64_t Nh = g.N / 2;
  auto col0 = [&](int b) -> int64_t {  // first output column of block b
    return swiglu ? (int64_t)nt * (BN / 2) + 16 * wave : (int64_t)nt * BN + 32 * wave + 16 * b;
  };
  auto block_base = [&](int b) -> int64_t {  // first weight row of block b (clamped)
    if (swiglu) {
      const int64_t j0 = col0(b);
      const int64_t jc = j0 < Nh ? j0 : Nh - 16;
      return b == 0 ? jc : Nh + jc;
    }
    const int64_t n0 = col0(b);
    return n0 < g.N ? n0 : g.N - 16;
  };
  int64_t ncol[RNB];
  bool nvalid[RNB];
  int64_t rbk[RNB];  // run (16-row block) index of each block
#pragma unroll
  for (int b = 0; b < RNB; ++b) {
    ncol[b] = col0(b) + lr;
    nvalid[b] = col0(b) < (swiglu ? Nh : g.N);
    rbk[b] = ((int64_t)expert * g.N + block_base(b)) >> 4;
  }

  // int4 (group >= 64): tile kt lies in scale group kt >> gsh; IQ2_XXS and
  // Q2_K: in super-block kt >> 2; MXFP4: the tile holds two 32-value blocks
  // (its own 32 exponent bytes per 16-row block)
  const int gsh = (IQ2 || Q2K || Q4K || Q6K) ? 2 : (MX || Q8) ? 0 : __builtin_ctz((unsigned)g.group) - 6;
  const int64_t K = g.K;
  const int T = KT, G = T >> gsh;

  // ---- per-lane load descriptors
  // activation chunks: load j (0..9) fills slots 64j .. 64j+63; wave w issues
  // loads w and w + 8
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc((void*)g.a, (short)0, (int)g.a_bytes, 0x00020000);
  const int n_aload = (wave + RW < R_ACH / 64) ? 2 : 1;
  uint32_t aoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = 64 * (wave + RW * i) + lane;  // LDS chunk slot this lane fills
    const int r = p >> 3, c = (p & 7) ^ ring_swz(r);
    const int src = (r < 16 * mbn && p < R_ACH) ? rows_a[min(r, BM - 1)] : -1;
    aoff[i] = src >= 0 ? (uint32_t)((int64_t)src * K * 2 + 16 * c) : 0x80000000u;
  }
  // int4 weight runs (512 bytes per block and K tile): lanes 0-31 block 0,
  // lanes 32-63 block 1; scale|bias words (64 bytes per block and group):
  // lanes 0-15 block 0, 16-31 block 1 (lanes 32-63 repeat them).  IQ2_XXS
  // runs (256 bytes): lanes 0-15 block 0, 16-31 block 1; d halves (32 bytes
  // per block and super-block): lanes 0-7 block 0, 8-15 block 1 (the other
  // lanes repeat them into unused LDS).  Q2_K runs (512 bytes per block and
  // pair of K tiles, so 256 per tile on average) and MXFP4 runs (512 bytes)
  // as int4's; MXFP4 exponents (32 bytes per block and tile) as IQ2_XXS's d
  // halves.  The base (block
  // 0's run) is wave-uniform and lives in SGPRs; each lane adds a 32-bit byte
  // offset (block 1's run lies at most one expert's codes further)
  constexpr int WRUN = IQ2 ? 256 : Q2K ? 256 : (F8 || Q8) ? 1024 : 512, SRUN = (IQ2 || MX) ? 32 : 64;
  const int64_t rb0 = ((int64_t)expert * g.N + block_base(0)) >> 4;
  const int64_t rb1 = ((int64_t)expert * g.N + block_base(1)) >> 4;
  const uint8_t* wbase = (const uint8_t*)g.qs + rb0 * T * WRUN;
  const uint32_t woff = IQ2 ? (uint32_t)(((lane >> 4) & 1) * (rb1 - rb0) * T * WRUN + (lane & 15) * 16)
                            : (uint32_t)((lane >> 5) * (rb1 - rb0) * T * WRUN + (lane & 31) * 16);
  const uint8_t* sbase = (const uint8_t*)(IQ2 ? g.d : g.scales) + rb0 * G * SRUN;
  const uint32_t soff = (IQ2 || MX) ? (uint32_t)(((lane >> 3) & 1) * (rb1 - rb0) * G * SRUN + (lane & 7) * 4)
                            : (uint32_t)(((lane >> 4) & 1) * (rb1 - rb0) * G * SRUN + lr * 4);
  // MXFP4: whether every exponent of the workgroup's weight rows (all of K)
  // lets the scale go into the B operand exactly (2^-13 .. 2^13)
  bool fold = true;
  if constexpr (MX) {
    const int64_t KB = K / 32;  // 16-byte exponent vectors per 16-row block
    bool ok = true;
#pragma unroll
    for (int b = 0; b < RNB; ++b) {
      const u4_t* run_e = (const u4_t*)((const uint8_t*)g.scales + (b ? rb1 : rb0) * KB * 16);
      for (int64_t i = lane; i < KB; i += 64) {
        const u4_t v = run_e[i];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int j = 0; j < 4; ++j) ok = ok && ((v[q] >> (8 * j)) & 0xFFu) - 114u <= 26u;
      }
    }
    fold = __syncthreads_and(ok);
  }

  // Q2_K metadata of a tile, 256 bytes per wave from three arrays, so each
  // lane keeps its own 64-bit address: lanes 0-15 (16-31) take row lr's four
  // scale|min bytes of the tile's sub-blocks in block 0 (1), at 256 bytes per
  // super-block and 4 per tile; lanes 32-47 (48-63) take block 0's (1's) d
  // then dmin halves, two rows per lane, at 32 bytes per super-block.
  // Q4_K: load 1, lanes 0-15 (16-31) take row lr's scale word and
  // 32-47 (48-63) its min word holding the tile's two sub-blocks (word
  // (kt >> 1) & 1 of the row's 8 scales, resp. mins), block 0 then block 1;
  // load 2, lanes 0-7 (8-15) block 0's d (dmin) halves, 16-31 block 1's (the
  // upper lanes repeat them into unused LDS).
  const uint8_t* mptr = nullptr;
  const uint8_t* mptr2 = nullptr;
  uint32_t mstride = 0, minc = 0;
  if constexpr (Q4K) {
    const int64_t rb = (lane >> 5) ? rb1 : rb0;
    mptr = (const uint8_t*)g.scales + rb * G * 256 + lr * 16 + ((lane >> 4) & 1) * 8;
    const int i = lane & 31;
    const int64_t rb2 = (i >> 4) ? rb1 : rb0;
    mptr2 = (const uint8_t*)(((i >> 3) & 1) ? g.dmin : g.d) + rb2 * G * 32 + (i & 7) * 4;
  }
  // FP8: a 16-row block's codes of a tile are 1 KB (the Q8_0 tiling), one
  // 16-byte load per lane and block; the block's scale (its 128 x 128 scale
  // block's) by a scalar load per tile
  // (Q8_0 takes the same two code loads; its fp16 scales, 64 bytes per block
  // and tile, come as int4's scale words do)
  uint32_t woff2 = 0;
  if constexpr (F8 || Q8) woff2 = (uint32_t)((rb1 - rb0) * T * 1024 + lane * 16);
  const __attribute__((address_space(4))) float* fsc[RNB] = {nullptr, nullptr};
  if constexpr (F8) {
#pragma unroll
    for (int b = 0; b < RNB; ++b) {
      const int64_t si = (((int64_t)expert * g.N + block_base(b)) >> 7) * (K >> 7);
      fsc[b] = (const __attribute__((address_space(4))) float*)(uintptr_t)sgpr_ptr((const float*)g.scales + si);
    }
  }
  // Q6_K: lanes 0-31 as Q2_K's (the tile's four int8 sub-block scales of a
  // row), lanes 32-39 (40-47) block 0's (1's) d halves, 48-63 repeat them.
  // Its top-bit halves (512 bytes per block and tile pair) go by a 16-byte
  // load per lane into qh_ring for the first tile of a pair (and the first
  // tile of a K part): lanes 0-31 block 0, 32-63 block 1.
  const uint8_t* qbase = nullptr;
  uint32_t qoff = 0;
  if constexpr (Q6K) {
    if (lane < 32) {
      mptr = (const uint8_t*)g.scales + ((lane >> 4) ? rb1 : rb0) * G * 256 + lr * 16;
      mstride = 256;
      minc = 4;
    } else {
      mptr = (const uint8_t*)g.d + (((lane & 15) >> 3) ? rb1 : rb0) * G * 32 + (lane & 7) * 4;
      mstride = 32;
    }
    qbase = (const uint8_t*)g.aux + rb0 * T * 256;
    qoff = (uint32_t)((lane >> 5) * (rb1 - rb0) * T * 256 + (lane & 31) * 16);
  }
  if constexpr (Q2K) {
    const int b = lane < 32 ? (lane >> 4) : ((lane - 32) >> 4);
    const int64_t rb = b ? rb1 : rb0;
    if (lane < 32) {
      mptr = (const uint8_t*)g.scales + rb * G * 256 + lr * 16;
      mstride = 256;
      minc = 4;
    } else {
      const int i = lane & 15;
      mptr = (const uint8_t*)(i < 8 ? g.d : g.dmin) + rb * G * 32 + (i & 7) * 4;
      mstride = 32;
    }
  }

  // issue tile kt into ring stage `stage` (kt % RS, tracked by the caller);
  // `first`: the first tile of the K range
  auto issue = [&](int kt, int stage, bool first) {
    const uint32_t st = lds_addr(ring) + (uint32_t)(stage * STAGE);
    dma_buf16(arsrc, st + 64 * 16 * wave, aoff[0] + (uint32_t)kt * 128);
    if (n_aload == 2) dma_buf16(arsrc, st + 64 * 16 * (wave + RW), aoff[1] + (uint32_t)kt * 128);
    if constexpr (Q2K) {
      dma_glb16_s(wbase + (int64_t)(kt >> 1) * 512, woff, st + R_A + wave * BW);
      dma_glb4(mptr + (uint32_t)(kt >> 2) * mstride + (uint32_t)(kt & 3) * minc, st + R_A + RBB + wave * SBW);
    } else if constexpr (F8 || Q8) {
      dma_glb16_s(wbase + (int64_t)kt * WRUN, (uint32_t)lane * 16, st + R_A + wave * BW);
      dma_glb16_s(wbase + (int64_t)kt * WRUN, woff2, st + R_A + wave * BW + 1024);
      if constexpr (Q8) dma_glb4_s(sbase + (int64_t)kt * SRUN, soff, st + R_A + RBB + wave * SBW);
    } else if constexpr (Q6K) {
      dma_glb16_s(wbase + (int64_t)kt * WRUN, woff, st + R_A + wave * BW);
      dma_glb4(mptr + (uint32_t)(kt >> 2) * mstride + (uint32_t)(kt & 3) * minc, st + R_A + RBB + wave * SBW);
      if (!(kt & 1) || first)
        dma_glb16_s(qbase + (int64_t)(kt >> 1) * 512, qoff,
                    lds_addr(qh_ring) + (uint32_t)(((kt >> 1) & 1) * RW * 1024 + wave * 1024));
    } else if constexpr (Q4K) {
      dma_glb16_s(wbase + (int64_t)kt * WRUN, woff, st + R_A + wave * BW);
      dma_glb4(mptr + (uint32_t)(kt >> 2) * 256 + (uint32_t)((kt >> 1) & 1) * 4, st + R_A + RBB + wave * SBW);
      dma_glb4(mptr2 + (uint32_t)(kt >> 2) * 32, st + R_A + RBB + wave * SBW + 256);
    } else {
      dma_glb16_s(wbase + (int64_t)kt * WRUN, woff, st + R_A + wave * BW);
      dma_glb4_s(sbase + (int64_t)(kt >> gsh) * SRUN, soff, st + R_A + RBB + wave * SBW);
    }
  };

  // The K loop and epilogue for a tile of exactly MBV 16-row blocks (a
  // compile-time count keeps the m loops straight-line, so MFMA results are
  // consumed late enough to need no pipeline stalls).
  auto run = [&](auto mbv_c, auto part_c, auto fold_c) {
    constexpr bool FOLD = decltype(fold_c)::value;  // MXFP4: the scales go into the B operand
    constexpr int MBV = decltype(mbv_c)::value;
    constexpr bool PART = decltype(part_c)::value;  // a K part of a split unit (whole units keep the plain loop)
    const int kb = PART ? wk.kb : 0, ke = PART ? wk.ke : KT;
    f4_t acc[MBV][RNB];
#pragma unroll
    for (int m = 0; m < MBV; ++m)
#pragma unroll
      for (int b = 0; b < RNB; ++b) acc[m][b] = f4_t{0, 0, 0, 0};

    // chunk slots of this lane's activation reads in MFMA sub-tile 0 (sub-tile
    // m adds 128 m: the swizzle depends on the row mod 16 only)
    // (MXFP4 takes the plain k order: MFMA step s covers values 32s .. 32s+31,
    // lane group lg its chunk 4s + lg)
    const int slot_a0 = MX ? ring_slot(lr, lg) : ring_slot(lr, 2 * lg);
    const int slot_a1 = MX ? ring_slot(lr, 4 + lg) : ring_slot(lr, 2 * lg + 1);
    auto compute = [&](int kt, int stage) {
      const uint8_t* st = ring + stage * STAGE;
      const uint16_t* As = (const uint16_t*)st;
      const uint32_t* Bs = (const uint32_t*)(st + R_A + wave * BW);
      const uint32_t* Ss = (const uint32_t*)(st + R_A + RBB + wave * SBW);
      if constexpr (IQ2) {
        // lane group lg takes group lg >> 1 of the tile (its octets 2(lg & 1),
        // +1).  The octet's eight sign bits come from a 128-word table (the
        // sign byte in both halves); pair i's two bits are shifted to the
        // halves' fp16 sign positions in registers and inserted into the
        // (positive) magnitudes, which keeps the LDS reads per octet at one
        // 16-byte grid row and one word.
        const uint16_t* Ds = (const uint16_t*)Ss;
        u4_t bf[RNB][2];
#pragma unroll
        for (int b = 0; b < RNB; ++b) {
          const u2_t p = *(const u2_t*)(Bs + b * 64 + (lg >> 1) * 32 + lr * 2);
          const uint32_t idx = p[0], aux = p[1];
          const float bs = __builtin_fmaf((float)(aux >> 28), 0.25f, 0.125f);
          const _Float16 dbh = (_Float16)(f16_to_f32(Ds[b * 16 + lr]) * bs);
          const h2_t db2 = h2_t{dbh, dbh};
          const int j0 = 2 * (lg & 1);
#pragma unroll
          for (int o = 0; o < 2; ++o) {
            const int j = j0 + o;
            const u4_t row = *(const u4_t*)(lut_grid + 4 * __builtin_amdgcn_ubfe(idx, 8 * j, 8));
            const s2u_t sb = __builtin_bit_cast(s2u_t, lut_sbit[__builtin_amdgcn_ubfe(aux, 7 * j, 7)]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t sm = __builtin_bit_cast(uint32_t, sb << s2u_t{(uint16_t)(15 - 2 * i), (uint16_t)(14 - 2 * i)});
              const uint32_t w = (sm & 0x80008000u) | (row[i] & 0x7FFF7FFFu);
              bf[b][o][i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, w) * db2);
            }
          }
        }
#pragma unroll
        for (int m = 0; m < MBV; ++m) {
          const h8_t a0 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a0 + 128 * m)));
          const h8_t a1 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a1 + 128 * m)));
#pragma unroll
          for (int b = 0; b < RNB; ++b) {
            acc[m][b] = mfma(a0, __builtin_bit_cast(h8_t, bf[b][0]), acc[m][b]);
            acc[m][b] = mfma(a1, __builtin_bit_cast(h8_t, bf[b][1]), acc[m][b]);
          }
        }
        return;
      }
      if constexpr (MX) {
        // word lg of each 32-value block of row lr: eight E2M1 codes.  When
        // every exponent of the workgroup's weight rows lies in 2^-13 ..
        // 2^13 (FOLD) each code times its scale is an exact fp16 normal
        // number, so the scale goes into the hardware conversion and the
        // MFMAs accumulate directly; otherwise the exact codes enter the
        // MFMAs and the scale multiplies the fp32 partial sums.
        const uint8_t* Es = (const uint8_t*)Ss;  // [block][32-value block j][row] exponents
        uint32_t wd[RNB][2], ex[RNB][2];
#pragma unroll
        for (int b = 0; b < RNB; ++b)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            wd[b][j] = Bs[b * 128 + j * 64 + lr * 4 + lg];
            ex[b][j] = Es[b * 32 + j * 16 + lr];
          }
        if constexpr (FOLD) {
          u4_t bf[RNB][2];
#pragma unroll
          for (int b = 0; b < RNB; ++b)
#pragma unroll
            for (int j = 0; j < 2; ++j) bf[b][j] = fp4x8_pairs_scaled<ACT_F16>(wd[b][j], e8m0_to_f32(ex[b][j]));
#pragma unroll
          for (int m = 0; m < MBV; ++m) {
            const h8_t a0 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a0 + 128 * m)));
            const h8_t a1 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a1 + 128 * m)));
#pragma unroll
            for (int b = 0; b < RNB; ++b) {
              acc[m][b] = mfma(a0, __builtin_bit_cast(h8_t, bf[b][0]), acc[m][b]);
              acc[m][b] = mfma(a1, __builtin_bit_cast(h8_t, bf[b][1]), acc[m][b]);
            }
          }
        } else {
          u4_t cc[RNB][2];
          float dd[RNB][2];
#pragma unroll
          for (int b = 0; b < RNB; ++b)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              cc[b][j] = fp4x8_pairs<ACT_F16>(wd[b][j]);
              dd[b][j] = e8m0_to_f32(ex[b][j]);
            }
#pragma unroll
          for (int m = 0; m < MBV; ++m) {
            const h8_t a0 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a0 + 128 * m)));
            const h8_t a1 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a1 + 128 * m)));
#pragma unroll
            for (int b = 0; b < RNB; ++b) {
              const f4_t t0 = mfma(a0, __builtin_bit_cast(h8_t, cc[b][0]), f4_t{0, 0, 0, 0});
              const f4_t t1 = mfma(a1, __builtin_bit_cast(h8_t, cc[b][1]), f4_t{0, 0, 0, 0});
#pragma unroll
              for (int rr = 0; rr < 4; ++rr)
                acc[m][b][rr] = __builtin_fmaf(dd[b][1], t1[rr], __builtin_fmaf(dd[b][0], t0[rr], acc[m][b][rr]));
            }
          }
        }
        return;
      }
      if constexpr (Q8) {
        // chunk order: lane group lg takes chunk lg (values 16 lg .. +15) of
        // row lr and the d of its 32-value block lg >> 1
        const uint16_t* Dh = (const uint16_t*)Ss;  // [block][32-value block][row] fp16 d
        u4_t bf[RNB][2];
#pragma unroll
        for (int b = 0; b < RNB; ++b) {
          Raw rw;
          rw.v = *(const u4_t*)((const uint8_t*)Bs + b * 1024 + 256 * lg + 16 * lr);
          rw.x0 = Dh[b * 32 + (lg >> 1) * 16 + lr];
          frag_f16<QMOE_Q8_0>(rw, lg, nullptr, nullptr, bf[b][0], bf[b][1]);
        }
#pragma unroll
        for (int m = 0; m < MBV; ++m) {
          const h8_t a0 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a0 + 128 * m)));
          const h8_t a1 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a1 + 128 * m)));
#pragma unroll
          for (int b = 0; b < RNB; ++b) {
            acc[m][b] = mfma(a0, __builtin_bit_cast(h8_t, bf[b][0]), acc[m][b]);
            acc[m][b] = mfma(a1, __builtin_bit_cast(h8_t, bf[b][1]), acc[m][b]);
          }
        }
        return;
      }
      if constexpr (F8) {
        // chunk order: lane group lg takes chunk lg (values 16 lg .. +15) of
        // row lr; the E4M3 values enter the MFMAs exactly and the block scale
        // multiplies the tile's fp32 partial sums
        u4_t cc[RNB][2];
        float fs[RNB];
#pragma unroll
        for (int b = 0; b < RNB; ++b) {
          const u4_t v = *(const u4_t*)((const uint8_t*)Bs + b * 1024 + 256 * lg + 16 * lr);
          const u2_t p0 = fp8x4_pairs<ACT_F16>(v[0]), p1 = fp8x4_pairs<ACT_F16>(v[1]);
          const u2_t p2 = fp8x4_pairs<ACT_F16>(v[2]), p3 = fp8x4_pairs<ACT_F16>(v[3]);
          cc[b][0] = u4_t{p0[0], p0[1], p1[0], p1[1]};
          cc[b][1] = u4_t{p2[0], p2[1], p3[0], p3[1]};
          fs[b] = fsc[b][kt >> 1];
        }
#pragma unroll
        for (int m = 0; m < MBV; ++m) {
          const h8_t a0 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a0 + 128 * m)));
          const h8_t a1 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a1 + 128 * m)));
#pragma unroll
          for (int b = 0; b < RNB; ++b) {
            f4_t t = mfma(a0, __builtin_bit_cast(h8_t, cc[b][0]), f4_t{0, 0, 0, 0});
            t = mfma(a1, __builtin_bit_cast(h8_t, cc[b][1]), t);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[m][b][rr] = __builtin_fmaf(fs[b], t[rr], acc[m][b][rr]);
          }
        }
        return;
      }
      if constexpr (Q6K) {
        // lane group lg takes sub-block 4 (kt & 3) + lg: low bits as Q4_K's
        // (bytes 16 (lg & 1) .. +15, nibble lg >> 1), top bits from the same
        // bytes of the pair's half, bit pair 2 (kt & 1) + (lg >> 1)
        const uint8_t* Sc8 = (const uint8_t*)Ss;         // [block][row][4] int8 scales
        const uint16_t* Dh = (const uint16_t*)Ss + 64;   // [block][16] d
        const uint8_t* QH = qh_ring + ((kt >> 1) & 1) * (RW * 1024) + wave * 1024;
        u4_t bf[RNB][2];
#pragma unroll
        for (int b = 0; b < RNB; ++b) {
          Raw rw;
          rw.v = *(const u4_t*)((const uint8_t*)Bs + b * 512 + lr * 32 + 16 * (lg & 1));
          rw.v2 = *(const u4_t*)(QH + b * 512 + lr * 32 + 16 * (lg & 1));
          rw.x0 = Sc8[b * 64 + lr * 4 + lg];
          rw.x1 = 4u * (uint32_t)(lg >> 1) | ((2u * (2u * (uint32_t)(kt & 1) + (uint32_t)(lg >> 1))) << 8);
          rw.x2 = Dh[b * 16 + lr];
          frag_f16<QMOE_Q6_K>(rw, lg, nullptr, nullptr, bf[b][0], bf[b][1]);
        }
#pragma unroll
        for (int m = 0; m < MBV; ++m) {
          const h8_t a0 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a0 + 128 * m)));
          const h8_t a1 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a1 + 128 * m)));
#pragma unroll
          for (int b = 0; b < RNB; ++b) {
            acc[m][b] = mfma(a0, __builtin_bit_cast(h8_t, bf[b][0]), acc[m][b]);
            acc[m][b] = mfma(a1, __builtin_bit_cast(h8_t, bf[b][1]), acc[m][b]);
          }
        }
        return;
      }
      if constexpr (Q4K) {
        // the tile is quarter kt & 3 of the super-block: lane group lg takes
        // bytes 16 (lg & 1) .. +15 of the row's 32, low nibbles (sub-block
        // 2 (kt & 3)) for lg < 2, high nibbles (the next sub-block) above
        const uint8_t* M8 = (const uint8_t*)Ss;             // [block][scale words, min words][row][4]
        const uint16_t* Dh = (const uint16_t*)Ss + 128;     // [block][d, dmin][16]
        u4_t bf[RNB][2];
#pragma unroll
        for (int b = 0; b < RNB; ++b) {
          Raw rw;
          rw.v = *(const u4_t*)((const uint8_t*)Bs + b * 512 + lr * 32 + 16 * (lg & 1));
          const int sj = b * 128 + lr * 4 + 2 * (kt & 1) + (lg >> 1);
          rw.x0 = (uint32_t)M8[sj] | ((uint32_t)M8[sj + 64] << 8);
          rw.x1 = 4u * (uint32_t)(lg >> 1);
          rw.x2 = Dh[b * 32 + lr];
          rw.x3 = Dh[b * 32 + 16 + lr];
          frag_f16<QMOE_Q4_K>(rw, lg, nullptr, nullptr, bf[b][0], bf[b][1]);
        }
#pragma unroll
        for (int m = 0; m < MBV; ++m) {
          const h8_t a0 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a0 + 128 * m)));
          const h8_t a1 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a1 + 128 * m)));
#pragma unroll
          for (int b = 0; b < RNB; ++b) {
            acc[m][b] = mfma(a0, __builtin_bit_cast(h8_t, bf[b][0]), acc[m][b]);
            acc[m][b] = mfma(a1, __builtin_bit_cast(h8_t, bf[b][1]), acc[m][b]);
          }
        }
        return;
      }
      if constexpr (Q2K) {
        // lane group lg takes sub-block 4 (kt & 3) + lg: bytes 16 (lg & 1) ..
        // +15 of the row's half, 2-bit field 2 (kt & 1) + (lg >> 1)
        const uint8_t* Sc = (const uint8_t*)Ss;          // [block][row][4] scale|min bytes
        const uint16_t* Dh = (const uint16_t*)Ss + 64;   // [block][d, dmin][16]
        const uint32_t shift = 4u * (uint32_t)(kt & 1) + 2u * (uint32_t)(lg >> 1);
        u4_t bf[RNB][2];
#pragma unroll
        for (int b = 0; b < RNB; ++b) {
          Raw rw;
          rw.v = *(const u4_t*)((const uint8_t*)Bs + b * 512 + lr * 32 + 16 * (lg & 1));
          rw.x0 = Sc[b * 64 + lr * 4 + lg];
          rw.x1 = shift;
          rw.x2 = Dh[b * 32 + lr];
          rw.x3 = Dh[b * 32 + 16 + lr];
          frag_f16<QMOE_Q2_K>(rw, lg, nullptr, nullptr, bf[b][0], bf[b][1]);
        }
#pragma unroll
        for (int m = 0; m < MBV; ++m) {
          const h8_t a0 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a0 + 128 * m)));
          const h8_t a1 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a1 + 128 * m)));
#pragma unroll
          for (int b = 0; b < RNB; ++b) {
            acc[m][b] = mfma(a0, __builtin_bit_cast(h8_t, bf[b][0]), acc[m][b]);
            acc[m][b] = mfma(a1, __builtin_bit_cast(h8_t, bf[b][1]), acc[m][b]);
          }
        }
        return;
      }
      u2_t q[RNB];
      uint32_t sbv[RNB];
#pragma unroll
      for (int b = 0; b < RNB; ++b) {
        q[b] = *(const u2_t*)(Bs + b * 128 + lane * 2);
        sbv[b] = Ss[b * 16 + lr];
      }
      if constexpr (!BF) {
        u4_t bf[RNB][2];
#pragma unroll
        for (int b = 0; b < RNB; ++b) {
          Raw rw;
          rw.v[0] = q[b][0];
          rw.v[1] = q[b][1];
          rw.x0 = sbv[b];
          frag_f16<QMOE_INT4>(rw, lg, nullptr, nullptr, bf[b][0], bf[b][1]);
        }
#pragma unroll
        for (int m = 0; m < MBV; ++m) {
          const h8_t a0 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a0 + 128 * m)));
          const h8_t a1 = __builtin_bit_cast(h8_t, *(const u4_t*)(As + 8 * (slot_a1 + 128 * m)));
#pragma unroll
          for (int b = 0; b < RNB; ++b) {
            acc[m][b] = mfma(a0, __builtin_bit_cast(h8_t, bf[b][0]), acc[m][b]);
            acc[m][b] = mfma(a1, __builtin_bit_cast(h8_t, bf[b][1]), acc[m][b]);
          }
        }
      } else {
        // exact codes (128+q) as bf16; the per-group scale goes on the fp32
        // partial sums of the tile, the row sums feed the bias term at the end
        const b8_t ones = __builtin_bit_cast(b8_t, u4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
        const uint32_t magic = 0x43004300u;
        const int gi = kt >> gsh;
        const bool first_of_group = (kt & ((1 << gsh) - 1)) == 0 || (PART && kt == kb);
        u4_t c0[RNB], c1[RNB];
        float sc[RNB];
#pragma unroll
        for (int b = 0; b < RNB; ++b) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            c0[b][i] = and_or_b32(q[b][0] >> (4 * i), 0x000F000Fu, magic);
            c1[b][i] = and_or_b32(q[b][1] >> (4 * i), 0x000F000Fu, magic);
          }
          sc[b] = f16_to_f32(sbv[b]);
        }
#pragma unroll
        for (int m = 0; m < MBV; ++m) {
          const b8_t a0 = __builtin_bit_cast(b8_t, *(const u4_t*)(As + 8 * (slot_a0 + 128 * m)));
          const b8_t a1 = __builtin_bit_cast(b8_t, *(const u4_t*)(As + 8 * (slot_a1 + 128 * m)));
#pragma unroll
          for (int b = 0; b < RNB; ++b) {
            f4_t t = mfma(a0, __builtin_bit_cast(b8_t, c0[b]), f4_t{0, 0, 0, 0});
            t = mfma(a1, __builtin_bit_cast(b8_t, c1[b]), t);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) acc[m][b][rr] = __builtin_fmaf(sc[b], t[rr], acc[m][b][rr]);
          }
        }
        // row sums of the tile's activations (bias term): wave w < MBV takes block w
        if (wave < MBV) {
          const b8_t a0 = __builtin_bit_cast(b8_t, *(const u4_t*)(As + 8 * (slot_a0 + 128 * wave)));
          const b8_t a1 = __builtin_bit_cast(b8_t, *(const u4_t*)(As + 8 * (slot_a1 + 128 * wave)));
          f4_t xs = mfma(a0, ones, f4_t{0, 0, 0, 0});
          xs = mfma(a1, ones, xs);
          if (lr == 0) {  // lane (lg, 0) holds the sums of rows 16w + 4lg .. +3
            f4_t* dst = (f4_t*)&xg[gi * BM + 16 * wave + 4 * lg];
            *dst = first_of_group ? xs : *dst + xs;
          }
        }
      }
    };

    // ---- the K loop: tiles kt+1 and kt+2 stream while kt is computed.  The
    // last two tiles are peeled off so the steady-state loop has no tests;
    // `sc` is the ring stage of tile kt.
    auto wait_next = [&](int kt) {  // only tile kt + 1's loads may be outstanding
      if constexpr (Q6K) {
        if (kt & 1) {  // tile kt + 1 starts a pair: one more load (its top bits)
          if (n_aload == 2) wait_vmcnt<4 + NMETA>();
          else wait_vmcnt<3 + NMETA>();
          return;
        }
      }
      if (n_aload == 2) wait_vmcnt<3 + NMETA>();
      else wait_vmcnt<2 + NMETA>();
    };
    if constexpr (BF && PART) {  // a K part sums only its own groups: the others stay zero
      for (int i = tid; i < XG4 * BM; i += RW * 64) xg[i] = 0.f;
    }
    const int nk = ke - kb;
    if constexpr (NST == 2) {  // one tile in flight: wait for it, then refill the other stage
      if (nk > 0) issue(kb, 0, true);
      int sc = 0;
      for (int kt = kb; kt + 1 < ke; ++kt) {
        wait_vmcnt<0>();
        ring_barrier();
        issue(kt + 1, sc ^ 1, false);
        compute(kt, sc);
        sc ^= 1;
      }
      if (nk > 0) {
        wait_vmcnt<0>();
        ring_barrier();
        compute(ke - 1, sc);
      }
    } else {
    if (nk > 0) issue(kb, 0, true);
    if (nk > 1) issue(kb + 1, 1, false);
    int sc = 0;
    for (int kt = kb; kt + 2 < ke; ++kt) {
      wait_next(kt);
      ring_barrier();
      issue(kt + 2, sc == 0 ? 2 : sc - 1, false);
      compute(kt, sc);
      sc = sc == 2 ? 0 : sc + 1;
    }
    if (nk > 1) {
      wait_next(ke - 2);
      ring_barrier();
      compute(ke - 2, sc);
      sc = sc == 2 ? 0 : sc + 1;
    }
    if (nk > 0) {
      wait_vmcnt<0>();
      ring_barrier();
      compute(ke - 1, sc);
    }
    }

    // ---- bf16 bias term: sum_g (b - 128 s)[n, g] * X[m, g] by MFMA with hi/lo
    // bf16 splits of both factors (G <= 32: one 32-group step; lane group lg
    // holds groups 8lg .. 8lg+7).  The activation sums are split once per
    // workgroup into the idle ring ([row][hi: 32 groups][lo: 32 groups] bf16,
    // rows padded to 144 bytes so the 16-byte operand reads do not share
    // banks); each wave splits only its own rows' coefficients.
    if constexpr (BF) {
      uint32_t sv[RNB][8];
#pragma unroll
      for (int b = 0; b < RNB; ++b) {
        const uint32_t* sbrow = (const uint32_t*)g.scales + rbk[b] * G * 16 + lr;
#pragma unroll
        for (int i = 0; i < 8; ++i) sv[b][i] = sbrow[min(8 * lg + i, G - 1) * 16];
      }
      constexpr int XROW = 72;  // bf16 per staged row (64 + 8 of padding)
      uint16_t* xsp = (uint16_t*)ring;
      ring_barrier();  // every wave's row sums are in xg and the ring is idle
      for (int i = tid; i < 16 * MBV * 4; i += RW * 64) {  // (row, 8-group chunk)
        const int r = i >> 2, c = i & 3;
        u4_t hh, ll;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int g0 = 8 * c + 2 * j;
          const f2_t v = {g0 < G ? xg[g0 * BM + r] : 0.f, g0 + 1 < G ? xg[(g0 + 1) * BM + r] : 0.f};
          const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2_t));
          const f2_t hv = {__builtin_bit_cast(float, h << 16), __builtin_bit_cast(float, h & 0xFFFF0000u)};
          hh[j] = h;
          ll[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v - hv, b2_t));
        }
        *(u4_t*)(xsp + r * XROW + 8 * c) = hh;
        *(u4_t*)(xsp + r * XROW + 32 + 8 * c) = ll;
      }
      ring_barrier();
#pragma unroll
      for (int b = 0; b < RNB; ++b) {
        u4_t bh, bl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f2_t cb;
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            const uint32_t w = sv[b][2 * i + qq];
            cb[qq] = (8 * lg + 2 * i + qq < G) ? f16_to_f32(w >> 16) - 128.0f * f16_to_f32(w & 0xFFFFu) : 0.f;
          }
          const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(cb, b2_t));
          const f2_t hv = {__builtin_bit_cast(float, h << 16), __builtin_bit_cast(float, h & 0xFFFF0000u)};
          bh[i] = h;
          bl[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(cb - hv, b2_t));
        }
#pragma unroll
        for (int m = 0; m < MBV; ++m) {
          const uint16_t* xr = xsp + (16 * m + lr) * XROW + 8 * lg;
          const b8_t XH = __builtin_bit_cast(b8_t, *(const u4_t*)xr);
          const b8_t XL = __builtin_bit_cast(b8_t, *(const u4_t*)(xr + 32));
          acc[m][b] = mfma(XH, __builtin_bit_cast(b8_t, bh), acc[m][b]);
          acc[m][b] = mfma(XH, __builtin_bit_cast(b8_t, bl), acc[m][b]);
          acc[m][b] = mfma(XL, __builtin_bit_cast(b8_t, bh), acc[m][b]);
        }
      }
    }

    // ---- a unit split into K parts: every part parks its fp32 sums in its
    // slot and takes a ticket; the last to arrive adds the parts in part
    // order (so the result does not depend on which finished first) and
    // writes the unit.  Nobody waits.  The sums and the ticket travel as
    // device-scope relaxed atomics (coherent across the XCDs' L2s without
    // flushing or invalidating them); a part's stores are complete
    // (vmcnt(0)) before its ticket is taken.
    if (PART) {
      // 16-byte buffer accesses with the sc1 cache policy (device-scope
      // coherent), offsets in bytes within the unit's SK_PARTS slots
      const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)sgpr_ptr(g.sk_part + (int64_t)(wk.pslot - wk.part) * SK_PART_FLOATS), (short)0,
          (int)(SK_PARTS * SK_PART_FLOATS * sizeof(float)), 0x00020000);
      constexpr int SC1 = 16;
      int* tk = g.sk_tickets + wk.tslot;
#pragma unroll
      for (int m = 0; m < MBV; ++m)
#pragma unroll
        for (int b = 0; b < RNB; ++b)
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(u4_t, acc[m][b]), prs,
              (uint32_t)((wk.part * SK_PART_FLOATS + 4 * ((m * RNB + b) * (RW * 64) + tid)) * 4), 0, SC1);
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      __syncthreads();
      if (tid == 0) sk_arrival = __hip_atomic_fetch_add(tk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (sk_arrival != SK_PARTS - 1) return;
      if (tid == 0) __hip_atomic_store(tk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int m = 0; m < MBV; ++m)
#pragma unroll
        for (int b = 0; b < RNB; ++b) {
          acc[m][b] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int pp = 0; pp < SK_PARTS; ++pp)
            acc[m][b] += __builtin_bit_cast(f4_t, __builtin_amdgcn_raw_buffer_load_b128(
                prs, (uint32_t)((pp * SK_PART_FLOATS + 4 * ((m * RNB + b) * (RW * 64) + tid)) * 4), 0, SC1));
        }
    }

    // ---- epilogue
    if constexpr (EPI == QMOE_EPI_STORE || EPI == QMOE_EPI_SWIGLU) {
      // 2-byte outputs: the tile's values go to the (now idle) ring as rows
      // of the workgroup's W output columns, then every thread writes
      // 16-byte pieces, so each output row is written whole and contiguous
      // instead of 32 bytes per row per store instruction.
      if (g.stage_out) {
        constexpr int W = swiglu ? BN / 2 : BN;  // output columns per workgroup
        constexpr int CPR = W / 8;               // 16-byte pieces per row
        constexpr int LROW = 2 * W + 16;         // LDS row stride in bytes
        static_assert(BM * LROW <= NST * STAGE, "output tile fits in the ring");
        ring_barrier();  // every wave is done with the ring
        // two values per packed conversion: SwiGLU rows rr and rr + 1, STORE
        // the wave's two column blocks of one row
        auto stage_rows = [&](auto half_c) {
          constexpr bool HALF = decltype(half_c)::value;
          constexpr int LR16 = LROW / 2;
#pragma unroll
          for (int m = 0; m < MBV; ++m) {
            uint16_t* dst = (uint16_t*)(ring + (16 * m + 4 * lg) * LROW);
            if constexpr (swiglu) {
#pragma unroll
              for (int rr = 0; rr < 4; rr += 2) {
                const uint32_t p = f32x2_to_16<HALF>(silu_f32(acc[m][0][rr]) * acc[m][1][rr],
                                                   silu_f32(acc[m][0][rr + 1]) * acc[m][1][rr + 1]);
                dst[rr * LR16 + 16 * wave + lr] = (uint16_t)p;
                dst[(rr + 1) * LR16 + 16 * wave + lr] = (uint16_t)(p >> 16);
              }
            } else {
              static_assert(RNB == 2, "two column blocks per wave");
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const uint32_t p = f32x2_to_16<HALF>(acc[m][0][rr], acc[m][1][rr]);
                dst[rr * LR16 + 32 * wave + lr] = (uint16_t)p;
                dst[rr * LR16 + 32 * wave + 16 + lr] = (uint16_t)(p >> 16);
              }
            }
          }
        };
        if (g.out_dtype == QMOE_F16) stage_rows(std::true_type{});
        else stage_rows(std::false_type{});
        ring_barrier();
        const int64_t nlim = swiglu ? Nh : g.N;
        for (int i = tid; i < nrows * CPR; i += RW * 64) {
          const int r = i / CPR, c = i - r * CPR;
          const int64_t col = (int64_t)nt * W + 8 * c;
          if (col < nlim)
            *(u4_t*)((uint16_t*)g.out + (int64_t)rows_o[r] * g.ldo + col) = *(const u4_t*)(ring + r * LROW + 16 * c);
        }
        return;
      }
    }
#pragma unroll
    for (int m = 0; m < MBV; ++m) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int row = 16 * m + 4 * lg + rr;
        if (row >= nrows) continue;
        const int64_t orow = rows_o[row];
        if constexpr (EPI == QMOE_EPI_SWIGLU) {
          if (nvalid[0]) store_out(g.out, g.out_dtype, orow * g.ldo + ncol[0], silu_f32(acc[m][0][rr]) * acc[m][1][rr]);
        } else if constexpr (EPI == QMOE_EPI_STORE) {
#pragma unroll
          for (int b = 0; b < RNB; ++b)
            if (nvalid[b]) store_out(g.out, g.out_dtype, orow * g.ldo + ncol[b], acc[m][b][rr]);
        } else if constexpr (EPI == QMOE_EPI_WEIGHTED_COMBINE) {
          const float w = wts[row];
          float* o = (float*)g.out + orow * g.ldo;
#pragma unroll
          for (int b = 0; b < RNB; ++b)
            if (nvalid[b]) atomicAdd(o + ncol[b], w * acc[m][b][rr]);
        } else {  // ACCUMULATE
          float* o = (float*)g.out + orow * g.ldo;
#pragma unroll
          for (int b = 0; b < RNB; ++b)
            if (nvalid[b]) o[ncol[b]] += acc[m][b][rr];
        }
      }
    }
  };
  auto dispatch2 = [&](auto part_c, auto fold_c) {
    switch (mbn) {
      case 1: run(std::integral_constant<int, 1>{}, part_c, fold_c); break;
      case 2: run(std::integral_constant<int, 2>{}, part_c, fold_c); break;
      case 3: run(std::integral_constant<int, 3>{}, part_c, fold_c); break;
      case 4: run(std::integral_constant<int, 4>{}, part_c, fold_c); break;
      default: run(std::integral_constant<int, 5>{}, part_c, fold_c); break;
    }
  };
  auto dispatch = [&](auto part_c) {
    if constexpr (MX) {
      if (fold) dispatch2(part_c, std::true_type{});
      else dispatch2(part_c, std::false_type{});
    } else {
      dispatch2(part_c, std::true_type{});
    }
  };
  if (wk.part >= 0) dispatch(std::true_type{});
  else dispatch(std::false_type{});
}

template <int ACT, int EPI>
__global__ __launch_bounds__(RW * 64) __attribute__((amdgpu_waves_per_eu(4)))
void qmm_int4_kernel(GemmArgs g) {
  ring_body<QMOE_INT4, ACT, EPI>(g);
}

template <int EPI>
__global__ __launch_bounds__(RW * 64) __attribute__((amdgpu_waves_per_eu(4)))
void qmm_iq2_ring_kernel(GemmArgs g) {
  ring_body<QMOE_IQ2_XXS, ACT_F16, EPI>(g);
}

template <int EPI>
__global__ __launch_bounds__(RW * 64) __attribute__((amdgpu_waves_per_eu(4)))
void qmm_q2k_ring_kernel(GemmArgs g) {
  ring_body<QMOE_Q2_K, ACT_F16, EPI>(g);
}

template <int EPI>
__global__ __launch_bounds__(RW * 64) __attribute__((amdgpu_waves_per_eu(4)))
void qmm_mxfp4_ring_kernel(GemmArgs g) {
  ring_body<QMOE_MXFP4, ACT_F16, EPI>(g);
}

template <int EPI>
__global__ __launch_bounds__(RW * 64) __attribute__((amdgpu_waves_per_eu(4)))
void qmm_q4k_ring_kernel(GemmArgs g) {
  ring_body<QMOE_Q4_K, ACT_F16, EPI>(g);
}

template <int EPI>
__global__ __launch_bounds__(RW * 64) __attribute__((amdgpu_waves_per_eu(4)))
void qmm_q6k_ring_kernel(GemmArgs g) {
  ring_body<QMOE_Q6_K, ACT_F16, EPI>(g);
}

template <int EPI>
__global__ __launch_bounds__(RW * 64) __attribute__((amdgpu_waves_per_eu(4)))
void qmm_fp8_ring_kernel(GemmArgs g) {
  ring_body<QMOE_FP8, ACT_F16, EPI>(g);
}

template <int EPI>
__global__ __launch_bounds__(RW * 64) __attribute__((amdgpu_waves_per_eu(4)))
void qmm_q8_ring_kernel(GemmArgs g) {
  ring_body<QMOE_Q8_0, ACT_F16, EPI>(g);
}

// Whether the LDS-ring kernel takes this call: int4 with either activation
// type (groups of at least 64 values; bf16 keeps at most XG4 groups per row
// for the bias term), every other format with fp16 activations.  N must be
// whole 16-row blocks (32 with SwiGLU), and the per-lane byte offsets within
// one expert's codes must fit 31 bits.
static bool ring_ok(const GemmArgs& g, int fmt, int act, int epi) {
  if (g.N % (epi == QMOE_EPI_SWIGLU ? 32 : 16)) return false;
  if (fmt != QMOE_INT4 && act != QMOE_F16) return false;
  int64_t row_bytes;  // code bytes per weight row
  switch (fmt) {
    case QMOE_INT4:
      if (g.group < 64 || (act == QMOE_BF16 && g.K / g.group > XG4)) return false;
      row_bytes = g.K / 2;
      break;
    case QMOE_IQ2_XXS: case QMOE_Q2_K: row_bytes = g.K / 4; break;
    case QMOE_MXFP4: case QMOE_Q4_K: case QMOE_Q6_K: row_bytes = g.K / 2; break;
    case QMOE_FP8: case QMOE_Q8_0: row_bytes = g.K; break;
    default: return false;
  }
  return g.N * row_bytes < (1ll << 31);
}

using KernelFn = void (*)(GemmArgs);

// The ring kernel of a format and epilogue.
template <int EPI>
static KernelFn ring_kernel(int fmt, int act) {
  switch (fmt) {
    case QMOE_IQ2_XXS: return qmm_iq2_ring_kernel<EPI>;
    case QMOE_Q2_K: return qmm_q2k_ring_kernel<EPI>;
    case QMOE_MXFP4: return qmm_mxfp4_ring_kernel<EPI>;
    case QMOE_Q4_K: return qmm_q4k_ring_kernel<EPI>;
    case QMOE_Q6_K: return qmm_q6k_ring_kernel<EPI>;
    case QMOE_FP8: return qmm_fp8_ring_kernel<EPI>;
    case QMOE_Q8_0: return qmm_q8_ring_kernel<EPI>;
    default: return act == QMOE_F16 ? qmm_int4_kernel<ACT_F16, EPI> : qmm_int4_kernel<ACT_BF16, EPI>;
  }
}

static void launch_ring(const GemmArgs& g, int fmt, int act, int epi, hipStream_t s) {
  KernelFn k;
  switch (epi) {
    case QMOE_EPI_STORE: k = ring_kernel<QMOE_EPI_STORE>(fmt, act); break;
    case QMOE_EPI_SWIGLU: k = ring_kernel<QMOE_EPI_SWIGLU>(fmt, act); break;
    case QMOE_EPI_WEIGHTED_COMBINE: k = ring_kernel<QMOE_EPI_WEIGHTED_COMBINE>(fmt, act); break;
    default: k = ring_kernel<QMOE_EPI_ACCUMULATE>(fmt, act); break;
  }
  hipLaunchKernelGGL(k, dim3(g.n_blocks), dim3(RW * 64), 0, s, g);
}

template <int FMT, int ACT>
static void launch_fa(const GemmArgs& g, int epi, hipStream_t s) {
  const dim3 grid(g.n_blocks), block(256);
  switch (epi) {
    case QMOE_EPI_STORE: hipLaunchKernelGGL((qmm_kernel<FMT, ACT, QMOE_EPI_STORE>), grid, block, 0, s, g); break;
    case QMOE_EPI_SWIGLU: hipLaunchKernelGGL((qmm_kernel<FMT, ACT, QMOE_EPI_SWIGLU>), grid, block, 0, s, g); break;
    case QMOE_EPI_WEIGHTED_COMBINE: hipLaunchKernelGGL((qmm_kernel<FMT, ACT, QMOE_EPI_WEIGHTED_COMBINE>), grid, block, 0, s, g); break;
    default: hipLaunchKernelGGL((qmm_kernel<FMT, ACT, QMOE_EPI_ACCUMULATE>), grid, block, 0, s, g); break;
  }
}

template <int FMT>
static void launch_f(const GemmArgs& g, int act, int epi, hipStream_t s) {
  if (act == QMOE_F16) launch_fa<FMT, ACT_F16>(g, epi, s);
  else launch_fa<FMT, ACT_BF16>(g, epi, s);
}

// Workgroups of the int4 ring kernel resident at once on the current device
// (two per CU), a multiple of the 8 XCDs and at most 512 (the plan's
// balancing slots); 0 when the device cannot be queried.
static int resident_ring_blocks() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  static std::atomic<int> cache[64];
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    v = min(64, 2 * cus / 8) * 8;
    if (v <= 0) v = -1;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v > 0 ? v : 0;
}

// Groups per row the bf16 int4 path can keep (bias term), and the tallest tile.
int qmm_int4_bf16_max_groups() { return XG_MAX; }
int qmm_max_rows() { return BM; }

// Host launcher shared by qmoe_qmm_dense and qmoe_moe_gather_qmm.
void launch_qmm(const qmoe_weights* w, const void* a, int act, int amode, const int32_t* plan,
                int64_t t, int topk, int bm, int64_t M, const float* topk_w, int epi, void* out,
                int out_dtype, hipStream_t s) {
  GemmArgs g;
  g.qs = w->qs; g.aux = w->aux; g.scales = w->scales; g.biases = w->biases;
  g.d = w->d; g.dmin = w->dmin; g.grid = w->grid; g.signs = w->signs;
  g.N = w->n; g.K = w->k; g.group = w->group;
  g.amode = amode;
  g.a = (const uint16_t*)a;
  g.a_bytes = (amode == AM_DENSE ? M : amode == AM_GATHER ? t : t * topk) * w->k * 2;
  g.plan = plan;
  g.E = w->n_experts;
  g.topk = topk;
  g.P = t * topk;
  g.t = t;
  g.M = M;
  g.topk_w = topk_w;
  g.out = out;
  g.out_dtype = out_dtype;
  int64_t n_mt;
  g.bm = bm;
  if (amode == AM_DENSE) n_mt = (M + BM - 1) / BM;
  else n_mt = plan_max_tiles(g.P, g.E, bm);
  if (epi == QMOE_EPI_SWIGLU) { g.n_ntiles = (int)((w->n / 2 + BN / 2 - 1) / (BN / 2)); g.ldo = w->n / 2; }
  else { g.n_ntiles = (int)((w->n + BN - 1) / BN); g.ldo = w->n; }
  g.n_blocks = (int)((n_mt + 7) / 8 * 8 * g.n_ntiles);  // whole rounds of the 8 XCDs
  g.stage_out = (out_dtype == QMOE_F16 || out_dtype == QMOE_BF16) && g.ldo % 8 == 0 && (uintptr_t)out % 16 == 0;
  g.sk_slots_xcd = 0;
  g.sk_tickets = nullptr;
  g.sk_part = nullptr;
  if (g.n_blocks == 0) return;
  if (ring_ok(g, w->fmt, act, epi)) {
    // Plans of SK_MIN_PAIRS pairs and more carry a balancing area: the units
    // of a short last round are split along K (work_of_block), which needs
    // up to 3 * sx / 4 more workgroups per XCD.
    const int npb = amode != AM_DENSE && g.P >= SK_MIN_PAIRS ? resident_ring_blocks() : 0;
    if (npb > 0) {
      int32_t* sk = const_cast<int32_t*>(plan) + plan_sk_offset(g.P, g.E);
      g.sk_slots_xcd = npb / 8;
      g.sk_tickets = sk;
      g.sk_part = (float*)(sk + SK_SLOTS);
      g.n_blocks += 8 * (3 * g.sk_slots_xcd / 4);
    }
    launch_ring(g, w->fmt, act, epi, s);
    return;
  }
  switch (w->fmt) {
    case QMOE_Q8_0: launch_f<QMOE_Q8_0>(g, act, epi, s); break;
    case QMOE_Q2_K: launch_f<QMOE_Q2_K>(g, act, epi, s); break;
    case QMOE_Q4_K: launch_f<QMOE_Q4_K>(g, act, epi, s); break;
    case QMOE_Q6_K: launch_f<QMOE_Q6_K>(g, act, epi, s); break;
    case QMOE_IQ2_XXS: launch_f<QMOE_IQ2_XXS>(g, act, epi, s); break;
    case QMOE_MXFP4: launch_f<QMOE_MXFP4>(g, act, epi, s); break;
    case QMOE_FP8: launch_f<QMOE_FP8>(g, act, epi, s); break;
    default: launch_f<QMOE_INT4>(g, act, epi, s); break;
  }
}

}  // namespace qmoe
