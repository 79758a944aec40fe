// Prefill matmul over quantised weights: the gathered MoE tile GEMM and the
// dense qmm share one kernel.
//
// What is computed: for each tile of (up to 128) rows routed to one expert
// and a 128-wide slice of that expert's output rows, y = A . W[e]^T with fp32
// accumulation, followed by an epilogue (store, SwiGLU, top-k weighted
// scatter-add, or accumulate).  The DSV4 campaign page's tiled MoE prefill
// GEMM (map0 work queue, 64-slot iq2_xxs gate/up tile, q2_K SoA down twin)
// and the metaltile shim page's mt_qmm_mma / mt_moe_gather_qmm kernels are the
// prior art; the tiling here is built for CDNA4 instead.
//
// Layout on gfx950:
//  * 256 threads = 4 waves.  A workgroup owns one (row tile, column tile).
//    Wave w owns 32 weight rows as two 16-column MFMA blocks (SwiGLU: 16 gate
//    rows and the 16 matching up rows, so silu(g)*u is lane-local).
//  * K advances in 64-wide tiles.  The activation tile (128 x 64) is gathered
//    by routed row straight into LDS, double buffered, one barrier per tile.
//  * B fragments are dequantised in registers from the weight bytes each lane
//    loads itself (one wide load per lane per tile) and fed to
//    v_mfma_f32_16x16x32_{f16,bf16}; each fragment is reused by every 16-row
//    block of the tile.
//  * Within a 64-wide K tile, lane group g (lanes 16g..16g+15) owns the 16
//    contiguous k-values [16g, 16g+16); MFMA step s consumes values
//    16g+8s..16g+8s+7 of every lane group (the A fragments are read from LDS
//    with the same permutation, so the contraction is unchanged).  Formats
//    whose scale changes every 32 values use the plain k order instead
//    (MFMA step s = values 32s..32s+31).
//  * fp16 activations: weights are dequantised to fp16 in registers (one or
//    two fp16 roundings per weight).  bf16 activations: the MFMA consumes the
//    integer codes, which are exact in bf16, and the per-group scale and bias
//    are applied to the fp32 partial sums, so no weight is ever rounded to
//    bf16's 8-bit significand.
#include "common.h"

namespace qmoe {

constexpr int BM = 128;       // rows per tile
constexpr int BK = 64;        // k per LDS tile
constexpr int LDA = BK + 8;   // LDS row stride in halves (144 B, conflict-free b128 reads)
constexpr int MB = BM / 16;   // 16-row MFMA blocks per tile

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
  const int32_t* plan;
  int E, topk, bm;
  int64_t P;
  int64_t M;  // dense rows
  const float* topk_w;
  void* out;
  int out_dtype;
  int64_t ldo;
  int n_ntiles;
  int n_blocks;
};

// Which k order a (format, activation) path uses inside a 64-wide tile.
template <int FMT, int ACT>
struct KOrder {
  // true: lane group g owns k in [16g, 16g+16); false: MFMA step s covers [32s, 32s+32)
  static constexpr bool chunk = !(ACT == ACT_BF16 && (FMT == QMOE_Q8_0 || FMT == QMOE_IQ2_XXS));
};

// Raw weight bytes one lane needs for one 64-wide K tile of one output row.
struct Raw {
  u4_t v;        // codes
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
    const int64_t kk = k0 + 16 * lg;
    const u2_t q = *(const u2_t*)((const uint32_t*)g.qs + R * (K / 8) + kk / 8);
    r.v = u4_t{q[0], q[1], 0u, 0u};
    const int64_t gi = R * (K / g.group) + kk / g.group;
    r.x0 = ((const uint16_t*)g.scales)[gi];
    r.x1 = ((const uint16_t*)g.biases)[gi];
  } else if constexpr (FMT == QMOE_Q8_0) {
    if constexpr (KOrder<FMT, ACT>::chunk) {
      const int64_t kk = k0 + 16 * lg;
      r.v = *(const u4_t*)((const int8_t*)g.qs + R * K + kk);
      r.x0 = ((const uint16_t*)g.scales)[R * (K / 32) + kk / 32];
    } else {
      const int8_t* base = (const int8_t*)g.qs + R * K + k0 + 8 * lg;
      const u2_t q0 = *(const u2_t*)base;
      const u2_t q1 = *(const u2_t*)(base + 32);
      r.v = u4_t{q0[0], q0[1], q1[0], q1[1]};
      r.x0 = ((const uint16_t*)g.scales)[R * (K / 32) + k0 / 32];
      r.x2 = ((const uint16_t*)g.scales)[R * (K / 32) + k0 / 32 + 1];
    }
  } else if constexpr (FMT == QMOE_Q2_K) {
    const int64_t B = R * (K / 256) + k0 / 256;
    const int e0 = (int)(k0 & 255) + 16 * lg;
    const int byte = 32 * (e0 >> 7) + (e0 & 31);
    r.v = *(const u4_t*)((const uint32_t*)g.qs + B * 16 + byte / 4);
    r.x0 = ((const uint8_t*)g.scales)[B * 16 + (e0 >> 4)];
    r.x2 = ((const uint16_t*)g.d)[B];
    r.x3 = ((const uint16_t*)g.dmin)[B];
  } else {  // IQ2_XXS
    const int64_t B = R * (K / 256) + k0 / 256;
    if constexpr (KOrder<FMT, ACT>::chunk) {
      const int G = ((int)(k0 & 255) + 16 * lg) >> 5;
      r.x0 = ((const uint32_t*)g.qs)[B * 8 + G];
      r.x1 = ((const uint32_t*)g.aux)[B * 8 + G];
    } else {
      const int G = (int)(k0 & 255) >> 5;
      r.x0 = ((const uint32_t*)g.qs)[B * 8 + G];
      r.x1 = ((const uint32_t*)g.aux)[B * 8 + G];
      r.x2 = ((const uint32_t*)g.qs)[B * 8 + G + 1];
      r.x3 = ((const uint32_t*)g.aux)[B * 8 + G + 1];
    }
    r.x4 = ((const uint16_t*)g.d)[B];
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
                                         const uint32_t* lut_sign, h8_t& f0, h8_t& f1) {
  u4_t o0, o1;
  if constexpr (FMT == QMOE_INT4) {
    const h2_t s2 = h2_t{__builtin_bit_cast(_Float16, (uint16_t)r.x0), __builtin_bit_cast(_Float16, (uint16_t)r.x0)};
    const h2_t b2 = h2_t{__builtin_bit_cast(_Float16, (uint16_t)r.x1), __builtin_bit_cast(_Float16, (uint16_t)r.x1)};
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
    // r.v: 16 code bytes; element shift from the lane's position (baked by caller in x1)
    const uint32_t sc = r.x0;
    const float d = f16_to_f32(r.x2), dm = f16_to_f32(r.x3);
    const _Float16 dl = (_Float16)(d * (float)(sc & 15u));
    const _Float16 ml = (_Float16)(-(dm * (float)(sc >> 4)));
    const h2_t dl2 = h2_t{dl, dl}, ml2 = h2_t{ml, ml};
    const h2_t off = h2_t{(_Float16)1024.0f, (_Float16)1024.0f};
    const uint32_t shift = r.x1;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t t = (r.v[w] >> shift) & 0x03030303u;
      const h2_t lo = __builtin_bit_cast(h2_t, perm_b32(0x64646464u, t, SEL_B01)) - off;
      const h2_t hi = __builtin_bit_cast(h2_t, perm_b32(0x64646464u, t, SEL_B23)) - off;
      const uint32_t vl = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(lo, dl2, ml2));
      const uint32_t vh = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(hi, dl2, ml2));
      if (w < 2) { o0[2 * w] = vl; o0[2 * w + 1] = vh; }
      else { o1[2 * (w - 2)] = vl; o1[2 * (w - 2) + 1] = vh; }
    }
  } else {  // IQ2_XXS: octets j0, j0+1 of the group, j0 = 2 * (lg & 1)
    const uint32_t idx = r.x0, aux = r.x1;
    const float db = f16_to_f32(r.x4) * (0.5f + (float)(aux >> 28)) * 0.25f;
    const _Float16 dbh = (_Float16)db;
    const h2_t db2 = h2_t{dbh, dbh};
    const int j0 = 2 * (lg & 1);
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const int j = j0 + o;
      const uint32_t gi = (idx >> (8 * j)) & 0xFFu;
      const uint32_t si = (aux >> (7 * j)) & 0x7Fu;
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
  f0 = __builtin_bit_cast(h8_t, o0);
  f1 = __builtin_bit_cast(h8_t, o1);
}

// ------------------------------------------------------------------ kernel

template <int FMT, int ACT, int EPI>
__global__ __launch_bounds__(256, 2) void qmm_kernel(GemmArgs g) {
  typedef typename ActT<ACT>::v8 v8_t;
  constexpr bool CHUNK = KOrder<FMT, ACT>::chunk;
  constexpr bool NEED_X = (ACT == ACT_BF16 && FMT == QMOE_INT4);
  constexpr bool IQ2 = (FMT == QMOE_IQ2_XXS);

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDA];
  __shared__ int rows_a[BM];
  __shared__ int rows_o[BM];
  __shared__ float wts[BM];
  __shared__ __attribute__((aligned(16))) float xs[2][BM];
  __shared__ __attribute__((aligned(16))) uint32_t lut_grid[IQ2 ? 256 * 4 : 4];
  __shared__ __attribute__((aligned(16))) uint32_t lut_sign[IQ2 ? 128 * 4 : 4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lr = lane & 15;

  const int v = xcd_remap(blockIdx.x, g.n_blocks);
  const int mt = v / g.n_ntiles, nt = v - mt * g.n_ntiles;

  int expert, row0, nrows;
  if (g.amode == AM_DENSE) {
    expert = 0;
    row0 = mt * BM;
    if (row0 >= g.M) return;
    nrows = (int)min<int64_t>(BM, g.M - row0);
  } else {
    if (mt >= g.plan[1]) return;
    const PlanLayout L = plan_layout(g.P, g.E);
    const int32_t* tl = g.plan + L.tiles + 4 * (int64_t)mt;
    expert = tl[0];
    row0 = tl[1];
    nrows = tl[2];
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
  if (g.amode == AM_DENSE && tid < BM) {
    rows_a[tid] = tid < nrows ? row0 + tid : -1;
    rows_o[tid] = row0 + tid;
    wts[tid] = 0.f;
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

  const int mbn = (nrows + 15) >> 4;  // valid 16-row blocks

  // Weight rows of this lane for its two column blocks.
  const bool swiglu = (EPI == QMOE_EPI_SWIGLU);
  const int64_t Nh = g.N / 2;
  int64_t ncol[2];     // output column (or h column) index of this lane per block
  int64_t wrow[2];     // weight row (within the expert)
  bool nvalid[2];
  if (swiglu) {
    const int64_t j = (int64_t)nt * 64 + 16 * wave + lr;
    ncol[0] = ncol[1] = j;
    nvalid[0] = nvalid[1] = j < Nh;
    const int64_t jc = j < Nh ? j : Nh - 1;
    wrow[0] = jc;
    wrow[1] = Nh + jc;
  } else {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t n = (int64_t)nt * 128 + 32 * wave + 16 * b + lr;
      ncol[b] = n;
      nvalid[b] = n < g.N;
      wrow[b] = n < g.N ? n : g.N - 1;
    }
  }
  const int64_t Rb0 = (int64_t)expert * g.N + wrow[0];
  const int64_t Rb1 = (int64_t)expert * g.N + wrow[1];

  f4_t acc[MB][2];
#pragma unroll
  for (int m = 0; m < MB; ++m) { acc[m][0] = f4_t{0, 0, 0, 0}; acc[m][1] = f4_t{0, 0, 0, 0}; }

  const int KT = (int)(g.K / BK);
  const uint16_t* __restrict__ A = g.a;

  // ---- activation staging (4 x 16 B per thread per tile)
  u4_t astage[4];
  auto load_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 3, part = c & 7;
      const int src = rows_a[r];
      if (src >= 0) astage[i] = *(const u4_t*)(A + (int64_t)src * g.K + (int64_t)kt * BK + 8 * part);
      else astage[i] = u4_t{0u, 0u, 0u, 0u};
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 3, part = c & 7;
      *(u4_t*)(&As[buf][r * LDA + 8 * part]) = astage[i];
      if constexpr (NEED_X) {
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          s += bf16_to_f32(astage[i][q] & 0xFFFFu);
          s += bf16_to_f32(astage[i][q] >> 16);
        }
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        if (part == 0) xs[buf][r] = s;
      }
    }
  };

  Raw rc0, rc1, rn0, rn1;
  load_a(0);
  rc0 = load_raw<FMT, ACT>(g, Rb0, 0, lg);
  rc1 = load_raw<FMT, ACT>(g, Rb1, 0, lg);
  store_a(0);

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    __syncthreads();
    const bool more = kt + 1 < KT;
    if (more) {
      load_a(kt + 1);
      rn0 = load_raw<FMT, ACT>(g, Rb0, (int64_t)(kt + 1) * BK, lg);
      rn1 = load_raw<FMT, ACT>(g, Rb1, (int64_t)(kt + 1) * BK, lg);
    }
    const uint16_t* Ab = &As[buf][0];

    if constexpr (ACT == ACT_F16) {
      if constexpr (FMT == QMOE_Q2_K) {
        const int e0 = (kt * BK & 255) + 16 * lg;
        rc0.x1 = rc1.x1 = 2u * (uint32_t)((e0 & 127) >> 5);
      }
      h8_t b00, b01, b10, b11;
      frag_f16<FMT>(rc0, lg, lut_grid, lut_sign, b00, b01);
      frag_f16<FMT>(rc1, lg, lut_grid, lut_sign, b10, b11);
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if (m < mbn) {
          const uint16_t* ar = Ab + (16 * m + lr) * LDA + 16 * lg;
          const h8_t a0 = __builtin_bit_cast(h8_t, *(const u4_t*)ar);
          const h8_t a1 = __builtin_bit_cast(h8_t, *(const u4_t*)(ar + 8));
          acc[m][0] = mfma(a0, b00, acc[m][0]);
          acc[m][1] = mfma(a0, b10, acc[m][1]);
          acc[m][0] = mfma(a1, b01, acc[m][0]);
          acc[m][1] = mfma(a1, b11, acc[m][1]);
        }
      }
    } else {
      // ---------------- bf16 activations: integer codes into the MFMA,
      // scales on the fp32 partial sums.
      if constexpr (FMT == QMOE_INT4) {
        u4_t c0a, c0b, c1a, c1b;  // codes (128+q) as bf16 pairs, steps 0/1, blocks 0/1
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c0a[i] = ((rc0.v[0] >> (4 * i)) & 0x000F000Fu) | 0x43004300u;
          c0b[i] = ((rc0.v[1] >> (4 * i)) & 0x000F000Fu) | 0x43004300u;
          c1a[i] = ((rc1.v[0] >> (4 * i)) & 0x000F000Fu) | 0x43004300u;
          c1b[i] = ((rc1.v[1] >> (4 * i)) & 0x000F000Fu) | 0x43004300u;
        }
        const float s0 = f16_to_f32(rc0.x0), s1 = f16_to_f32(rc1.x0);
        const float cb0 = f16_to_f32(rc0.x1) - 128.0f * s0;
        const float cb1 = f16_to_f32(rc1.x1) - 128.0f * s1;
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          if (m < mbn) {
            const uint16_t* ar = Ab + (16 * m + lr) * LDA + 16 * lg;
            const b8_t a0 = __builtin_bit_cast(b8_t, *(const u4_t*)ar);
            const b8_t a1 = __builtin_bit_cast(b8_t, *(const u4_t*)(ar + 8));
            f4_t t0 = f4_t{0, 0, 0, 0}, t1 = f4_t{0, 0, 0, 0};
            t0 = mfma(a0, __builtin_bit_cast(b8_t, c0a), t0);
            t1 = mfma(a0, __builtin_bit_cast(b8_t, c1a), t1);
            t0 = mfma(a1, __builtin_bit_cast(b8_t, c0b), t0);
            t1 = mfma(a1, __builtin_bit_cast(b8_t, c1b), t1);
            const f4_t X = *(const f4_t*)(&xs[buf][16 * m + 4 * lg]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              acc[m][0][r] = __builtin_fmaf(s0, t0[r], __builtin_fmaf(cb0, X[r], acc[m][0][r]));
              acc[m][1][r] = __builtin_fmaf(s1, t1[r], __builtin_fmaf(cb1, X[r], acc[m][1][r]));
            }
          }
        }
      } else if constexpr (FMT == QMOE_Q8_0) {
        // plain k order: step s = one 32-value block; codes converted exactly
        u4_t c[2][2];  // [block][step]
        float dsc[2][2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const Raw& r = b ? rc1 : rc0;
          dsc[b][0] = f16_to_f32(r.x0);
          dsc[b][1] = f16_to_f32(r.x2);
#pragma unroll
          for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t w = r.v[2 * s + (i >> 1)];
              const int sh = 16 * (i & 1);
              const float lo = (float)(int8_t)((w >> sh) & 0xFFu);
              const float hi = (float)(int8_t)((w >> (sh + 8)) & 0xFFu);
              c[b][s][i] = (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
            }
          }
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          if (m < mbn) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const uint16_t* ar = Ab + (16 * m + lr) * LDA + 32 * s + 8 * lg;
              const b8_t a = __builtin_bit_cast(b8_t, *(const u4_t*)ar);
              const f4_t t0 = mfma(a, __builtin_bit_cast(b8_t, c[0][s]), f4_t{0, 0, 0, 0});
              const f4_t t1 = mfma(a, __builtin_bit_cast(b8_t, c[1][s]), f4_t{0, 0, 0, 0});
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                acc[m][0][r] = __builtin_fmaf(dsc[0][s], t0[r], acc[m][0][r]);
                acc[m][1][r] = __builtin_fmaf(dsc[1][s], t1[r], acc[m][1][r]);
              }
            }
          }
        }
      } else if constexpr (FMT == QMOE_IQ2_XXS) {
        // plain k order: step s = one 32-value group, octet lg of it
        u4_t c[2][2];
        float dsc[2][2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const Raw& r = b ? rc1 : rc0;
          const float d = f16_to_f32(r.x4);
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const uint32_t idx = s ? r.x2 : r.x0;
            const uint32_t aux = s ? r.x3 : r.x1;
            dsc[b][s] = d * (0.5f + (float)(aux >> 28)) * 0.25f;
            const uint32_t gi = (idx >> (8 * lg)) & 0xFFu;
            const uint32_t si = (aux >> (7 * lg)) & 0x7Fu;
            const u4_t row = *(const u4_t*)(lut_grid + 4 * gi);
            const u4_t msk = *(const u4_t*)(lut_sign + 4 * si);
            c[b][s] = row ^ msk;
          }
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          if (m < mbn) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const uint16_t* ar = Ab + (16 * m + lr) * LDA + 32 * s + 8 * lg;
              const b8_t a = __builtin_bit_cast(b8_t, *(const u4_t*)ar);
              const f4_t t0 = mfma(a, __builtin_bit_cast(b8_t, c[0][s]), f4_t{0, 0, 0, 0});
              const f4_t t1 = mfma(a, __builtin_bit_cast(b8_t, c[1][s]), f4_t{0, 0, 0, 0});
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                acc[m][0][r] = __builtin_fmaf(dsc[0][s], t0[r], acc[m][0][r]);
                acc[m][1][r] = __builtin_fmaf(dsc[1][s], t1[r], acc[m][1][r]);
              }
            }
          }
        }
      } else {  // Q2_K, chunk order: lane chunk = one 16-value sub-block
        const int e0 = (kt * BK & 255) + 16 * lg;
        const uint32_t shift = 2u * (uint32_t)((e0 & 127) >> 5);
        u4_t cq[2][2], cm[2];
        float dd[2], dm[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const Raw& r = b ? rc1 : rc0;
          const float a = (float)(r.x0 & 15u);
          const float mn = (float)(r.x0 >> 4);
          dd[b] = f16_to_f32(r.x2);
          dm[b] = f16_to_f32(r.x3);
          const uint32_t mb16 = __builtin_bit_cast(uint32_t, mn) >> 16;
          cm[b] = u4_t{mb16 | (mb16 << 16), mb16 | (mb16 << 16), mb16 | (mb16 << 16), mb16 | (mb16 << 16)};
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t t = (r.v[w] >> shift) & 0x03030303u;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const float lo = a * (float)((t >> (16 * h)) & 0xFFu);
              const float hi = a * (float)((t >> (16 * h + 8)) & 0xFFu);
              cq[b][w >> 1][2 * (w & 1) + h] = (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
            }
          }
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          if (m < mbn) {
            const uint16_t* ar = Ab + (16 * m + lr) * LDA + 16 * lg;
            const b8_t a0 = __builtin_bit_cast(b8_t, *(const u4_t*)ar);
            const b8_t a1 = __builtin_bit_cast(b8_t, *(const u4_t*)(ar + 8));
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              f4_t tq = f4_t{0, 0, 0, 0}, tm = f4_t{0, 0, 0, 0};
              tq = mfma(a0, __builtin_bit_cast(b8_t, cq[b][0]), tq);
              tq = mfma(a1, __builtin_bit_cast(b8_t, cq[b][1]), tq);
              tm = mfma(a0, __builtin_bit_cast(b8_t, cm[b]), tm);
              tm = mfma(a1, __builtin_bit_cast(b8_t, cm[b]), tm);
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc[m][b][r] = __builtin_fmaf(dd[b], tq[r], __builtin_fmaf(-dm[b], tm[r], acc[m][b][r]));
            }
          }
        }
      }
    }

    if (more) {
      store_a(buf ^ 1);
      rc0 = rn0;
      rc1 = rn1;
    }
  }

  // ---------------------------------------------------------------- epilogue
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (m >= mbn) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * m + 4 * lg + r;
      if (row >= nrows) continue;
      const int64_t orow = rows_o[row];
      if constexpr (EPI == QMOE_EPI_SWIGLU) {
        if (nvalid[0]) store_out(g.out, g.out_dtype, orow * g.ldo + ncol[0], silu_f32(acc[m][0][r]) * acc[m][1][r]);
      } else if constexpr (EPI == QMOE_EPI_STORE) {
        if (nvalid[0]) store_out(g.out, g.out_dtype, orow * g.ldo + ncol[0], acc[m][0][r]);
        if (nvalid[1]) store_out(g.out, g.out_dtype, orow * g.ldo + ncol[1], acc[m][1][r]);
      } else if constexpr (EPI == QMOE_EPI_WEIGHTED_COMBINE) {
        const float w = wts[row];
        float* o = (float*)g.out + orow * g.ldo;
        if (nvalid[0]) atomicAdd(o + ncol[0], w * acc[m][0][r]);
        if (nvalid[1]) atomicAdd(o + ncol[1], w * acc[m][1][r]);
      } else {  // ACCUMULATE
        float* o = (float*)g.out + orow * g.ldo;
        if (nvalid[0]) o[ncol[0]] += acc[m][0][r];
        if (nvalid[1]) o[ncol[1]] += acc[m][1][r];
      }
    }
  }
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
  g.plan = plan;
  g.E = w->n_experts;
  g.topk = topk;
  g.P = t * topk;
  g.M = M;
  g.topk_w = topk_w;
  g.out = out;
  g.out_dtype = out_dtype;
  int64_t n_mt;
  g.bm = bm;
  if (amode == AM_DENSE) n_mt = (M + BM - 1) / BM;
  else n_mt = plan_max_tiles(g.P, g.E, bm);
  if (epi == QMOE_EPI_SWIGLU) { g.n_ntiles = (int)((w->n / 2 + 63) / 64); g.ldo = w->n / 2; }
  else { g.n_ntiles = (int)((w->n + 127) / 128); g.ldo = w->n; }
  g.n_blocks = (int)(n_mt * g.n_ntiles);
  if (g.n_blocks == 0) return;
  switch (w->fmt) {
    case QMOE_Q8_0: launch_f<QMOE_Q8_0>(g, act, epi, s); break;
    case QMOE_Q2_K: launch_f<QMOE_Q2_K>(g, act, epi, s); break;
    case QMOE_IQ2_XXS: launch_f<QMOE_IQ2_XXS>(g, act, epi, s); break;
    default: launch_f<QMOE_INT4>(g, act, epi, s); break;
  }
}

}  // namespace qmoe
