// Standalone dequantisation kernels (bit-exact).
//
// Formats as the GGUF block-dequant page defines them ("Kernels" 1-3 and the
// IQ2_XXS sign-fix commit) plus the MLX-style int4 affine slabs of the
// "Everything Bagel 2" expert-indexed GEMV.  Each value is formed in fp32 as
// the format defines it -- every product there is exact in fp32, so at most
// one rounding (the Q2_K subtraction, the int4 bias add) happens -- and is then
// rounded once, to nearest even, to the output dtype.  One thread decodes one
// 8-value unit and writes it with a single 16-byte (32-byte for fp32) store.
#include "common.h"

namespace qmoe {

template <int OUT>
__device__ __forceinline__ void store8(void* out, int64_t u, const float (&v)[8]) {
  if constexpr (OUT == QMOE_F32) {
    f4_t* o = (f4_t*)out + 2 * u;
    o[0] = f4_t{v[0], v[1], v[2], v[3]};
    o[1] = f4_t{v[4], v[5], v[6], v[7]};
  } else {
    u4_t w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo, hi;
      if constexpr (OUT == QMOE_F16) { lo = f32_to_f16(v[2 * i]); hi = f32_to_f16(v[2 * i + 1]); }
      else { lo = f32_to_bf16(v[2 * i]); hi = f32_to_bf16(v[2 * i + 1]); }
      w[i] = lo | (hi << 16);
    }
    ((u4_t*)out)[u] = w;
  }
}

// Q8_0: value = code * d over 32-value blocks.  Tiled layout (qmoe.h): unit
// u is values 8(u % (k/8)) .. +7 of row R = u / (k/8).
template <int OUT>
__global__ __launch_bounds__(256) void dequant_q8_0_kernel(const int8_t* __restrict__ qs,
                                                           const uint16_t* __restrict__ d,
                                                           int64_t n_units, int64_t k, void* __restrict__ out) {
  const int64_t upr = k / 8, KT = k / 64;
  for (int64_t u = blockIdx.x * 256ll + threadIdx.x; u < n_units; u += (int64_t)gridDim.x * 256) {
    const int64_t R = u / upr, kk = 8 * (u - R * upr);
    const int64_t rb = R >> 4, r = R & 15, kt = kk >> 6, c = (kk & 63) >> 4;
    const u2_t q = *(const u2_t*)(qs + (((rb * KT + kt) * 4 + c) * 16 + r) * 16 + (kk & 15));
    const float s = f16_to_f32(d[(rb * (k / 32) + (kk >> 5)) * 16 + r]);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int8_t cd = (int8_t)((q[i >> 2] >> (8 * (i & 3))) & 0xFF);
      v[i] = (float)cd * s;
    }
    store8<OUT>(out, u, v);
  }
}

// Q4_K (tiled layout, qmoe.h): value = (d * sc_j) * q - dmin * m_j for
// sub-block j = e / 32; both products are exact in fp32 (11 + 6 + 4 and 11 + 6
// bits), so only the subtraction rounds.  Unit u is elements 8p .. 8p+7 of a
// super-block of row R: the low (p % 8 < 4) or high nibbles of code bytes
// 8 (p % 4) .. +7 of quarter p / 8.
template <int OUT>
__global__ __launch_bounds__(256) void dequant_q4_k_kernel(const uint8_t* __restrict__ qs,
                                                           const uint8_t* __restrict__ sc,
                                                           const uint16_t* __restrict__ d,
                                                           const uint16_t* __restrict__ dmin,
                                                           int64_t n_units, int64_t SB, void* __restrict__ out) {
  for (int64_t u = blockIdx.x * 256ll + threadIdx.x; u < n_units; u += (int64_t)gridDim.x * 256) {
    const int64_t R = u / (SB * 32), ur = u - R * SB * 32;
    const int64_t sb = ur >> 5, t = (R >> 4) * SB + sb, r = R & 15;
    const int p = (int)(ur & 31);
    const int h = p >> 3, cb = 8 * (p & 3), shift = 4 * ((p >> 2) & 1), j = p >> 2;
    const u2_t q = *(const u2_t*)(qs + ((t * 4 + h) * 16 + r) * 32 + cb);
    const float dl = f16_to_f32(d[t * 16 + r]) * (float)sc[(t * 16 + r) * 16 + j];
    const float ml = f16_to_f32(dmin[t * 16 + r]) * (float)sc[(t * 16 + r) * 16 + 8 + j];
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = (q[i >> 2] >> (8 * (i & 3) + shift)) & 15u;
      v[i] = dl * (float)c - ml;
    }
    store8<OUT>(out, u, v);
  }
}

// Q6_K (tiled layout, qmoe.h): value = (d * sc_s) * (q - 32) for sub-block
// s = e / 16; d * sc is exact in fp32, the product with q - 32 rounds once.
// Unit u is elements 8p .. 8p+7 of a super-block of row R: low nibbles from
// quarter p / 8 of qs (high nibbles when p % 8 >= 4), top bit pairs from half
// p / 16 of qh at bits 2 ((p % 16) / 4).
template <int OUT>
__global__ __launch_bounds__(256) void dequant_q6_k_kernel(const uint8_t* __restrict__ qs,
                                                           const uint8_t* __restrict__ qh,
                                                           const int8_t* __restrict__ sc,
                                                           const uint16_t* __restrict__ d,
                                                           int64_t n_units, int64_t SB, void* __restrict__ out) {
  for (int64_t u = blockIdx.x * 256ll + threadIdx.x; u < n_units; u += (int64_t)gridDim.x * 256) {
    const int64_t R = u / (SB * 32), ur = u - R * SB * 32;
    const int64_t sb = ur >> 5, t = (R >> 4) * SB + sb, r = R & 15;
    const int p = (int)(ur & 31);
    const int cb = 8 * (p & 3);
    const int sn = 4 * ((p >> 2) & 1), sh = 2 * ((p & 15) >> 2);
    const u2_t lo = *(const u2_t*)(qs + ((t * 4 + (p >> 3)) * 16 + r) * 32 + cb);
    const u2_t hi = *(const u2_t*)(qh + ((t * 2 + (p >> 4)) * 16 + r) * 32 + cb);
    const float ds = f16_to_f32(d[t * 16 + r]) * (float)sc[(t * 16 + r) * 16 + (p >> 1)];
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = ((lo[i >> 2] >> (8 * (i & 3) + sn)) & 15u) | (((hi[i >> 2] >> (8 * (i & 3) + sh)) & 3u) << 4);
      v[i] = ds * (float)((int)c - 32);
    }
    store8<OUT>(out, u, v);
  }
}

// Q2_K: value = (d * a) * q - dmin * m with the sub-block's scale a (low
// nibble) and min m (high nibble); element e's 2-bit code is in code byte
// 32*(e/128) + e%32 at bit 2*((e%128)/32).  Tiled layout (qmoe.h): unit u
// is 8-value unit p of super-block sb of row R.
template <int OUT>
__global__ __launch_bounds__(256) void dequant_q2_k_kernel(const uint8_t* __restrict__ qs,
                                                           const uint8_t* __restrict__ sc,
                                                           const uint16_t* __restrict__ d,
                                                           const uint16_t* __restrict__ dmin,
                                                           int64_t n_units, int64_t SB, void* __restrict__ out) {
  for (int64_t u = blockIdx.x * 256ll + threadIdx.x; u < n_units; u += (int64_t)gridDim.x * 256) {
    const int64_t R = u / (SB * 32), ur = u - R * SB * 32;
    const int64_t sb = ur >> 5, t = (R >> 4) * SB + sb, r = R & 15;
    const int p = (int)(ur & 31);            // elements 8p .. 8p+7 of the block
    const int h = p >> 4, cb = 8 * (p & 3);  // code bytes 32h + cb .. +7
    const int shift = 2 * ((p & 15) >> 2);
    const u2_t q = *(const u2_t*)(qs + ((t * 2 + h) * 16 + r) * 32 + cb);
    const uint32_t s = sc[(t * 16 + r) * 16 + (p >> 1)];
    const float dl = f16_to_f32(d[t * 16 + r]) * (float)(s & 15u);
    const float ml = f16_to_f32(dmin[t * 16 + r]) * (float)(s >> 4);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t c = (q[i >> 2] >> (8 * (i & 3) + shift)) & 3u;
      v[i] = dl * (float)c - ml;
    }
    store8<OUT>(out, u, v);
  }
}

// IQ2_XXS: octet j of group g takes magnitudes grid[idx_j][0..7], signs from
// signs[(aux >> 7j) & 127] (bit l negates element l), scale d*(0.5+aux>>28)/4.
// Tiled layout (qmoe.h): (index word, aux word) pairs by group and row.
template <int OUT>
__global__ __launch_bounds__(256) void dequant_iq2_xxs_kernel(const uint32_t* __restrict__ qs,
                                                              const uint16_t* __restrict__ d,
                                                              const uint8_t* __restrict__ grid,
                                                              const uint8_t* __restrict__ signs,
                                                              int64_t n_units, int64_t SB, void* __restrict__ out) {
  __shared__ uint8_t lgrid[2048];
  __shared__ uint8_t lsign[128];
  for (int i = threadIdx.x; i < 512; i += 256) ((uint32_t*)lgrid)[i] = ((const uint32_t*)grid)[i];
  if (threadIdx.x < 32) ((uint32_t*)lsign)[threadIdx.x] = ((const uint32_t*)signs)[threadIdx.x];
  __syncthreads();
  for (int64_t u = blockIdx.x * 256ll + threadIdx.x; u < n_units; u += (int64_t)gridDim.x * 256) {
    const int64_t R = u / (SB * 32), ur = u - R * SB * 32;
    const int64_t sb = ur >> 5, t = (R >> 4) * SB + sb, r = R & 15;
    const int p = (int)(ur & 31);
    const int g = p >> 2, j = p & 3;
    const u2_t ia = *(const u2_t*)(qs + ((t * 8 + g) * 16 + r) * 2);
    const uint32_t ix = (ia[0] >> (8 * j)) & 0xFFu;
    const uint32_t a = ia[1];
    const uint32_t mask = lsign[(a >> (7 * j)) & 127u];
    const float db = f16_to_f32(d[t * 16 + r]) * (0.5f + (float)(a >> 28)) * 0.25f;
    float v[8];
#pragma unroll
    for (int l = 0; l < 8; ++l) {
      const float m = db * (float)lgrid[ix * 8 + l];
      v[l] = ((mask >> l) & 1u) ? -m : m;
    }
    store8<OUT>(out, u, v);
  }
}

// int4 affine: value = s * q + b per group, read from the tiled GPU layout
// (qmoe.h): unit u is word w = u % (k/8) of row R = u / (k/8).
template <int OUT>
__global__ __launch_bounds__(256) void dequant_int4_kernel(const uint32_t* __restrict__ qs,
                                                           const uint32_t* __restrict__ sb,
                                                           int64_t n_units, int64_t words_per_row,
                                                           int group, void* __restrict__ out) {
  const int64_t kt_n = words_per_row / 8, G = words_per_row * 8 / group;
  for (int64_t u = blockIdx.x * 256ll + threadIdx.x; u < n_units; u += (int64_t)gridDim.x * 256) {
    const int64_t R = u / words_per_row;
    const int64_t w = u - R * words_per_row;
    const int64_t rb = R >> 4, r = R & 15;
    const int64_t kt = w >> 3, g = (w >> 1) & 3, h = w & 1;
    const uint32_t word = qs[((rb * kt_n + kt) * 64 + 16 * g + r) * 2 + h];
    const uint32_t p = sb[(rb * G + (w * 8) / group) * 16 + r];
    const float s = f16_to_f32(p & 0xFFFFu);
    const float bb = f16_to_f32(p >> 16);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = s * (float)((word >> (4 * i)) & 15u) + bb;
      v[2 * i + 1] = s * (float)((word >> (4 * i + 16)) & 15u) + bb;
    }
    store8<OUT>(out, u, v);
  }
}

static inline unsigned grid_for(int64_t units) {
  int64_t g = (units + 255) / 256;
  if (g > (1 << 20)) g = 1 << 20;
  return (unsigned)(g < 1 ? 1 : g);
}

// MXFP4: value = e2m1(code) * 2^(e - 127) over 32-value blocks (OCP MX, the
// GGUF page's MXFP4 dequant commit).  The E2M1 values are exact in fp16, the
// product with the power-of-two scale is exact in fp32 unless it leaves fp32's
// range.  Tiled layout (qmoe.h): unit u is tiled word w (elements 8w .. 8w+7)
// of block j of row R.
template <int OUT>
__global__ __launch_bounds__(256) void dequant_mxfp4_kernel(const uint32_t* __restrict__ qs,
                                                            const uint8_t* __restrict__ e,
                                                            int64_t n_units, int64_t k, void* __restrict__ out) {
  const int64_t upr = k / 8, KT = k / 64;
  for (int64_t u = blockIdx.x * 256ll + threadIdx.x; u < n_units; u += (int64_t)gridDim.x * 256) {
    const int64_t R = u / upr, kk = 8 * (u - R * upr);
    const int64_t rb = R >> 4, r = R & 15, kt = kk >> 6, j = (kk & 63) >> 5, w = (kk & 31) >> 3;
    const uint32_t q = qs[(((rb * KT + kt) * 2 + j) * 16 + r) * 4 + w];
    const float s = e8m0_to_f32(e[(rb * (k / 32) + (kk >> 5)) * 16 + r]);
    const u4_t p = fp4x8_pairs<ACT_F16>(q);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = f16_to_f32((p[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) * s;
    store8<OUT>(out, u, v);
  }
}

// FP8 block weights: value = e4m3(code) * scale of the 128 x 128 block (the
// GGUF page's FP8 block dequant commit).  The code converts exactly to fp32
// (v_cvt_pk_f32_fp8, OCP E4M3 on gfx950, 0x7F / 0xFF NaN) and the product
// rounds once.  Codes tiled like Q8_0's; unit u is values 8(u % (k/8)) .. +7
// of row R = u / (k/8).
template <int OUT>
__global__ __launch_bounds__(256) void dequant_fp8_kernel(const uint8_t* __restrict__ qs,
                                                          const float* __restrict__ scales,
                                                          int64_t n_units, int64_t k, void* __restrict__ out) {
  const int64_t upr = k / 8, KT = k / 64;
  for (int64_t u = blockIdx.x * 256ll + threadIdx.x; u < n_units; u += (int64_t)gridDim.x * 256) {
    const int64_t R = u / upr, kk = 8 * (u - R * upr);
    const int64_t rb = R >> 4, r = R & 15, kt = kk >> 6, c = (kk & 63) >> 4;
    const u2_t q = *(const u2_t*)(qs + (((rb * KT + kt) * 4 + c) * 16 + r) * 16 + (kk & 15));
    const float s = scales[(R >> 7) * (k >> 7) + (kk >> 7)];
    float v[8];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const f2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[w], false);
      const f2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[w], true);
      v[4 * w + 0] = lo[0] * s;
      v[4 * w + 1] = lo[1] * s;
      v[4 * w + 2] = hi[0] * s;
      v[4 * w + 3] = hi[1] * s;
    }
    store8<OUT>(out, u, v);
  }
}

#define QMOE_DISPATCH_OUT(dtype, KERNEL, ...)                                         \
  do {                                                                                \
    if ((dtype) == QMOE_F32) hipLaunchKernelGGL(KERNEL<QMOE_F32>, __VA_ARGS__);       \
    else if ((dtype) == QMOE_F16) hipLaunchKernelGGL(KERNEL<QMOE_F16>, __VA_ARGS__);  \
    else hipLaunchKernelGGL(KERNEL<QMOE_BF16>, __VA_ARGS__);                          \
  } while (0)

void launch_dequant_q8_0(const int8_t* qs, const uint16_t* d, int64_t rows, int64_t k, void* out,
                         int dtype, hipStream_t s) {
  const int64_t units = rows * (k / 8);
  QMOE_DISPATCH_OUT(dtype, dequant_q8_0_kernel, dim3(grid_for(units)), dim3(256), 0, s, qs, d,
                    units, k, out);
}
void launch_dequant_q2_k(const uint32_t* qs, const uint8_t* sc, const uint16_t* d,
                         const uint16_t* dmin, int64_t rows, int64_t k, void* out, int dtype,
                         hipStream_t s) {
  const int64_t units = rows * (k / 8);
  QMOE_DISPATCH_OUT(dtype, dequant_q2_k_kernel, dim3(grid_for(units)), dim3(256), 0, s, (const uint8_t*)qs, sc,
                    d, dmin, units, k / 256, out);
}
void launch_dequant_q4_k(const uint8_t* qs, const uint8_t* sc, const uint16_t* d, const uint16_t* dmin,
                         int64_t rows, int64_t k, void* out, int dtype, hipStream_t s) {
  const int64_t units = rows * (k / 8);
  QMOE_DISPATCH_OUT(dtype, dequant_q4_k_kernel, dim3(grid_for(units)), dim3(256), 0, s, qs, sc, d, dmin, units,
                    k / 256, out);
}
void launch_dequant_q6_k(const uint8_t* qs, const uint8_t* qh, const int8_t* sc, const uint16_t* d, int64_t rows,
                         int64_t k, void* out, int dtype, hipStream_t s) {
  const int64_t units = rows * (k / 8);
  QMOE_DISPATCH_OUT(dtype, dequant_q6_k_kernel, dim3(grid_for(units)), dim3(256), 0, s, qs, qh, sc, d, units,
                    k / 256, out);
}
void launch_dequant_iq2_xxs(const uint32_t* qs, const uint16_t* d, const uint8_t* grid, const uint8_t* signs,
                            int64_t rows, int64_t k, void* out, int dtype, hipStream_t s) {
  const int64_t units = rows * (k / 8);
  QMOE_DISPATCH_OUT(dtype, dequant_iq2_xxs_kernel, dim3(grid_for(units)), dim3(256), 0, s, qs, d, grid, signs,
                    units, k / 256, out);
}
void launch_dequant_mxfp4(const uint32_t* qs, const uint8_t* e, int64_t rows, int64_t k, void* out,
                          int dtype, hipStream_t s) {
  const int64_t units = rows * (k / 8);
  QMOE_DISPATCH_OUT(dtype, dequant_mxfp4_kernel, dim3(grid_for(units)), dim3(256), 0, s, qs, e, units, k, out);
}
void launch_dequant_fp8(const uint8_t* qs, const float* sc, int64_t rows, int64_t k, void* out, int dtype,
                        hipStream_t s) {
  const int64_t units = rows * (k / 8);
  QMOE_DISPATCH_OUT(dtype, dequant_fp8_kernel, dim3(grid_for(units)), dim3(256), 0, s, qs, sc, units, k, out);
}
void launch_dequant_int4(const uint32_t* qs, const uint32_t* sb, int64_t rows, int64_t k, int group,
                         void* out, int dtype, hipStream_t s) {
  const int64_t units = rows * (k / 8);
  QMOE_DISPATCH_OUT(dtype, dequant_int4_kernel, dim3(grid_for(units)), dim3(256), 0, s, qs, sb,
                    units, k / 8, group, out);
}

}  // namespace qmoe
