// Top-k combine kernels.
//
// The Everything Bagel 2 page accumulates the top-K expert outputs into one
// hidden-state vector with a device-scalar FMA (out = base + w * value, fused
// 8-way for top-8); the DSV4 campaign page folds the weighted sum into the
// down projection.  Here:
//  * combine_cast_kernel finishes the atomic scatter-add of the prefill down
//    GEMM: one rounding of the fp32 accumulator to the output dtype, and the
//    accumulator is cleared for the next call (no separate memset launch);
//  * moe_combine_kernel is the deterministic alternative: for each token it
//    adds its k expert outputs (gathered through the plan's inverse map) in
//    ascending j, in fp32, then rounds once.
#include "common.h"

namespace qmoe {

template <int OUT>
__global__ __launch_bounds__(256) void combine_cast_kernel(float* __restrict__ acc, int64_t n4,
                                                           void* __restrict__ out) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const f4_t v = ((f4_t*)acc)[i];
    ((f4_t*)acc)[i] = f4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (OUT == QMOE_F32) {
      ((f4_t*)out)[i] = v;
    } else if constexpr (OUT == QMOE_F16) {
      ((u2_t*)out)[i] = u2_t{(uint32_t)f32_to_f16(v[0]) | ((uint32_t)f32_to_f16(v[1]) << 16),
                             (uint32_t)f32_to_f16(v[2]) | ((uint32_t)f32_to_f16(v[3]) << 16)};
    } else {
      ((u2_t*)out)[i] = u2_t{(uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                             (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16)};
    }
  }
}

__global__ __launch_bounds__(256) void combine_cast_tail_kernel(float* __restrict__ acc, int64_t i0,
                                                                int64_t n, void* __restrict__ out,
                                                                int out_dtype) {
  const int64_t i = i0 + threadIdx.x;
  if (i < n) {
    store_out(out, out_dtype, i, acc[i]);
    acc[i] = 0.f;
  }
}

// grid = T * ceil(N / 256) blocks.
__global__ __launch_bounds__(256) void moe_combine_kernel(const void* __restrict__ y, int y_dtype,
                                                          const int32_t* __restrict__ plan, int64_t P,
                                                          int E, int topk, const float* __restrict__ w,
                                                          int64_t N, const float* __restrict__ base,
                                                          void* __restrict__ out, int out_dtype) {
  const int64_t nb = (N + 255) / 256;
  const int64_t t = blockIdx.x / nb;
  const int64_t n = (blockIdx.x - t * nb) * 256 + threadIdx.x;
  if (n >= N) return;
  const PlanLayout L = plan_layout(P, E);
  float acc = base ? base[t * N + n] : 0.f;
  for (int j = 0; j < topk; ++j) {
    const int pos = plan[L.inv + t * topk + j];
    if (pos < 0) continue;
    const int64_t i = (int64_t)pos * N + n;
    float v;
    if (y_dtype == QMOE_F32) v = ((const float*)y)[i];
    else if (y_dtype == QMOE_F16) v = f16_to_f32(((const uint16_t*)y)[i]);
    else v = bf16_to_f32(((const uint16_t*)y)[i]);
    acc = __builtin_fmaf(w[t * topk + j], v, acc);
  }
  store_out(out, out_dtype, t * N + n, acc);
}

void launch_combine_cast(float* acc, int64_t n, void* out, int out_dtype, hipStream_t s) {
  const int64_t n4 = n / 4;
  if (n4 > 0) {
    int64_t g = (n4 + 255) / 256;
    if (g > 8192) g = 8192;
    if (out_dtype == QMOE_F32) hipLaunchKernelGGL(combine_cast_kernel<QMOE_F32>, dim3(g), dim3(256), 0, s, acc, n4, out);
    else if (out_dtype == QMOE_F16) hipLaunchKernelGGL(combine_cast_kernel<QMOE_F16>, dim3(g), dim3(256), 0, s, acc, n4, out);
    else hipLaunchKernelGGL(combine_cast_kernel<QMOE_BF16>, dim3(g), dim3(256), 0, s, acc, n4, out);
  }
  if (n4 * 4 < n)
    hipLaunchKernelGGL(combine_cast_tail_kernel, dim3(1), dim3(256), 0, s, acc, n4 * 4, n, out, out_dtype);
}

void launch_moe_combine(const void* y, int y_dtype, const int32_t* plan, int64_t t, int topk, int E,
                        const float* w, int64_t N, const float* base, void* out, int out_dtype,
                        hipStream_t s) {
  const dim3 grid((unsigned)(((N + 255) / 256) * t));
  hipLaunchKernelGGL(moe_combine_kernel, grid, dim3(256), 0, s, y, y_dtype, plan, t * topk, E, topk,
                     w, N, base, out, out_dtype);
}

}  // namespace qmoe
