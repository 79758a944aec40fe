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
//    ascending j, in fp32, then rounds once.  Optionally the sum starts from
//    a shared expert's output, scaled by the sigmoid of a per-token gate
//    logit, and the residual stream is added before the rounding (the page's
//    sigmoid-gated scalar FMA with the post-MoE residual folded in).
#include "common.h"

namespace qmoe {

// The plan must name this call's tokens, top-k and experts (its tile height
// does not matter here); otherwise its inverse map has another layout.
__device__ __forceinline__ bool plan_header_ok(const int32_t* plan, int64_t P, int E, int topk) {
  return plan[4] == (int32_t)(P / topk) && plan[5] == topk && plan[6] == E;
}

template <int OUT>
__global__ __launch_bounds__(256) void combine_cast_kernel(float* __restrict__ acc, int64_t n4,
                                                           void* __restrict__ out) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const f4_t v = ((f4_t*)acc)[i];
    ((f4_t*)acc)[i] = f4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (OUT == QMOE_F32) {
      ((f4_t*)out)[i] = v;
    } else {
      constexpr bool HALF = (OUT == QMOE_F16);
      ((u2_t*)out)[i] = u2_t{f32x2_to_16<HALF>(v[0], v[1]), f32x2_to_16<HALF>(v[2], v[3])};
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
                                                          const float* __restrict__ gate, const void* res,
                                                          int res_dtype, void* out, int out_dtype) {
  const int64_t nb = (N + 255) / 256;
  const int64_t t = blockIdx.x / nb;
  const int64_t n = (blockIdx.x - t * nb) * 256 + threadIdx.x;
  if (n >= N) return;
  if (!plan_header_ok(plan, P, E, topk)) return;
  const PlanLayout L = plan_layout(P, E);
  float acc = base ? base[t * N + n] * (gate ? sigmoid_f32(gate[t]) : 1.0f) : 0.f;
  for (int j = 0; j < topk; ++j) {
    const int pos = plan[L.inv + t * topk + j];
    if (pos < 0) continue;
    const int64_t i = (int64_t)pos * N + n;
    const float v = load_act(y, y_dtype, i);
    acc = __builtin_fmaf(w[t * topk + j], v, acc);
  }
  if (res) acc += load_act(res, res_dtype, t * N + n);
  store_out(out, out_dtype, t * N + n, acc);
}

// The same sum, eight consecutive outputs per thread: a token's expert rows
// are read with 16-byte loads, all issued before the first FMA (buffer loads:
// a dropped pair reads zeros at no cost and is then skipped).  Requires N % 8
// == 0 and y under 4 GiB.  Sum order as above, so results are identical.
template <int YT>
__global__ __launch_bounds__(256) void moe_combine_vec_kernel(const void* __restrict__ y,
                                                              const int32_t* __restrict__ plan, int64_t P,
                                                              int E, int topk, const float* __restrict__ w,
                                                              int64_t N, const float* __restrict__ base,
                                                              const float* __restrict__ gate, const void* res,
                                                              int res_dtype, void* out, int out_dtype) {
  const int64_t nb = (N + 2047) / 2048;
  const int64_t t = blockIdx.x / nb;
  const int64_t n0 = ((blockIdx.x - t * nb) * 256 + threadIdx.x) * 8;
  if (n0 >= N) return;
  if (!plan_header_ok(plan, P, E, topk)) return;
  const PlanLayout L = plan_layout(P, E);
  constexpr int ES = YT == QMOE_F32 ? 4 : 2;  // bytes per y element
  const __amdgpu_buffer_rsrc_t yr =
      __builtin_amdgcn_make_buffer_rsrc((void*)y, (short)0, (int)(uint32_t)(P * N * ES), 0x00020000);
  int pos[QMOE_MAX_TOPK];
  float wt[QMOE_MAX_TOPK];
  u4_t v[QMOE_MAX_TOPK][ES / 2];
#pragma unroll
  for (int j = 0; j < QMOE_MAX_TOPK; ++j) {
    pos[j] = j < topk ? plan[L.inv + t * topk + j] : -1;
    wt[j] = j < topk ? w[t * topk + j] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < QMOE_MAX_TOPK; ++j) {
    const uint32_t off = pos[j] >= 0 ? (uint32_t)(((int64_t)pos[j] * N + n0) * ES) : 0x80000000u;
#pragma unroll
    for (int h = 0; h < ES / 2; ++h)
      v[j][h] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(yr, off + 16 * h, 0, 0));
  }
  float acc[8];
  const float gs = gate ? sigmoid_f32(gate[t]) : 1.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = base ? base[t * N + n0 + i] * gs : 0.f;
#pragma unroll
  for (int j = 0; j < QMOE_MAX_TOPK; ++j) {
    if (pos[j] < 0) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x;
      if constexpr (YT == QMOE_F32) {
        // through a scalar: a bit_cast applied to the vector element itself
        // reads element 0 with this compiler
        const uint32_t b = v[j][i / 4][i % 4];
        x = __builtin_bit_cast(float, b);
      } else {
        const uint32_t b = (v[j][0][i / 2] >> (16 * (i & 1))) & 0xFFFFu;
        x = YT == QMOE_F16 ? f16_to_f32(b) : bf16_to_f32(b);
      }
      acc[i] = __builtin_fmaf(wt[j], x, acc[i]);
    }
  }
  const int64_t o = t * N + n0;
  if (res) {
    // read before the store below: out may be the residual buffer itself
    if (res_dtype == QMOE_F32) {
      const f4_t r0 = ((const f4_t*)res)[o / 4], r1 = ((const f4_t*)res)[o / 4 + 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += r0[i];
        acc[4 + i] += r1[i];
      }
    } else {
      const u4_t r = ((const u4_t*)res)[o / 8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t b = (r[i / 2] >> (16 * (i & 1))) & 0xFFFFu;
        acc[i] += res_dtype == QMOE_F16 ? f16_to_f32(b) : bf16_to_f32(b);
      }
    }
  }
  if (out_dtype == QMOE_F32) {
    ((f4_t*)out)[o / 4] = f4_t{acc[0], acc[1], acc[2], acc[3]};
    ((f4_t*)out)[o / 4 + 1] = f4_t{acc[4], acc[5], acc[6], acc[7]};
  } else {
    u4_t r;
    if (out_dtype == QMOE_F16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = f32x2_to_16<true>(acc[2 * i], acc[2 * i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = f32x2_to_16<false>(acc[2 * i], acc[2 * i + 1]);
    }
    ((u4_t*)out)[o / 8] = r;
  }
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
                        const float* w, int64_t N, const float* base, const float* gate, const void* res,
                        int res_dtype, void* out, int out_dtype, hipStream_t s) {
  const int64_t ybytes = t * topk * N * (y_dtype == QMOE_F32 ? 4 : 2);
  if (N % 8 == 0 && ybytes < (1ll << 32)) {
    const dim3 grid((unsigned)(((N + 2047) / 2048) * t));
    if (y_dtype == QMOE_F32)
      hipLaunchKernelGGL(moe_combine_vec_kernel<QMOE_F32>, grid, dim3(256), 0, s, y, plan, t * topk, E, topk, w, N,
                         base, gate, res, res_dtype, out, out_dtype);
    else if (y_dtype == QMOE_F16)
      hipLaunchKernelGGL(moe_combine_vec_kernel<QMOE_F16>, grid, dim3(256), 0, s, y, plan, t * topk, E, topk, w, N,
                         base, gate, res, res_dtype, out, out_dtype);
    else
      hipLaunchKernelGGL(moe_combine_vec_kernel<QMOE_BF16>, grid, dim3(256), 0, s, y, plan, t * topk, E, topk, w, N,
                         base, gate, res, res_dtype, out, out_dtype);
    return;
  }
  const dim3 grid((unsigned)(((N + 255) / 256) * t));
  hipLaunchKernelGGL(moe_combine_kernel, grid, dim3(256), 0, s, y, y_dtype, plan, t * topk, E, topk,
                     w, N, base, gate, res, res_dtype, out, out_dtype);
}

}  // namespace qmoe
