// Router top-k: per token, the k best experts and their gather weights, from
// the router logits, on the device.
//
// Two scorings:
//   * softmax top-k [Everything Bagel 2, the commit moving the MoE router
//     top-K to the GPU]: the k largest logits; weights are a softmax over the
//     selected logits (they sum to 1).  With a per-expert bias (the LFM2-MoE
//     softmax-then-bias routing on the same page): p = softmax over all
//     experts, the k largest p + bias are selected, weights are the selected
//     p renormalised;
//   * DeepSeek V4 sqrtsoftplus [GGUF block-dequant + DSv4 kernel surface, the
//     routing scoring commit]: score s = sqrt(softplus(logit)) with the stable
//     softplus max(x, 0) + log(1 + exp(-|x|)); the k largest s + bias are
//     selected; the weight is s times the routed scaling factor.
//
// One wave per token.  Lane l holds experts l, l + 64, ... (NS slots, coalesced
// loads of the logit row).  Each expert's selection score becomes a 64-bit key
// whose unsigned order is (score, then lower expert index first): the high
// word is the score's bits mapped to an order-preserving integer (-0 and +0
// share one, NaN sorts below every number), the low word is ~expert.  A round
// is a per-lane maximum over its free slots and a wave maximum (DPP steps
// inside rows, then the four row maxima in scalar registers); the winner's key
// is cleared.  Integer keys make every
// lane agree on the winner, and the order of equal scores is fixed.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace qmoe {

constexpr int RT_WAVES = 4;  // tokens per 256-thread workgroup
constexpr int ROUTER_SOFTMAX_BIAS = 2;  // softmax scoring with a bias given

struct RouterArgs {
  const void* logits;
  int64_t t;
  int E, k, scoring;
  const float* bias;
  float scale;
  int32_t* ids;
  float* w;
};

__device__ __forceinline__ uint32_t score_key(float v) {
  if (v != v) return 0u;                                        // NaN: below everything
  const int32_t b = __builtin_bit_cast(int32_t, v == 0.0f ? 0.0f : v);
  return (uint32_t)(b ^ ((b >> 31) & 0x7fffffff)) ^ 0x80000000u;  // monotone, unsigned
}
// Inverse of score_key (the map is an involution on the low 31 bits): the
// selection score back from a key; the NaN key gives a NaN.
__device__ __forceinline__ float key_score(uint32_t k) {
  const int32_t b = (int32_t)(k ^ 0x80000000u);
  return __builtin_bit_cast(float, b ^ ((b >> 31) & 0x7fffffff));
}

// One maximum step with the partner lane given by a DPP control (quad
// permutes and row mirrors stay inside a row of 16 lanes).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, 0xf, 0xf, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > v ? o : v;
}

// Wave maximum of a 64-bit key, uniform result: lane swaps 1 and 2 inside each
// quad, then the half-row and row mirrors, leave every lane of a row holding
// the row's maximum; the four row maxima are read into scalar registers.
// The whole wave must be active.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_max_step<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_max_step<0x141>(v);  // row_half_mirror
  v = dpp_max_step<0x140>(v);  // row_mirror
  uint64_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 16 * r);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 16 * r);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    m = o > m ? o : m;
  }
  return m;
}

// Wave sum of a float with the same partner pattern; every lane gets the same
// bits (each step adds the same two values on both partners).
__device__ __forceinline__ float wave_sum_f32(float v) {
  auto step = [](float x, auto ctrl) {
    const uint32_t o = __builtin_amdgcn_update_dpp(0u, __builtin_bit_cast(uint32_t, x), decltype(ctrl)::value,
                                                   0xf, 0xf, false);
    return x + __builtin_bit_cast(float, o);
  };
  v = step(v, std::integral_constant<int, 0xB1>{});
  v = step(v, std::integral_constant<int, 0x4E>{});
  v = step(v, std::integral_constant<int, 0x141>{});
  v = step(v, std::integral_constant<int, 0x140>{});
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(uint32_t, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(uint32_t, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(uint32_t, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(uint32_t, v), 48));
  return (r0 + r1) + (r2 + r3);
}

template <int DT>
__device__ __forceinline__ float load_logit(const void* p, int64_t i) {
  if constexpr (DT == QMOE_F32) return ((const float*)p)[i];
  else if constexpr (DT == QMOE_F16) return f16_to_f32(((const uint16_t*)p)[i]);
  else return bf16_to_f32(((const uint16_t*)p)[i]);
}

template <int DT, int NS, int SCORING>
__global__ __launch_bounds__(64 * RT_WAVES) void router_topk_kernel(RouterArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * RT_WAVES + (threadIdx.x >> 6);
  if (tok >= a.t) return;  // whole wave leaves; no barrier follows

  // Softmax selects on the logit itself, which the winning key gives back;
  // the other scorings keep the weight's value (unbiased score or
  // probability) beside the key.
  constexpr int NV = SCORING == QMOE_ROUTER_SOFTMAX ? 1 : NS;
  uint64_t key[NS];  // 0: no expert (past E) or already selected
  float val[NV];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int e = lane + 64 * s;
    key[s] = 0;
    if (s < NV) val[s] = 0.0f;
    if (e < a.E) {
      const float x = load_logit<DT>(a.logits, tok * a.E + e);
      float sel = x;
      if constexpr (SCORING == QMOE_ROUTER_SQRTSOFTPLUS) {
        const float sp = fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
        const float sc = sqrtf(sp);
        sel = a.bias ? sc + a.bias[e] : sc;
        val[s] = sc;
      } else if constexpr (SCORING == ROUTER_SOFTMAX_BIAS) {
        val[s] = x;  // the logit, until the softmax below
      }
      key[s] = ((uint64_t)score_key(sel) << 32) | (uint32_t)~(uint32_t)e;
    }
  }
  if constexpr (SCORING == ROUTER_SOFTMAX_BIAS) {
    // p = softmax over all experts in fp32, then the selection key p + bias
    uint64_t kmax = key[0];
#pragma unroll
    for (int s = 1; s < NS; ++s) kmax = key[s] > kmax ? key[s] : kmax;
    const float m = key_score((uint32_t)(wave_max_u64(kmax) >> 32));
    float part = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float ex = key[s] ? expf(val[s] - m) : 0.0f;
      val[s] = ex;
      part += ex;
    }
    const float inv = 1.0f / wave_sum_f32(part);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int e = lane + 64 * s;
      if (key[s]) {
        val[s] *= inv;
        key[s] = ((uint64_t)score_key(val[s] + a.bias[e]) << 32) | (uint32_t)~(uint32_t)e;
      }
    }
  }

  // k rounds; lane j keeps the expert and value of round j.  Every lane sees
  // the same winners, so the softmax maximum (round 0) and sum are uniform.
  int idj = 0;
  float vj = 0.0f, m = 0.0f, sum = 0.0f;
  for (int j = 0; j < a.k; ++j) {
    uint64_t best = key[0];
    float bv = val[0];
#pragma unroll
    for (int s = 1; s < NS; ++s) {
      const bool ok = key[s] > best;
      best = ok ? key[s] : best;
      if constexpr (NV == NS) bv = ok ? val[s] : bv;
    }
    const uint64_t win = wave_max_u64(best);
#pragma unroll
    for (int s = 0; s < NS; ++s) key[s] = key[s] == win ? 0ull : key[s];  // keys are unique
    const int e = (int)~(uint32_t)win;
    float v;
    if constexpr (SCORING == QMOE_ROUTER_SOFTMAX) v = key_score((uint32_t)(win >> 32));
    else v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(uint32_t, bv), e & 63));
    if constexpr (SCORING == QMOE_ROUTER_SOFTMAX) {
      if (j == 0) m = v;  // the first selection is the largest logit
      sum += expf(v - m);
    } else if constexpr (SCORING == ROUTER_SOFTMAX_BIAS) {
      sum += v;
    }
    if (j == lane) { idj = e; vj = v; }
  }

  float wj;
  if constexpr (SCORING == QMOE_ROUTER_SQRTSOFTPLUS) wj = vj * a.scale;
  else if constexpr (SCORING == ROUTER_SOFTMAX_BIAS) wj = vj / sum;
  else wj = expf(vj - m) / sum;
  if (lane < a.k) {
    a.ids[tok * a.k + lane] = idj;
    a.w[tok * a.k + lane] = wj;
  }
}

// One instantiation per slot count ceil(E / 64) = 1 .. 16.
template <int DT, int SCORING, int NS = 1>
static void launch_ns(const RouterArgs& a, int ns, dim3 g, hipStream_t s) {
  if constexpr (NS < 16) {
    if (ns > NS) return launch_ns<DT, SCORING, NS + 1>(a, ns, g, s);
  }
  hipLaunchKernelGGL((router_topk_kernel<DT, NS, SCORING>), g, dim3(64 * RT_WAVES), 0, s, a);
}

template <int DT>
static void launch_dt(const RouterArgs& a, int ns, dim3 g, hipStream_t s) {
  if (a.scoring == QMOE_ROUTER_SQRTSOFTPLUS) launch_ns<DT, QMOE_ROUTER_SQRTSOFTPLUS>(a, ns, g, s);
  else if (a.bias) launch_ns<DT, ROUTER_SOFTMAX_BIAS>(a, ns, g, s);
  else launch_ns<DT, QMOE_ROUTER_SOFTMAX>(a, ns, g, s);
}

void launch_router_topk(const void* logits, int dtype, int64_t t, int E, int k, int scoring,
                        const float* bias, float scale, int32_t* ids, float* w, hipStream_t s) {
  RouterArgs a{logits, t, E, k, scoring, bias, scale, ids, w};
  const int ns = (E + 63) / 64;
  const dim3 g((unsigned)((t + RT_WAVES - 1) / RT_WAVES));
  if (dtype == QMOE_F32) launch_dt<QMOE_F32>(a, ns, g, s);
  else if (dtype == QMOE_F16) launch_dt<QMOE_F16>(a, ns, g, s);
  else launch_dt<QMOE_BF16>(a, ns, g, s);
}

}  // namespace qmoe
