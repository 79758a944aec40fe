// Routing plan: expert histogram, offsets and tile list (one workgroup), then
// a stable expert-sorted scatter of the routed pairs (one workgroup per
// expert).  The DSV4 campaign page's map0 work queue maps experts to tiles of
// routed tokens for the tiled MoE prefill GEMM; the Everything Bagel 2 page
// keeps router ids on the device.  Pairs keep ascending pair order inside an
// expert, so the plan is unique and identical from run to run.
#include "common.h"

namespace qmoe {

// One workgroup of 1024 threads: counts, exclusive offsets, tile list, header.
__global__ __launch_bounds__(1024) void plan_count_kernel(const int32_t* __restrict__ ids, int64_t P,
                                                          int E, int bm, int64_t t, int topk,
                                                          int32_t* __restrict__ plan) {
  __shared__ int hist[QMOE_MAX_EXPERTS];
  __shared__ int scan_a[QMOE_MAX_EXPERTS];
  __shared__ int scan_t[QMOE_MAX_EXPERTS];
  __shared__ int dropped;
  const int tid = threadIdx.x;
  if (tid < QMOE_MAX_EXPERTS) hist[tid] = 0;
  if (tid == 0) dropped = 0;
  __syncthreads();
  int my_drop = 0;
  for (int64_t p = tid; p < P; p += 1024) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    else ++my_drop;
  }
  if (my_drop) atomicAdd(&dropped, my_drop);
  __syncthreads();
  // inclusive scans of counts and of tiles-per-expert (Hillis-Steele over 1024 slots)
  const int c = (tid < E) ? hist[tid] : 0;
  const int nt = (c + bm - 1) / bm;
  scan_a[tid] = c;
  scan_t[tid] = nt;
  __syncthreads();
  for (int off = 1; off < QMOE_MAX_EXPERTS; off <<= 1) {
    const int va = tid >= off ? scan_a[tid - off] : 0;
    const int vt = tid >= off ? scan_t[tid - off] : 0;
    __syncthreads();
    scan_a[tid] += va;
    scan_t[tid] += vt;
    __syncthreads();
  }
  const PlanLayout L = plan_layout(P, E);
  if (tid < E) {
    const int row0 = scan_a[tid] - c;     // exclusive offset
    const int tile0 = scan_t[tid] - nt;
    plan[L.counts + tid] = c;
    plan[L.offsets + tid] = row0;
    for (int i = 0; i < nt; ++i) {
      int32_t* tl = plan + L.tiles + 4 * (int64_t)(tile0 + i);
      tl[0] = tid;
      tl[1] = row0 + i * bm;
      tl[2] = min(bm, c - i * bm);
      tl[3] = 0;
    }
  }
  if (tid == 0) {
    const int total = scan_a[QMOE_MAX_EXPERTS - 1];
    plan[0] = dropped;
    plan[1] = scan_t[QMOE_MAX_EXPERTS - 1];
    plan[2] = total;
    plan[3] = bm;
    plan[4] = (int32_t)t;
    plan[5] = topk;
    plan[6] = E;
    plan[7] = 0;
    plan[L.offsets + E] = total;
  }
}

// Workgroup e writes expert e's pairs, in ascending pair order, to
// sorted[offsets[e] + rank] and records the inverse map.  Workgroup 0 also
// marks dropped pairs in the inverse map.
__global__ __launch_bounds__(256) void plan_scatter_kernel(const int32_t* __restrict__ ids, int64_t P,
                                                           int E, int bm, int32_t* __restrict__ plan) {
  const int e = blockIdx.x;
  const PlanLayout L = plan_layout(P, E);
  const int count = plan[L.counts + e];
  if (count == 0 && e != 0) return;
  const int base = plan[L.offsets + e];
  __shared__ int wave_n[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int found = 0;
  for (int64_t p0 = 0; p0 < P && (found < count || e == 0); p0 += 256) {
    const int64_t p = p0 + tid;
    const int id = p < P ? ids[p] : -1;
    const bool hit = (p < P) && id == e;
    if (e == 0 && p < P && !(id >= 0 && id < E)) plan[L.inv + p] = -1;
    const uint64_t bal = __ballot(hit);
    if (lane == 0) wave_n[wave] = __popcll(bal);
    __syncthreads();
    int before = found;
    for (int w = 0; w < wave; ++w) before += wave_n[w];
    const int total = wave_n[0] + wave_n[1] + wave_n[2] + wave_n[3];
    if (hit) {
      const int rank = before + __popcll(bal & ((1ull << lane) - 1ull));
      plan[L.sorted + base + rank] = (int32_t)p;
      plan[L.inv + p] = base + rank;
    }
    found += total;
    __syncthreads();
  }
}

void launch_plan(const int32_t* ids, int64_t t, int topk, int E, int bm, int32_t* plan,
                 hipStream_t s) {
  const int64_t P = t * topk;
  hipLaunchKernelGGL(plan_count_kernel, dim3(1), dim3(1024), 0, s, ids, P, E, bm, t, topk, plan);
  hipLaunchKernelGGL(plan_scatter_kernel, dim3(E), dim3(256), 0, s, ids, P, E, bm, plan);
}

}  // namespace qmoe
