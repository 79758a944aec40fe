// Routing plan: the expert-sorted token gather with per-expert tiles.
//
// The DSV4 campaign page's map0 work queue maps experts to tiles of routed
// tokens for the tiled MoE prefill GEMM; the Everything Bagel 2 page keeps the
// router ids on the device.  Pairs keep ascending pair order inside an expert,
// so the plan is unique and identical from run to run.
//
// Two short launches over chunks of 1024 pairs (one 1024-thread workgroup
// per chunk, one pair per thread):
//   1. chunk histograms: per-expert counts of each chunk;
//   2. each chunk sums the histograms into expert counts, its own bases and
//      the offsets (chunk 0 also writes the counts, offsets, tile list and
//      header), recomputes its in-chunk ranks and scatters its pairs.
// A wave finds the lanes that share its expert with one ballot per bit of the
// expert id, so ranks are exact without sorting; waves are combined through
// per-wave counts in LDS in wave order.  Chunk histograms live in the plan
// buffer's scratch area after the inverse map.
#include "common.h"

namespace qmoe {

constexpr int PC = PLAN_CHUNK;  // pairs per chunk (per workgroup)

struct PlanArgs {
  const int32_t* ids;
  int64_t P;
  int E, bm, topk;
  int64_t t;
  int32_t* plan;
  int nchunks;
  int nbits;  // expert ids are below 2^nbits
};

__device__ __forceinline__ int64_t hist_off(const PlanLayout& L) { return L.total; }

// Lanes of this wave holding the same key: one ballot per key bit (keys are
// below 2^nbits); lanes with key < 0 get an empty mask.
__device__ __forceinline__ uint64_t peers_of(int key, int nbits) {
  uint64_t m = __ballot(key >= 0);
  for (int bit = 0; bit < nbits; ++bit) {
    const bool on = (key >> bit) & 1;
    const uint64_t bal = __ballot(on);
    m &= on ? bal : ~bal;
  }
  return key >= 0 ? m : 0ull;
}

// One pair per thread: the expert of pair p (or -1), its rank among the
// wave's pairs of that expert, and per-wave counts in wcnt[wave][e].
__device__ __forceinline__ int wave_rank(const PlanArgs& a, int64_t p, int lane, int* wcnt_w,
                                         int& key) {
  int e = -1;
  if (p < a.P) {
    const int v = a.ids[p];
    e = (v >= 0 && v < a.E) ? v : -1;
  }
  const uint64_t peers = peers_of(e, a.nbits);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int before = __popcll(peers & lt);
  if (e >= 0 && before == 0) wcnt_w[e] = __popcll(peers);
  key = e;
  return before;
}

__global__ __launch_bounds__(1024) void plan_hist_kernel(PlanArgs a) {
  extern __shared__ int wcnt[];  // [16][E]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 16 * a.E; i += 1024) wcnt[i] = 0;
  __syncthreads();
  int key;
  wave_rank(a, (int64_t)blockIdx.x * PC + tid, lane, wcnt + wave * a.E, key);
  __syncthreads();
  const PlanLayout L = plan_layout(a.P, a.E);
  int32_t* hist = a.plan + hist_off(L) + (int64_t)blockIdx.x * a.E;
  for (int e = tid; e < a.E; e += 1024) {
    int s = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) s += wcnt[w * a.E + e];
    hist[e] = s;
  }
}

// Scan and scatter in one launch, one workgroup per chunk (thread = expert
// for the scan).  Every workgroup reads all chunk histograms: an expert's
// count is their sum, and this chunk's base within the expert is the sum
// over the chunks before it.  Offsets and tile counts come from a prefix sum
// over the experts in LDS; workgroup 0 also writes the counts, offsets, tile
// list and header.  Then each pair is placed at offset + chunk base + the
// ranks of earlier waves + its rank in its wave.
__global__ __launch_bounds__(1024) void plan_scan_scatter_kernel(PlanArgs a) {
  extern __shared__ int wcnt[];  // [16][E], then base[E]
  __shared__ int sa[QMOE_MAX_EXPERTS], st[QMOE_MAX_EXPERTS], sp[QMOE_MAX_EXPERTS];
  int* base = wcnt + 16 * a.E;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const PlanLayout L = plan_layout(a.P, a.E);
  const int32_t* hist = a.plan + hist_off(L);
  const int chunk = blockIdx.x;

  int c_e = 0, cb = 0;
  if (tid < a.E) {
    // unrolled so that eight histogram loads are in flight at a time
#pragma unroll 8
    for (int c = 0; c < a.nchunks; ++c) {
      const int v = hist[(int64_t)c * a.E + tid];
      if (c == chunk) cb = c_e;
      c_e += v;
    }
  }
  // Tile order: every expert's full tiles (bm rows) first, in expert order,
  // then the experts' last partial tiles.  Workgroups of the matmul take
  // tiles in this order, so a launch ends on its smallest tiles.
  const int nfull = c_e / a.bm, part = (c_e % a.bm) != 0;
  sa[tid] = c_e;
  st[tid] = nfull;
  sp[tid] = part;
  for (int i = tid; i < 16 * a.E; i += 1024) wcnt[i] = 0;
  __syncthreads();
  // inclusive scan over the first E entries (offsets up to the largest power
  // of two below E reach every earlier entry)
  for (int off = 1; off < a.E; off <<= 1) {
    const int va = tid >= off ? sa[tid - off] : 0;
    const int vt = tid >= off ? st[tid - off] : 0;
    const int vp = tid >= off ? sp[tid - off] : 0;
    __syncthreads();
    sa[tid] += va;
    st[tid] += vt;
    sp[tid] += vp;
    __syncthreads();
  }
  if (tid < a.E) {
    const int row0 = sa[tid] - c_e;
    base[tid] = row0 + cb;
    if (chunk == 0) {
      a.plan[L.counts + tid] = c_e;
      a.plan[L.offsets + tid] = row0;
      auto put = [&](int t, int i, int n) {
        int32_t* tl = a.plan + L.tiles + 4 * (int64_t)t;
        tl[0] = tid;
        tl[1] = row0 + i * a.bm;
        tl[2] = n;
        tl[3] = 0;
      };
      for (int i = 0; i < nfull; ++i) put(st[tid] - nfull + i, i, a.bm);
      if (part) put(st[a.E - 1] + sp[tid] - 1, nfull, c_e - nfull * a.bm);
    }
  }
  if (chunk == 0 && tid == 0) {
    const int total = sa[a.E - 1];
    a.plan[0] = (int32_t)(a.P - total);
    a.plan[1] = st[a.E - 1] + sp[a.E - 1];
    a.plan[2] = total;
    a.plan[3] = a.bm;
    a.plan[4] = (int32_t)a.t;
    a.plan[5] = a.topk;
    a.plan[6] = a.E;
    a.plan[7] = a.P >= SK_MIN_PAIRS ? SK_SLOTS : 0;
    a.plan[L.offsets + a.E] = total;
  }
  if (chunk == 0 && a.P >= SK_MIN_PAIRS) {  // work-balancing tickets start at zero
    int32_t* tk = a.plan + plan_sk_offset(a.P, a.E);
    for (int i = tid; i < SK_SLOTS; i += 1024) tk[i] = 0;
  }
  __syncthreads();  // base[] and the cleared counts

  int e;
  const int64_t p = (int64_t)chunk * PC + tid;
  const int rank = wave_rank(a, p, lane, wcnt + wave * a.E, e);
  __syncthreads();
  if (p >= a.P) return;
  if (e < 0) {
    a.plan[L.inv + p] = -1;
    return;
  }
  int wb = 0;
  for (int w = 0; w < wave; ++w) wb += wcnt[w * a.E + e];
  const int pos = base[e] + wb + rank;
  a.plan[L.sorted + pos] = (int32_t)p;
  a.plan[L.inv + p] = pos;
}

void launch_plan(const int32_t* ids, int64_t t, int topk, int E, int bm, int32_t* plan,
                 hipStream_t s) {
  PlanArgs a;
  a.ids = ids;
  a.P = t * topk;
  a.E = E;
  a.bm = bm;
  a.topk = topk;
  a.t = t;
  a.plan = plan;
  a.nchunks = (int)((a.P + PC - 1) / PC);
  a.nbits = 1;
  while ((1 << a.nbits) < E) ++a.nbits;
  const size_t lds = 16 * (size_t)E * sizeof(int);
  hipLaunchKernelGGL(plan_hist_kernel, dim3(a.nchunks), dim3(1024), lds, s, a);
  hipLaunchKernelGGL(plan_scan_scatter_kernel, dim3(a.nchunks), dim3(1024), lds + E * sizeof(int), s, a);
}

}  // namespace qmoe
