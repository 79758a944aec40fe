// C ABI of libqmoe: argument validation on the host, then kernel launches on
// the caller's stream.  Contracts are checked before any launch and reported
// as status codes (the DSV4 campaign page's review fix moves such contracts to
// host-checked launchers instead of silent zeros); nothing here synchronises
// or allocates.
#include <string.h>

#include <atomic>

#include "common.h"

namespace qmoe {
void launch_dequant_q8_0(const int8_t*, const uint16_t*, int64_t, int64_t, void*, int, hipStream_t);
void launch_dequant_q2_k(const uint32_t*, const uint8_t*, const uint16_t*, const uint16_t*, int64_t, int64_t,
                         void*, int, hipStream_t);
void launch_dequant_iq2_xxs(const uint32_t*, const uint16_t*, const uint8_t*, const uint8_t*, int64_t, int64_t,
                            void*, int, hipStream_t);
void launch_dequant_q4_k(const uint8_t*, const uint8_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, void*,
                         int, hipStream_t);
void launch_dequant_q6_k(const uint8_t*, const uint8_t*, const int8_t*, const uint16_t*, int64_t, int64_t, void*,
                         int, hipStream_t);
void launch_dequant_mxfp4(const uint32_t*, const uint8_t*, int64_t, int64_t, void*, int, hipStream_t);
void launch_dequant_fp8(const uint8_t*, const float*, int64_t, int64_t, void*, int, hipStream_t);
void launch_dequant_int4(const uint32_t*, const uint32_t*, int64_t, int64_t, int, void*, int,
                         hipStream_t);
void launch_plan(const int32_t*, int64_t, int, int, int, int32_t*, hipStream_t);
void launch_qmm(const qmoe_weights*, const void*, int, int, const int32_t*, int64_t, int, int,
                int64_t, const float*, int, void*, int, hipStream_t);
int qmm_int4_bf16_max_groups();
int qmm_max_rows();
int launch_gemv(const qmoe_weights*, const void*, int, int64_t, const int32_t*, const float*, int,
                 int, void*, int, hipStream_t);
int64_t gemv_max_k();
void launch_combine_cast(float*, int64_t, void*, int, hipStream_t);
void launch_router_topk(const void*, int, int64_t, int, int, int, const float*, float, int32_t*,
                        float*, hipStream_t);
void launch_moe_combine(const void*, int, const int32_t*, int64_t, int, int, const float*, int64_t,
                        const float*, const float*, const void*, int, void*, int, hipStream_t);
}  // namespace qmoe

using namespace qmoe;

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

int check_arch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QMOE_ERR_ARCH;
  if (dev < 0 || dev >= kMaxDevices) return QMOE_ERR_ARCH;
  int v = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return QMOE_ERR_ARCH;
    v = (strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_arch_ok[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? QMOE_OK : QMOE_ERR_ARCH;
}

inline bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
inline bool dtype_ok(int d) { return d == QMOE_F32 || d == QMOE_F16 || d == QMOE_BF16; }
inline bool act_ok(int d) { return d == QMOE_F16 || d == QMOE_BF16; }

int launched() {
  return hipGetLastError() == hipSuccess ? QMOE_OK : QMOE_ERR_LAUNCH;
}

// Shared validation of a weight descriptor.  need_k64: matmul entry points
// stage k in 64-wide tiles.  Any row count n is accepted: the splitter pads
// the stacked rows to a multiple of 16 and the kernels mask the tail rows
// (FP8 keeps its 128-row scale blocks).
int check_weights(const qmoe_weights* w, bool need_k64) {
  if (!w) return QMOE_ERR_ARG;
  if (w->n_experts < 1 || w->n < 1 || w->k < 1) return QMOE_ERR_ARG;
  if (w->n_experts > QMOE_MAX_EXPERTS) return QMOE_ERR_LIMIT;
  if (w->n > (1ll << 30) || w->k > (1ll << 24)) return QMOE_ERR_LIMIT;
  if (need_k64 && w->k % 64) return QMOE_ERR_BLOCK;
  if (!w->qs || !al16(w->qs)) return w->qs ? QMOE_ERR_ALIGN : QMOE_ERR_ARG;
  switch (w->fmt) {
    case QMOE_Q8_0:
      if (w->k % 64) return QMOE_ERR_BLOCK;
      if (!w->scales) return QMOE_ERR_ARG;
      if (!al16(w->scales)) return QMOE_ERR_ALIGN;
      break;
    case QMOE_Q2_K:
      if (w->k % 256) return QMOE_ERR_BLOCK;
      if (!w->scales || !w->d || !w->dmin) return QMOE_ERR_ARG;
      if (!al16(w->scales) || !al16(w->d) || !al16(w->dmin)) return QMOE_ERR_ALIGN;
      break;
    case QMOE_Q4_K:
      if (w->k % 256) return QMOE_ERR_BLOCK;
      if (!w->scales || !w->d || !w->dmin) return QMOE_ERR_ARG;
      if (!al16(w->scales) || !al16(w->d) || !al16(w->dmin)) return QMOE_ERR_ALIGN;
      break;
    case QMOE_Q6_K:
      if (w->k % 256) return QMOE_ERR_BLOCK;
      if (!w->aux || !w->scales || !w->d) return QMOE_ERR_ARG;
      if (!al16(w->aux) || !al16(w->scales) || !al16(w->d)) return QMOE_ERR_ALIGN;
      break;
    case QMOE_IQ2_XXS:
      if (w->k % 256) return QMOE_ERR_BLOCK;
      if (!w->d || !w->grid || !w->signs) return QMOE_ERR_ARG;
      if (!al16(w->d) || !al16(w->grid) || !al16(w->signs)) return QMOE_ERR_ALIGN;
      break;
    case QMOE_MXFP4:
      if (w->k % 64) return QMOE_ERR_BLOCK;
      if (!w->scales) return QMOE_ERR_ARG;
      if (!al16(w->scales)) return QMOE_ERR_ALIGN;
      break;
    case QMOE_FP8:
      // one scale per 128 x 128 block: scale rows follow expert * n / 128 + row / 128
      if (w->k % 128 || w->n % 128) return QMOE_ERR_BLOCK;
      if (!w->scales) return QMOE_ERR_ARG;
      if (!al16(w->scales)) return QMOE_ERR_ALIGN;
      break;
    case QMOE_INT4:
      if (!(w->group == 32 || w->group == 64 || w->group == 128 || w->group == 256)) return QMOE_ERR_BLOCK;
      if (w->k % w->group || w->k % 64) return QMOE_ERR_BLOCK;
      if (!w->scales) return QMOE_ERR_ARG;
      if (!al16(w->scales)) return QMOE_ERR_ALIGN;
      break;
    default:
      return QMOE_ERR_UNSUPPORTED;
  }
  return QMOE_OK;
}

}  // namespace

#define QMOE_TRY(expr)            \
  do {                            \
    const int _st = (expr);       \
    if (_st != QMOE_OK) return _st; \
  } while (0)

extern "C" {

int qmoe_check_device(void) { return check_arch(); }

const char* qmoe_strerror(int status) {
  switch (status) {
    case QMOE_OK: return "ok";
    case QMOE_ERR_ARG: return "invalid argument (NULL pointer, negative size or bad enum)";
    case QMOE_ERR_UNSUPPORTED: return "unsupported format / dtype / epilogue combination";
    case QMOE_ERR_BLOCK: return "size is not a multiple of the format block";
    case QMOE_ERR_LIMIT: return "size limit exceeded (topk, experts, batch or dimension)";
    case QMOE_ERR_WORKSPACE: return "plan or workspace buffer too small";
    case QMOE_ERR_ALIGN: return "pointer not aligned as required";
    case QMOE_ERR_ARCH: return "current HIP device is not gfx950";
    case QMOE_ERR_LAUNCH: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

// ------------------------------------------------------------------ dequant

int qmoe_dequant_q8_0(const int8_t* qs, const uint16_t* d, int64_t rows, int64_t k, void* out, int32_t out_dtype,
                      void* stream) {
  if (!qs || !d || !out || rows < 0 || k < 0 || !dtype_ok(out_dtype)) return QMOE_ERR_ARG;
  if (k % 64) return QMOE_ERR_BLOCK;
  if (!al16(qs) || !al16(d) || !al16(out)) return QMOE_ERR_ALIGN;
  if (rows == 0 || k == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  launch_dequant_q8_0(qs, d, rows, k, out, out_dtype, (hipStream_t)stream);
  return launched();
}

int qmoe_dequant_mxfp4(const uint32_t* qs, const uint8_t* e, int64_t rows, int64_t k, void* out,
                       int32_t out_dtype, void* stream) {
  if (!qs || !e || !out || rows < 0 || k < 0 || !dtype_ok(out_dtype)) return QMOE_ERR_ARG;
  if (k % 64) return QMOE_ERR_BLOCK;
  if (!al16(qs) || !al16(e) || !al16(out)) return QMOE_ERR_ALIGN;
  if (rows == 0 || k == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  launch_dequant_mxfp4(qs, e, rows, k, out, out_dtype, (hipStream_t)stream);
  return launched();
}

int qmoe_dequant_fp8(const uint8_t* qs, const float* scales, int64_t rows, int64_t k, void* out,
                     int32_t out_dtype, void* stream) {
  if (!qs || !scales || !out || rows < 0 || k < 0 || !dtype_ok(out_dtype)) return QMOE_ERR_ARG;
  if (rows % 128 || k % 128) return QMOE_ERR_BLOCK;
  if (!al16(qs) || !al16(scales) || !al16(out)) return QMOE_ERR_ALIGN;
  if (rows == 0 || k == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  launch_dequant_fp8(qs, scales, rows, k, out, out_dtype, (hipStream_t)stream);
  return launched();
}

int qmoe_dequant_q2_k(const uint32_t* qs, const uint8_t* scales, const uint16_t* d,
                      const uint16_t* dmin, int64_t rows, int64_t k, void* out, int32_t out_dtype,
                      void* stream) {
  if (!qs || !scales || !d || !dmin || !out || rows < 0 || k < 0 || !dtype_ok(out_dtype)) return QMOE_ERR_ARG;
  if (k % 256) return QMOE_ERR_BLOCK;
  if (!al16(qs) || !al16(scales) || !al16(d) || !al16(dmin) || !al16(out)) return QMOE_ERR_ALIGN;
  if (rows == 0 || k == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  launch_dequant_q2_k(qs, scales, d, dmin, rows, k, out, out_dtype, (hipStream_t)stream);
  return launched();
}
int qmoe_dequant_q4_k(const uint8_t* qs, const uint8_t* scales, const uint16_t* d, const uint16_t* dmin,
                      int64_t rows, int64_t k, void* out, int32_t out_dtype, void* stream) {
  if (!qs || !scales || !d || !dmin || !out || rows < 0 || k < 0 || !dtype_ok(out_dtype)) return QMOE_ERR_ARG;
  if (k % 256) return QMOE_ERR_BLOCK;
  if (!al16(qs) || !al16(scales) || !al16(d) || !al16(dmin) || !al16(out)) return QMOE_ERR_ALIGN;
  if (rows == 0 || k == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  launch_dequant_q4_k(qs, scales, d, dmin, rows, k, out, out_dtype, (hipStream_t)stream);
  return launched();
}

int qmoe_dequant_q6_k(const uint8_t* qs, const uint8_t* qh, const int8_t* scales, const uint16_t* d,
                      int64_t rows, int64_t k, void* out, int32_t out_dtype, void* stream) {
  if (!qs || !qh || !scales || !d || !out || rows < 0 || k < 0 || !dtype_ok(out_dtype)) return QMOE_ERR_ARG;
  if (k % 256) return QMOE_ERR_BLOCK;
  if (!al16(qs) || !al16(qh) || !al16(scales) || !al16(d) || !al16(out)) return QMOE_ERR_ALIGN;
  if (rows == 0 || k == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  launch_dequant_q6_k(qs, qh, scales, d, rows, k, out, out_dtype, (hipStream_t)stream);
  return launched();
}

int qmoe_dequant_iq2_xxs(const uint32_t* qs, const uint16_t* d, const uint8_t* grid, const uint8_t* signs,
                         int64_t rows, int64_t k, void* out, int32_t out_dtype, void* stream) {
  if (!qs || !d || !grid || !signs || !out || rows < 0 || k < 0 || !dtype_ok(out_dtype)) return QMOE_ERR_ARG;
  if (k % 256) return QMOE_ERR_BLOCK;
  if (!al16(qs) || !al16(d) || !al16(grid) || !al16(signs) || !al16(out)) return QMOE_ERR_ALIGN;
  if (rows == 0 || k == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  launch_dequant_iq2_xxs(qs, d, grid, signs, rows, k, out, out_dtype, (hipStream_t)stream);
  return launched();
}

int qmoe_dequant_int4(const uint32_t* qs, const uint32_t* sb, int64_t rows, int64_t k, int32_t group,
                      void* out, int32_t out_dtype, void* stream) {
  if (!qs || !sb || !out || rows < 0 || k < 0 || !dtype_ok(out_dtype)) return QMOE_ERR_ARG;
  if (!(group == 32 || group == 64 || group == 128 || group == 256) || k % group) return QMOE_ERR_BLOCK;
  if (k % 64) return QMOE_ERR_BLOCK;
  if (!al16(qs) || !al16(sb) || !al16(out)) return QMOE_ERR_ALIGN;
  if (rows == 0 || k == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  launch_dequant_int4(qs, sb, rows, k, group, out, out_dtype, (hipStream_t)stream);
  return launched();
}

// ------------------------------------------------------------------ dense qmm

int qmoe_qmm_dense(const qmoe_weights* w, const void* x, int32_t act_dtype, int64_t m,
                   int32_t epilogue, void* out, int32_t out_dtype, void* stream) {
  QMOE_TRY(check_weights(w, true));
  if (!x || !out || m < 0 || !act_ok(act_dtype) || !dtype_ok(out_dtype)) return QMOE_ERR_ARG;
  if (w->n_experts != 1) return QMOE_ERR_ARG;
  if (epilogue == QMOE_EPI_SWIGLU) {
    if (w->n % 2) return QMOE_ERR_ARG;
  } else if (epilogue == QMOE_EPI_ACCUMULATE) {
    if (out_dtype != QMOE_F32) return QMOE_ERR_UNSUPPORTED;
  } else if (epilogue != QMOE_EPI_STORE) {
    return QMOE_ERR_UNSUPPORTED;
  }
  if (act_dtype == QMOE_BF16 && w->fmt == QMOE_INT4 && w->group % 64) return QMOE_ERR_UNSUPPORTED;
  if (act_dtype == QMOE_BF16 && w->fmt == QMOE_INT4 && w->k / w->group > qmm_int4_bf16_max_groups())
    return QMOE_ERR_LIMIT;
  if (!al16(x) || !al16(out)) return QMOE_ERR_ALIGN;
  if (m * w->k * 2 >= (1ll << 31)) return QMOE_ERR_LIMIT;  // 32-bit activation byte offsets
  if (m == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  launch_qmm(w, x, act_dtype, 2 /*dense*/, nullptr, 0, 1, 128, m, nullptr, epilogue, out, out_dtype,
             (hipStream_t)stream);
  return launched();
}

// ------------------------------------------------------------------ workspace

size_t qmoe_workspace_bytes(int32_t what, const qmoe_weights* w, int64_t t, int32_t topk, int32_t bm) {
  if (!w || t < 0 || topk < 1 || w->n_experts < 1 || w->n < 1) return 0;
  if (what == QMOE_WS_PLAN) return qmoe_plan_bytes(t, topk, w->n_experts, bm);
  if (what == QMOE_WS_COMBINE_ACC) return (size_t)t * (size_t)w->n * sizeof(float);
  return 0;
}

// ------------------------------------------------------------------ plan

size_t qmoe_plan_bytes(int64_t t, int32_t topk, int32_t n_experts, int32_t bm) {
  (void)bm;
  if (t < 0 || topk < 1 || n_experts < 1) return 0;
  const int64_t P = t * topk;
  return (size_t)plan_words(P, n_experts) * sizeof(int32_t);
}

// Tile heights the plan and the gathered matmul accept: a multiple of 16 up
// to the matmul's register tile (80 rows).
static bool bm_ok(int bm) { return bm >= 16 && bm <= 128 && bm % 16 == 0; }
static bool bm_fits(int bm) { return bm <= qmm_max_rows(); }

int qmoe_moe_plan(const int32_t* ids, int64_t t, int32_t topk, int32_t n_experts, int32_t bm,
                  int32_t* plan, size_t plan_bytes, void* stream) {
  if (!ids || !plan || t < 0 || topk < 1 || n_experts < 1) return QMOE_ERR_ARG;
  if (topk > QMOE_MAX_TOPK || n_experts > QMOE_MAX_EXPERTS) return QMOE_ERR_LIMIT;
  if (t * topk > (1ll << 30)) return QMOE_ERR_LIMIT;
  if (!bm_ok(bm)) return QMOE_ERR_ARG;
  if (!bm_fits(bm)) return QMOE_ERR_UNSUPPORTED;
  if (!al4(ids) || !al16(plan)) return QMOE_ERR_ALIGN;
  if (plan_bytes < qmoe_plan_bytes(t, topk, n_experts, bm)) return QMOE_ERR_WORKSPACE;
  QMOE_TRY(check_arch());
  if (t == 0) return QMOE_OK;
  launch_plan(ids, t, topk, n_experts, bm, plan, (hipStream_t)stream);
  return launched();
}

// ------------------------------------------------------------------ gathered MoE qmm

// Argument checks of the gathered matmul (shared by the no-allocation variant).
static int gather_checks(const qmoe_weights* w, const int32_t* plan, int64_t t, int32_t topk, int32_t bm,
                         const void* a, int32_t act_dtype, int32_t a_mode, const float* topk_w,
                         int32_t epilogue, const void* out, int32_t out_dtype) {
  QMOE_TRY(check_weights(w, true));
  if (!plan || !a || !out || t < 0 || topk < 1 || !act_ok(act_dtype) || !dtype_ok(out_dtype))
    return QMOE_ERR_ARG;
  if (topk > QMOE_MAX_TOPK) return QMOE_ERR_LIMIT;
  if (t * topk > (1ll << 30)) return QMOE_ERR_LIMIT;
  if (!bm_ok(bm)) return QMOE_ERR_ARG;
  if (a_mode != QMOE_A_GATHER_TOKENS && a_mode != QMOE_A_SORTED_ROWS) return QMOE_ERR_ARG;
  if (epilogue == QMOE_EPI_SWIGLU) {
    if (w->n % 2) return QMOE_ERR_ARG;
  } else if (epilogue == QMOE_EPI_WEIGHTED_COMBINE) {
    if (!topk_w) return QMOE_ERR_ARG;
    if (out_dtype != QMOE_F32) return QMOE_ERR_UNSUPPORTED;
    if (!al4(topk_w)) return QMOE_ERR_ALIGN;
  } else if (epilogue != QMOE_EPI_STORE) {
    return QMOE_ERR_UNSUPPORTED;
  }
  if (act_dtype == QMOE_BF16 && w->fmt == QMOE_INT4 && w->group % 64) return QMOE_ERR_UNSUPPORTED;
  if (act_dtype == QMOE_BF16 && w->fmt == QMOE_INT4 && w->k / w->group > qmm_int4_bf16_max_groups())
    return QMOE_ERR_LIMIT;
  if (!bm_fits(bm)) return QMOE_ERR_UNSUPPORTED;
  // activation rows are addressed with 32-bit byte offsets
  if ((a_mode == QMOE_A_GATHER_TOKENS ? t : t * topk) * w->k * 2 >= (1ll << 31)) return QMOE_ERR_LIMIT;
  if (!al16(plan) || !al16(a) || !al16(out)) return QMOE_ERR_ALIGN;
  return QMOE_OK;
}

int qmoe_moe_gather_qmm(const qmoe_weights* w, const int32_t* plan, int64_t t, int32_t topk,
                        int32_t bm, const void* a, int32_t act_dtype, int32_t a_mode,
                        const float* topk_w, int32_t epilogue, void* out, int32_t out_dtype,
                        void* stream) {
  QMOE_TRY(gather_checks(w, plan, t, topk, bm, a, act_dtype, a_mode, topk_w, epilogue, out, out_dtype));
  if (t == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  launch_qmm(w, a, act_dtype, a_mode == QMOE_A_GATHER_TOKENS ? 0 : 1, plan, t, topk, bm, 0, topk_w,
             epilogue, out, out_dtype, (hipStream_t)stream);
  return launched();
}

static int combine_checks(const void* y, int32_t y_dtype, const int32_t* plan, int64_t t, int32_t topk,
                          int32_t n_experts, const float* topk_w, int64_t n, const float* base,
                          const void* out, int32_t out_dtype) {
  if (!y || !plan || !topk_w || !out || t < 0 || n < 0 || topk < 1 || n_experts < 1) return QMOE_ERR_ARG;
  if (!dtype_ok(y_dtype) || !dtype_ok(out_dtype)) return QMOE_ERR_ARG;
  if (topk > QMOE_MAX_TOPK || n_experts > QMOE_MAX_EXPERTS) return QMOE_ERR_LIMIT;
  if (t * topk > (1ll << 30) || ((n + 255) / 256) * t > (1ll << 31) - 1) return QMOE_ERR_LIMIT;
  if (!al16(y) || !al16(plan) || !al4(topk_w) || !al16(out) || (base && !al4(base))) return QMOE_ERR_ALIGN;
  return QMOE_OK;
}

int qmoe_moe_combine(const void* y, int32_t y_dtype, const int32_t* plan, int64_t t, int32_t topk,
                     int32_t n_experts, const float* topk_w, int64_t n, const float* base, void* out,
                     int32_t out_dtype, void* stream) {
  QMOE_TRY(combine_checks(y, y_dtype, plan, t, topk, n_experts, topk_w, n, base, out, out_dtype));
  if (t == 0 || n == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  launch_moe_combine(y, y_dtype, plan, t, topk, n_experts, topk_w, n, base, nullptr, nullptr, QMOE_F32, out,
                     out_dtype, (hipStream_t)stream);
  return launched();
}

int qmoe_moe_combine_shared(const void* y, int32_t y_dtype, const int32_t* plan, int64_t t, int32_t topk,
                            int32_t n_experts, const float* topk_w, int64_t n, const float* shared,
                            const float* shared_gate, const void* residual, int32_t residual_dtype,
                            void* out, int32_t out_dtype, void* stream) {
  QMOE_TRY(combine_checks(y, y_dtype, plan, t, topk, n_experts, topk_w, n, shared, out, out_dtype));
  if (shared_gate && !shared) return QMOE_ERR_ARG;
  if (residual && !dtype_ok(residual_dtype)) return QMOE_ERR_ARG;
  if ((shared_gate && !al4(shared_gate)) || (residual && !al16(residual))) return QMOE_ERR_ALIGN;
  // out may be the residual buffer itself (same dtype), any other overlap is an error
  if (residual && residual != out) {
    const int64_t rb = t * n * (residual_dtype == QMOE_F32 ? 4 : 2);
    const int64_t ob = t * n * (out_dtype == QMOE_F32 ? 4 : 2);
    const uintptr_t r0 = (uintptr_t)residual, o0 = (uintptr_t)out;
    if (r0 < o0 + ob && o0 < r0 + rb) return QMOE_ERR_ARG;
  }
  if (residual && residual == out && residual_dtype != out_dtype) return QMOE_ERR_ARG;
  if (t == 0 || n == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  launch_moe_combine(y, y_dtype, plan, t, topk, n_experts, topk_w, n, shared, shared_gate, residual,
                     residual ? residual_dtype : QMOE_F32, out, out_dtype, (hipStream_t)stream);
  return launched();
}

int qmoe_combine_cast(float* acc, int64_t n_elems, void* out, int32_t out_dtype, void* stream) {
  if (!acc || !out || n_elems < 0 || !dtype_ok(out_dtype)) return QMOE_ERR_ARG;
  if (!al16(acc) || !al16(out)) return QMOE_ERR_ALIGN;
  if (n_elems == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  launch_combine_cast(acc, n_elems, out, out_dtype, (hipStream_t)stream);
  return launched();
}

// ------------------------------------------------------------------ no-allocation variant
//
// The WEIGHTED_COMBINE gathered matmul plus the cast, with its fp32
// accumulator in a fixed device array instead of a caller buffer, for
// callers that cannot allocate (code under graph capture, tight serving
// loops).  Every call on a device shares that device's copy of the array.

}  // extern "C"

namespace {

constexpr size_t kStaticAccBytes = size_t(32) << 20;  // 32 MiB: t * n <= 8M fp32 values

static __device__ __align__(256) float scratch[kStaticAccBytes / sizeof(float)];

std::atomic<float*> g_scratch[kMaxDevices];

// The current device's address of `scratch`, looked up once per device with
// that device current (each GPU holds its own copy at its own address).  The
// array's name is only a host stand-in and is never passed to a kernel.
int scratch_ptr(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QMOE_ERR_ARCH;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return QMOE_ERR_LAUNCH;
    p = (float*)q;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return QMOE_OK;
}

// Zero n floats (a kernel rather than a memset, so the call can be captured).
__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, int64_t n) {
  const int64_t n4 = n / 4;
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    ((f4_t*)p)[i] = f4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t tail = n4 * 4 + blockIdx.x * 256ll + threadIdx.x;
  if (blockIdx.x == 0 && tail < n) p[tail] = 0.f;
}

}  // namespace

extern "C" {

int qmoe_moe_gather_qmm_combine_static(const qmoe_weights* w, const int32_t* plan, int64_t t, int32_t topk,
                                       int32_t bm, const void* a, int32_t act_dtype, int32_t a_mode,
                                       const float* topk_w, void* out, int32_t out_dtype, void* stream) {
  QMOE_TRY(gather_checks(w, plan, t, topk, bm, a, act_dtype, a_mode, topk_w, QMOE_EPI_WEIGHTED_COMBINE, out,
                         QMOE_F32));
  if (!dtype_ok(out_dtype)) return QMOE_ERR_ARG;
  if ((size_t)t * (size_t)w->n * sizeof(float) > kStaticAccBytes) return QMOE_ERR_WORKSPACE;
  if (t == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  float* acc = nullptr;
  QMOE_TRY(scratch_ptr(&acc));
  const int64_t n = t * w->n;
  const hipStream_t s = (hipStream_t)stream;
  int64_t grid = (n / 4 + 255) / 256;
  grid = grid < 1 ? 1 : (grid > 4096 ? 4096 : grid);
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)grid), dim3(256), 0, s, acc, n);
  launch_qmm(w, a, act_dtype, a_mode == QMOE_A_GATHER_TOKENS ? 0 : 1, plan, t, topk, bm, 0, topk_w,
             QMOE_EPI_WEIGHTED_COMBINE, acc, QMOE_F32, s);
  launch_combine_cast(acc, n, out, out_dtype, s);
  return launched();
}

size_t qmoe_static_acc_bytes(void) { return kStaticAccBytes; }

// ------------------------------------------------------------------ router top-k

int qmoe_router_topk(const void* logits, int32_t logits_dtype, int64_t t, int32_t n_experts,
                     int32_t topk, int32_t scoring, const float* bias, float scale,
                     int32_t* ids, float* weights, void* stream) {
  if (!logits || !ids || !weights || t < 0 || topk < 1 || n_experts < 1 || !dtype_ok(logits_dtype))
    return QMOE_ERR_ARG;
  if (scoring != QMOE_ROUTER_SOFTMAX && scoring != QMOE_ROUTER_SQRTSOFTPLUS) return QMOE_ERR_ARG;
  if (scoring == QMOE_ROUTER_SOFTMAX && scale != 1.0f) return QMOE_ERR_ARG;
  if (topk > QMOE_MAX_TOPK || n_experts > QMOE_MAX_EXPERTS || t > (1ll << 31)) return QMOE_ERR_LIMIT;
  if (topk > n_experts) return QMOE_ERR_ARG;
  const uintptr_t esz = logits_dtype == QMOE_F32 ? 4 : 2;
  if ((uintptr_t)logits % esz || !al4(ids) || !al4(weights) || (bias && !al4(bias)))
    return QMOE_ERR_ALIGN;
  if (t == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  launch_router_topk(logits, logits_dtype, t, n_experts, topk, scoring, bias, scale, ids, weights,
                     (hipStream_t)stream);
  return launched();
}

// ------------------------------------------------------------------ decode GEMV

int qmoe_moe_gemv(const qmoe_weights* w, const void* a, int32_t act_dtype, int64_t b,
                  const int32_t* ids, const float* topk_w, int32_t topk, int32_t epilogue,
                  void* out, int32_t out_dtype, void* stream) {
  QMOE_TRY(check_weights(w, false));
  if (!a || !ids || !out || b < 0 || topk < 1 || !act_ok(act_dtype) || !dtype_ok(out_dtype))
    return QMOE_ERR_ARG;
  if (topk > QMOE_MAX_TOPK || b > QMOE_MAX_GEMV_BATCH) return QMOE_ERR_LIMIT;
  if (w->k % 32) return QMOE_ERR_BLOCK;
  if (w->k > gemv_max_k()) return QMOE_ERR_LIMIT;
  if (epilogue == QMOE_EPI_SWIGLU) {
    if (w->n % 2) return QMOE_ERR_ARG;
  } else if (epilogue == QMOE_EPI_WEIGHTED_COMBINE) {
    if (!topk_w) return QMOE_ERR_ARG;
    if (!al4(topk_w)) return QMOE_ERR_ALIGN;
    if (w->n > (1ll << 31) / 64) return QMOE_ERR_LIMIT;
  } else if (epilogue != QMOE_EPI_STORE) {
    return QMOE_ERR_UNSUPPORTED;
  }
  if (!al16(a) || !al4(ids) || !al16(out)) return QMOE_ERR_ALIGN;
  if (b == 0) return QMOE_OK;
  QMOE_TRY(check_arch());
  QMOE_TRY(launch_gemv(w, a, act_dtype, b, ids, topk_w, topk, epilogue, out, out_dtype, (hipStream_t)stream));
  return launched();
}

}  // extern "C"
