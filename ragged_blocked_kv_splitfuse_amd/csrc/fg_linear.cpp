// Dense projections either side of attention (the QKV projection feeding fg_kv_append and
// the output projection after fg_ragged_attention), as plain bf16 GEMMs through hipBLASLt.
//
// y[T][N] = x[T][K] . w[N][K]^T, row-major.  In hipBLASLt's column-major terms that is
// D (N x T, ld N) = op(A) (N x K) . op(B) (K x T) with A = w stored K x N (ld K, op = T) and
// B = x stored K x T (ld K, op = N).  fp32 accumulation and scale, bf16 output.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cstdint>
#include <map>
#include <mutex>
#include <tuple>

#include "fg_internal.h"

using fgi::fail;

namespace {

constexpr size_t WORKSPACE_BYTES = 32u << 20;
constexpr size_t MAX_PLANS = 4096;  // cached (T, K, N) algorithm choices per device

struct Plan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
  hipblasLtMatmulAlgo_t algo{};
  size_t ws = 0;
};

// One hipBLASLt handle and plan cache per device; one workspace per (device, stream), so that
// GEMMs enqueued on different streams never share scratch memory while they may overlap.
struct DeviceState {
  hipblasLtHandle_t handle = nullptr;
  std::map<void *, void *> workspace;  // stream -> workspace
  std::map<std::tuple<int32_t, int32_t, int32_t>, Plan> plans;
};

std::mutex g_mu;
std::map<int, DeviceState> g_dev;

const char *blas_name(hipblasStatus_t s) {
  switch (s) {
    case HIPBLAS_STATUS_SUCCESS: return "success";
    case HIPBLAS_STATUS_NOT_INITIALIZED: return "not initialized";
    case HIPBLAS_STATUS_ALLOC_FAILED: return "allocation failed";
    case HIPBLAS_STATUS_INVALID_VALUE: return "invalid value";
    case HIPBLAS_STATUS_ARCH_MISMATCH: return "architecture mismatch";
    case HIPBLAS_STATUS_EXECUTION_FAILED: return "execution failed";
    case HIPBLAS_STATUS_NOT_SUPPORTED: return "not supported";
    default: return "error";
  }
}

#define BLAS_TRY(call)                                                            \
  do {                                                                            \
    const hipblasStatus_t s_ = (call);                                            \
    if (s_ != HIPBLAS_STATUS_SUCCESS)                                             \
      return fail(FG_E_HIP, "%s: hipBLASLt %s", #call, blas_name(s_));            \
  } while (0)

void destroy_plan(Plan &p) {
  if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
  if (p.a) hipblasLtMatrixLayoutDestroy(p.a);
  if (p.b) hipblasLtMatrixLayoutDestroy(p.b);
  if (p.d) hipblasLtMatrixLayoutDestroy(p.d);
  p = Plan{};
}

fg_status make_plan_(DeviceState &ds, int32_t T, int32_t K, int32_t N, Plan &p) {
  BLAS_TRY(hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F));
  const int32_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
  BLAS_TRY(hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT,
                                           sizeof(opT)));
  BLAS_TRY(hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN,
                                           sizeof(opN)));
  BLAS_TRY(hipblasLtMatrixLayoutCreate(&p.a, HIP_R_16BF, (uint64_t)K, (uint64_t)N, K));
  BLAS_TRY(hipblasLtMatrixLayoutCreate(&p.b, HIP_R_16BF, (uint64_t)K, (uint64_t)T, K));
  BLAS_TRY(hipblasLtMatrixLayoutCreate(&p.d, HIP_R_16BF, (uint64_t)N, (uint64_t)T, N));
  hipblasLtMatmulPreference_t pref = nullptr;
  BLAS_TRY(hipblasLtMatmulPreferenceCreate(&pref));
  const uint64_t cap = WORKSPACE_BYTES;
  hipblasStatus_t s = hipblasLtMatmulPreferenceSetAttribute(
      pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap, sizeof(cap));
  hipblasLtMatmulHeuristicResult_t res[1];
  int found = 0;
  if (s == HIPBLAS_STATUS_SUCCESS)
    s = hipblasLtMatmulAlgoGetHeuristic(ds.handle, p.desc, p.a, p.b, p.d, p.d, pref, 1, res,
                                        &found);
  hipblasLtMatmulPreferenceDestroy(pref);
  if (s != HIPBLAS_STATUS_SUCCESS) return fail(FG_E_HIP, "hipBLASLt heuristic: %s", blas_name(s));
  if (found < 1 || res[0].state != HIPBLAS_STATUS_SUCCESS)
    return fail(FG_E_UNSUPPORTED, "hipBLASLt has no algorithm for T=%d K=%d N=%d", T, K, N);
  p.algo = res[0].algo;
  p.ws = res[0].workspaceSize;
  return FG_OK;
}

fg_status make_plan(DeviceState &ds, int32_t T, int32_t K, int32_t N, Plan &p) {
  const fg_status st = make_plan_(ds, T, K, N, p);
  if (st != FG_OK) destroy_plan(p);
  return st;
}

}  // namespace

extern "C" fg_status fg_linear_bf16(const void *x, const void *w, void *y, int32_t T, int32_t K,
                                    int32_t N, void *stream) {
  fgi::clear_error();
  if (T < 0 || K < 1 || N < 1) return fail(FG_E_ARG, "sizes T=%d K=%d N=%d", T, K, N);
  if (T == 0) return FG_OK;
  if (!x || !w || !y) return fail(FG_E_ARG, "null x, w or y");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(FG_E_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState &ds = g_dev[dev];
  if (!ds.handle) BLAS_TRY(hipblasLtCreate(&ds.handle));
  void *&ws = ds.workspace[stream];
  if (!ws && hipMalloc(&ws, WORKSPACE_BYTES) != hipSuccess) {
    ws = nullptr;
    ds.workspace.erase(stream);
    return fail(FG_E_HIP, "hipMalloc of the %zu-byte GEMM workspace failed", WORKSPACE_BYTES);
  }
  if (ds.plans.size() >= MAX_PLANS) {  // many distinct token counts: start over
    for (auto &kv : ds.plans) destroy_plan(kv.second);
    ds.plans.clear();
  }
  auto key = std::make_tuple(T, K, N);
  auto it = ds.plans.find(key);
  if (it == ds.plans.end()) {
    Plan p;
    const fg_status st = make_plan(ds, T, K, N, p);
    if (st != FG_OK) return st;
    it = ds.plans.emplace(key, p).first;
  }
  const Plan &p = it->second;
  const float alpha = 1.f, beta = 0.f;
  BLAS_TRY(hipblasLtMatmul(ds.handle, p.desc, &alpha, w, p.a, x, p.b, &beta, y, p.d, y, p.d,
                           &p.algo, ws, WORKSPACE_BYTES, (hipStream_t)stream));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FG_E_HIP, "GEMM launch: %s", hipGetErrorString(e));
  return FG_OK;
}
