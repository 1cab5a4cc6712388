// The output projection for long token counts as a plain library GEMM:
// y[T][N] = a[T][1024] . o[N][1024]^T in bf16 with fp32 accumulation, run by
// hipBLASLt (task page "Whole decoder layer", section "What to compute": the
// gated attention output times o^T).  In column-major terms y^T (N x T) =
// op(A) . B with A = o seen as 1024 x N (transposed by the GEMM) and B = a seen
// as 1024 x T.
//
// One hipBLASLt handle per device, and one plan (descriptors and the
// heuristic's first algorithm, no workspace) per (T, N), both made at the
// first call of a shape and kept: a caller that captures the projection in a
// graph runs each shape once before capturing it.  At most MAX_PLANS shapes
// are kept per device; past that the cache is emptied first.
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <utility>

#include "launch.h"

namespace museattn {
namespace {

constexpr int MAX_PLANS = 64;

struct Plan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo{};
  bool ok = false;   // a usable algorithm was found
};

struct Device {
  hipblasLtHandle_t handle = nullptr;
  bool unusable = false;   // the handle could not be made
  std::map<std::pair<int, int>, Plan> plans;
};

std::mutex g_mutex;
std::map<int, Device> g_devices;

void destroy(Plan &p) {
  if (p.la) hipblasLtMatrixLayoutDestroy(p.la);
  if (p.lb) hipblasLtMatrixLayoutDestroy(p.lb);
  if (p.lc) hipblasLtMatrixLayoutDestroy(p.lc);
  if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
  p = Plan{};
}

Plan make_plan(hipblasLtHandle_t h, int T, int N) {
  constexpr int K = HQ * D;
  Plan p;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  bool good = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) ==
                  HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) ==
                  HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, K, N, K) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, K, T, K) == HIPBLAS_STATUS_SUCCESS &&
              hipblasLtMatrixLayoutCreate(&p.lc, HIP_R_16BF, N, T, N) == HIPBLAS_STATUS_SUCCESS;
  if (good) {
    hipblasLtMatmulPreference_t pref = nullptr;
    if (hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS) {
      const uint64_t ws = 0;   // no workspace: nothing to allocate per call
      hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws,
                                            sizeof(ws));
      hipblasLtMatmulHeuristicResult_t res[1];
      int n = 0;
      if (hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.la, p.lb, p.lc, p.lc, pref, 1, res, &n) ==
              HIPBLAS_STATUS_SUCCESS &&
          n > 0 && res[0].state == HIPBLAS_STATUS_SUCCESS && res[0].workspaceSize == 0) {
        p.algo = res[0].algo;
        p.ok = true;
      }
      hipblasLtMatmulPreferenceDestroy(pref);
    }
  }
  if (!p.ok) destroy(p);
  return p;
}

}  // namespace

bool gemm_oproj(const uint16_t *a, const uint16_t *o, uint16_t *y, int T, int N, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lock(g_mutex);
  Device &d = g_devices[dev];
  if (d.unusable) return false;
  if (!d.handle && hipblasLtCreate(&d.handle) != HIPBLAS_STATUS_SUCCESS) {
    d.handle = nullptr;
    d.unusable = true;
    return false;
  }
  const auto key = std::make_pair(T, N);
  auto it = d.plans.find(key);
  if (it == d.plans.end()) {
    if ((int)d.plans.size() >= MAX_PLANS) {
      for (auto &kv : d.plans) destroy(kv.second);
      d.plans.clear();
    }
    it = d.plans.emplace(key, make_plan(d.handle, T, N)).first;
  }
  const Plan &p = it->second;
  if (!p.ok) return false;
  const float alpha = 1.0f, beta = 0.0f;
  return hipblasLtMatmul(d.handle, p.desc, &alpha, o, p.la, a, p.lb, &beta, y, p.lc, y, p.lc,
                         &p.algo, nullptr, 0, stream) == HIPBLAS_STATUS_SUCCESS;
}

}  // namespace museattn
