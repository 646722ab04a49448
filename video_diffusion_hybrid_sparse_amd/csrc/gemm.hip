// Output projections of both branches plus the residual, as one GEMM.
//
// Each branch has its own output projection and both add into the residual stream
// (VDN-MiniMax-H3 article, modelscope.csdn.net, section "独立门控，融合两条注意力分支").
// With the branch outputs stored side by side per token, [a_s | a_l] (N x 2Hd), and the
// weights side by side per output row, [W_s | W_l] (D x 2Hd):
//     out = x + a_s W_s^T + a_l W_l^T = x + [a_s | a_l] [W_s | W_l]^T,
// a plain GEMM with K = 2Hd and beta = 1 on the residual.  It runs on hipBLASLt.
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "gemm.h"

namespace vdn {

namespace {

struct Plan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo;
  size_t ws = 0;
};

std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;
std::map<std::tuple<int, int, int64_t, int64_t, int64_t, size_t>, Plan> g_plans;
std::map<std::tuple<int, int, int, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, size_t>, Plan> g_gplans;

int get_handle(int dev, hipblasLtHandle_t* handle, const char** err) {
  auto hit = g_handles.find(dev);
  if (hit != g_handles.end()) {
    *handle = hit->second;
    return 0;
  }
  if (hipblasLtCreate(handle) != HIPBLAS_STATUS_SUCCESS) { *err = "hipblasLtCreate failed"; return -1; }
  g_handles[dev] = *handle;
  return 0;
}

}  // namespace

int projection_gemm(bool bf16, int64_t n_tokens, int64_t d_model, int64_t k2, const void* a_cat,
                    const void* w_cat, const void* residual, void* out, void* ws, size_t ws_bytes,
                    hipStream_t stream, const char** err) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) { *err = "hipGetDevice failed"; return -1; }
  std::lock_guard<std::mutex> lock(g_mu);
  hipblasLtHandle_t handle;
  auto hit = g_handles.find(dev);
  if (hit == g_handles.end()) {
    if (hipblasLtCreate(&handle) != HIPBLAS_STATUS_SUCCESS) { *err = "hipblasLtCreate failed"; return -1; }
    g_handles[dev] = handle;
  } else {
    handle = hit->second;
  }
  const auto key = std::make_tuple(dev, bf16 ? 1 : 0, n_tokens, d_model, k2, ws_bytes);
  auto pit = g_plans.find(key);
  if (pit == g_plans.end()) {
    Plan p;
    const hipDataType dt = bf16 ? HIP_R_16BF : HIP_R_32F;
    // Column-major view: out^T (D x N) = W_cat^T... with W_cat stored row-major [D, K]
    // = column-major K x D (ld K), a_cat row-major [N, K] = column-major K x N (ld K).
    // op(A) = transpose(W_colmajor) : D x K;  op(B) = a_cat_colmajor : K x N.
    if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) {
      *err = "hipblasLtMatmulDescCreate failed";
      return -1;
    }
    int32_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
    hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT));
    hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN));
    hipblasLtMatrixLayoutCreate(&p.la, dt, k2, d_model, k2);
    hipblasLtMatrixLayoutCreate(&p.lb, dt, k2, n_tokens, k2);
    hipblasLtMatrixLayoutCreate(&p.lc, dt, d_model, n_tokens, d_model);
    hipblasLtMatmulPreference_t pref;
    hipblasLtMatmulPreferenceCreate(&pref);
    uint64_t wsz = ws_bytes;
    hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsz, sizeof(wsz));
    hipblasLtMatmulHeuristicResult_t res[1];
    int nres = 0;
    hipblasStatus_t st = hipblasLtMatmulAlgoGetHeuristic(handle, p.desc, p.la, p.lb, p.lc, p.lc, pref, 1, res, &nres);
    hipblasLtMatmulPreferenceDestroy(pref);
    if (st != HIPBLAS_STATUS_SUCCESS || nres < 1) {
      *err = "hipBLASLt found no algorithm for the projection GEMM";
      return -1;
    }
    p.algo = res[0].algo;
    p.ws = res[0].workspaceSize;
    pit = g_plans.emplace(key, p).first;
  }
  const Plan& p = pit->second;
  const float alpha = 1.0f, beta = 1.0f;
  hipblasStatus_t st = hipblasLtMatmul(handle, p.desc, &alpha, w_cat, p.la, a_cat, p.lb, &beta, residual,
                                       p.lc, out, p.lc, &p.algo, ws, p.ws, stream);
  if (st != HIPBLAS_STATUS_SUCCESS) { *err = "hipblasLtMatmul failed"; return -1; }
  return 0;
}

int gemm_bf16_f32out(bool trans_a, bool trans_b, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda,
                     const void* B, int64_t ldb, float* D, int64_t ldd, void* ws, size_t ws_bytes,
                     hipStream_t stream, const char** err) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) { *err = "hipGetDevice failed"; return -1; }
  std::lock_guard<std::mutex> lock(g_mu);
  hipblasLtHandle_t handle;
  if (get_handle(dev, &handle, err) != 0) return -1;
  const auto key = std::make_tuple(dev, trans_a ? 1 : 0, trans_b ? 1 : 0, m, n, k, lda, ldb, ldd, ws_bytes);
  auto pit = g_gplans.find(key);
  if (pit == g_gplans.end()) {
    Plan p;
    if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) {
      *err = "hipblasLtMatmulDescCreate failed";
      return -1;
    }
    int32_t opa = trans_a ? HIPBLAS_OP_T : HIPBLAS_OP_N, opb = trans_b ? HIPBLAS_OP_T : HIPBLAS_OP_N;
    hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof(opa));
    hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof(opb));
    hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, trans_a ? k : m, trans_a ? m : k, lda);
    hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, trans_b ? n : k, trans_b ? k : n, ldb);
    hipblasLtMatrixLayoutCreate(&p.lc, HIP_R_32F, m, n, ldd);
    hipblasLtMatmulPreference_t pref;
    hipblasLtMatmulPreferenceCreate(&pref);
    uint64_t wsz = ws_bytes;
    hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsz, sizeof(wsz));
    hipblasLtMatmulHeuristicResult_t res[1];
    int nres = 0;
    hipblasStatus_t st = hipblasLtMatmulAlgoGetHeuristic(handle, p.desc, p.la, p.lb, p.lc, p.lc, pref, 1, res, &nres);
    hipblasLtMatmulPreferenceDestroy(pref);
    if (st != HIPBLAS_STATUS_SUCCESS || nres < 1) {
      *err = "hipBLASLt found no algorithm for a backward GEMM";
      return -1;
    }
    p.algo = res[0].algo;
    p.ws = res[0].workspaceSize;
    pit = g_gplans.emplace(key, p).first;
  }
  const Plan& p = pit->second;
  const float alpha = 1.0f, beta = 0.0f;
  hipblasStatus_t st = hipblasLtMatmul(handle, p.desc, &alpha, A, p.la, B, p.lb, &beta, D, p.lc, D, p.lc, &p.algo,
                                       ws, p.ws, stream);
  if (st != HIPBLAS_STATUS_SUCCESS) { *err = "hipblasLtMatmul failed"; return -1; }
  return 0;
}

}  // namespace vdn
