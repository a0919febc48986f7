// Plain (unfused) GEMMs through hipBLASLt, the vendor GEMM library.
//
// The prefill projections (x W_DQ, x W_DKV, c_q W_UQ, K_nope = C W_UK^T) and
// the W_O projection have no epilogue of their own, so they are library
// GEMMs: on MI355X hipBLASLt runs these shapes 15-45 % faster than the
// hand-written tile kernel (gemm_tile256.hip), which stays the path for
// everything hipBLASLt does not take (batched and blocked operands, fused
// epilogues, small shapes) and the fallback whenever the library reports an
// error.  MLA_GEMM=tile in the environment forces the tile kernel.
//
// One handle and one 32 MiB workspace per device, created on first use (not
// while the stream is being captured into a graph: a GEMM met first inside a
// capture takes the tile kernel).  The algorithm for a shape comes from the
// library's heuristic, asked once per shape.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "launch.h"

namespace mla {
namespace {

constexpr size_t kWsBytes = 32u << 20;

struct Plan {
  bool ok = false;
  hipblasLtMatmulDesc_t op{};
  hipblasLtMatrixLayout_t la{}, lb{}, lc{};
  hipblasLtMatmulAlgo_t algo{};
  size_t ws = 0;
};

struct Device {
  bool tried = false;
  hipblasLtHandle_t handle = nullptr;
  void* ws = nullptr;
  std::map<std::tuple<int, int, int, long, long, long, bool, bool>, Plan> plans;
};

std::mutex g_mu;
Device g_dev[64];

bool forced_off() {
  const char* e = std::getenv("MLA_GEMM");
  return e && std::strcmp(e, "tile") == 0;
}

// The device's handle and workspace, or null (creation failed, or it would
// have to allocate during a graph capture).
Device* device(hipStream_t st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  Device& d = g_dev[dev];
  if (d.handle) return &d;
  if (d.tried) return nullptr;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return nullptr;
  d.tried = true;
  if (hipblasLtCreate(&d.handle) != HIPBLAS_STATUS_SUCCESS) {
    d.handle = nullptr;
    return nullptr;
  }
  if (hipMalloc(&d.ws, kWsBytes) != hipSuccess) {
    hipblasLtDestroy(d.handle);
    d.handle = nullptr;
    d.ws = nullptr;
    return nullptr;
  }
  return &d;
}

// Row-major C [M, N] = alpha A [M, K] B, B row-major [K, N] (or given as Bt
// [N, K]).  In hipBLASLt's column-major terms that is C^T = B^T A^T: the
// library's A is our B (N x K; stored K x N and transposed when B comes
// transposed), its B is our A (K x M, ld = lda), its D is C^T (N x M).
Plan make_plan(hipblasLtHandle_t h, int M, int N, int K, long lda, long ldb, long ldc, bool c_f32,
               bool bt) {
  Plan p;
  if (hipblasLtMatmulDescCreate(&p.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS)
    return p;
  const hipblasOperation_t ta = bt ? HIPBLAS_OP_T : HIPBLAS_OP_N, tb = HIPBLAS_OP_N;
  bool ok =
      hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) ==
          HIPBLAS_STATUS_SUCCESS &&
      hipblasLtMatmulDescSetAttribute(p.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) ==
          HIPBLAS_STATUS_SUCCESS;
  ok = ok &&
       (bt ? hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, K, N, ldb)
           : hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, N, K, ldb)) == HIPBLAS_STATUS_SUCCESS &&
       hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, K, M, lda) == HIPBLAS_STATUS_SUCCESS &&
       hipblasLtMatrixLayoutCreate(&p.lc, c_f32 ? HIP_R_32F : HIP_R_16BF, N, M, ldc) ==
           HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulPreference_t pref = nullptr;
  ok = ok && hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
  uint64_t ws = kWsBytes;
  ok = ok && hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                   &ws, sizeof(ws)) == HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulHeuristicResult_t res{};
  int n = 0;
  ok = ok && hipblasLtMatmulAlgoGetHeuristic(h, p.op, p.la, p.lb, p.lc, p.lc, pref, 1, &res, &n) ==
                 HIPBLAS_STATUS_SUCCESS &&
       n > 0 && res.workspaceSize <= kWsBytes;
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (ok) {
    p.algo = res.algo;
    p.ws = res.workspaceSize;
    p.ok = true;
  }
  return p;
}

}  // namespace

bool blas_gemm_bf16(const void* A, const void* B, void* C, int M, int N, int K, long lda, long ldb,
                    long ldc, float alpha, bool c_f32, bool b_transposed, hipStream_t st) {
  if (forced_off() || M < 256 || N < 128 || K < 32) return false;
  std::lock_guard<std::mutex> lock(g_mu);
  Device* d = device(st);
  if (!d) return false;
  const auto key = std::make_tuple(M, N, K, lda, ldb, ldc, c_f32, b_transposed);
  auto it = d->plans.find(key);
  if (it == d->plans.end())
    it = d->plans.emplace(key, make_plan(d->handle, M, N, K, lda, ldb, ldc, c_f32, b_transposed))
             .first;
  const Plan& p = it->second;
  if (!p.ok) return false;
  const float beta = 0.f;
  return hipblasLtMatmul(d->handle, p.op, &alpha, B, p.la, A, p.lb, &beta, C, p.lc, C, p.lc,
                         &p.algo, d->ws, p.ws, st) == HIPBLAS_STATUS_SUCCESS;
}

}  // namespace mla
