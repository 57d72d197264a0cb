// block_gemm.cpp -- the two projections around the anchor attention in an attention block
// (plain GEMMs, run by hipBLASLt): D[T, N] = X[T, K] W[K, N] + bias[N], all row-major bf16
// with fp32 accumulation.
//
// hipBLASLt is column-major: a row-major [R, C] matrix is the column-major [C, R] matrix
// with leading dimension C, so D^T[N, T] = W^T[N, K] X^T[K, T] is computed with no
// transposes (A = W's memory as N x K, B = X's memory as K x T), and the bias (length N =
// rows of D^T) is broadcast over the T columns by the BIAS epilogue.  Of hipBLASLt's first
// eight heuristic candidates for a shape, the fastest measured on the first call is kept
// (at the ViT-S/16 block shapes the first candidate ran at about 0.28 PFLOP/s).
#include <hipblaslt/hipblaslt.h>

#include <new>
#include <vector>

#include "kernels.h"

namespace aa {

namespace {

constexpr int kMaxCandidates = 8;

struct GemmEntry {
  long long T;
  int K, N;
  bool bias;
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulAlgo_t algo[kMaxCandidates]{};
  int candidates = 0;
  int best = 0;
  bool timed = false;
};

}  // namespace

struct GemmCache {
  hipblasLtHandle_t handle = nullptr;
  std::vector<GemmEntry> entries;
};

GemmCache* gemm_cache_create() {
  GemmCache* c = new (std::nothrow) GemmCache;
  if (!c) return nullptr;
  if (hipblasLtCreate(&c->handle) != HIPBLAS_STATUS_SUCCESS) {
    delete c;
    return nullptr;
  }
  return c;
}

void gemm_cache_destroy(GemmCache* c) {
  if (!c) return;
  for (GemmEntry& e : c->entries) {
    if (e.desc) hipblasLtMatmulDescDestroy(e.desc);
    if (e.la) hipblasLtMatrixLayoutDestroy(e.la);
    if (e.lb) hipblasLtMatrixLayoutDestroy(e.lb);
    if (e.ld) hipblasLtMatrixLayoutDestroy(e.ld);
  }
  if (c->handle) hipblasLtDestroy(c->handle);
  delete c;
}

// Finds (or reuses) descriptors and an algorithm for this shape.  Returns nullptr when
// hipBLASLt has none; nothing is enqueued.
static GemmEntry* gemm_entry(GemmCache* c, long long T, int K, int N, bool bias) {
  for (GemmEntry& e : c->entries)
    if (e.T == T && e.K == K && e.N == N && e.bias == bias) return &e;
  GemmEntry e;
  e.T = T; e.K = K; e.N = N; e.bias = bias;
  bool ok = hipblasLtMatmulDescCreate(&e.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
  const hipblasOperation_t op = HIPBLAS_OP_N;
  if (ok) ok = hipblasLtMatmulDescSetAttribute(e.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &op, sizeof(op)) == HIPBLAS_STATUS_SUCCESS;
  if (ok) ok = hipblasLtMatmulDescSetAttribute(e.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &op, sizeof(op)) == HIPBLAS_STATUS_SUCCESS;
  if (ok && bias) {
    const hipblasLtEpilogue_t epi = HIPBLASLT_EPILOGUE_BIAS;
    const int32_t bt = HIP_R_16BF;
    ok = hipblasLtMatmulDescSetAttribute(e.desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi)) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(e.desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bt, sizeof(bt)) == HIPBLAS_STATUS_SUCCESS;
  }
  if (ok) ok = hipblasLtMatrixLayoutCreate(&e.la, HIP_R_16BF, N, K, N) == HIPBLAS_STATUS_SUCCESS;
  if (ok) ok = hipblasLtMatrixLayoutCreate(&e.lb, HIP_R_16BF, K, T, K) == HIPBLAS_STATUS_SUCCESS;
  if (ok) ok = hipblasLtMatrixLayoutCreate(&e.ld, HIP_R_16BF, N, T, N) == HIPBLAS_STATUS_SUCCESS;
  if (ok) {
    hipblasLtMatmulPreference_t pref = nullptr;
    ok = hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
    const uint64_t ws = kGemmWorkspaceBytes;
    if (ok) ok = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws, sizeof(ws)) == HIPBLAS_STATUS_SUCCESS;
    hipblasLtMatmulHeuristicResult_t res[kMaxCandidates]{};
    int found = 0;
    if (ok)
      ok = hipblasLtMatmulAlgoGetHeuristic(c->handle, e.desc, e.la, e.lb, e.ld, e.ld, pref,
                                           kMaxCandidates, res, &found) == HIPBLAS_STATUS_SUCCESS;
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    for (int i = 0; ok && i < found && i < kMaxCandidates; ++i)
      if (res[i].state == HIPBLAS_STATUS_SUCCESS) e.algo[e.candidates++] = res[i].algo;
    ok = ok && e.candidates > 0;
  }
  if (!ok) {
    if (e.desc) hipblasLtMatmulDescDestroy(e.desc);
    if (e.la) hipblasLtMatrixLayoutDestroy(e.la);
    if (e.lb) hipblasLtMatrixLayoutDestroy(e.lb);
    if (e.ld) hipblasLtMatrixLayoutDestroy(e.ld);
    return nullptr;
  }
  c->entries.push_back(e);
  return &c->entries.back();
}

bool gemm_prepare(GemmCache* c, long long T, int K, int N, bool bias) {
  return c && gemm_entry(c, T, K, N, bias) != nullptr;
}

static hipblasStatus_t matmul(GemmCache* c, GemmEntry* e, int i, const void* X, const void* W,
                              void* D, void* ws, hipStream_t s) {
  const float alpha = 1.f, beta = 0.f;
  return hipblasLtMatmul(c->handle, e->desc, &alpha, W, e->la, X, e->lb, &beta, D, e->ld, D,
                         e->ld, &e->algo[i], ws, kGemmWorkspaceBytes, s);
}

// The first call of a shape times each candidate algorithm on the caller's own operands
// (four runs after one warm-up, on the caller's stream, which this synchronizes), in two
// passes over the candidates so that clock ramp-up during the first pass does not decide
// the pick, and keeps the candidate with the lowest time of either pass; later calls of the
// shape use it directly.
static void pick_fastest(GemmCache* c, GemmEntry* e, const void* X, const void* W, void* D,
                         void* ws, hipStream_t s) {
  e->timed = true;
  if (e->candidates < 2) return;
  hipEvent_t t0 = nullptr, t1 = nullptr;
  if (hipEventCreate(&t0) != hipSuccess || hipEventCreate(&t1) != hipSuccess) {
    if (t0) (void)hipEventDestroy(t0);
    (void)hipGetLastError();
    return;
  }
  float best = 1e30f;
  for (int pass = 0; pass < 2; ++pass) {
    for (int i = 0; i < e->candidates; ++i) {
      if (matmul(c, e, i, X, W, D, ws, s) != HIPBLAS_STATUS_SUCCESS) continue;
      bool ok = hipEventRecord(t0, s) == hipSuccess;
      for (int r = 0; ok && r < 4; ++r) ok = matmul(c, e, i, X, W, D, ws, s) == HIPBLAS_STATUS_SUCCESS;
      ok = ok && hipEventRecord(t1, s) == hipSuccess && hipEventSynchronize(t1) == hipSuccess;
      float ms = 0.f;
      if (ok && hipEventElapsedTime(&ms, t0, t1) == hipSuccess && ms < best) {
        best = ms;
        e->best = i;
      }
    }
  }
  (void)hipEventDestroy(t0);
  (void)hipEventDestroy(t1);
  (void)hipGetLastError();
}

hipError_t gemm_run(GemmCache* c, const void* X, const void* W, const void* bias, void* D,
                    long long T, int K, int N, void* ws, hipStream_t s) {
  GemmEntry* e = c ? gemm_entry(c, T, K, N, bias != nullptr) : nullptr;
  if (!e) return hipErrorInvalidValue;
  if (bias &&
      hipblasLtMatmulDescSetAttribute(e->desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias,
                                      sizeof(bias)) != HIPBLAS_STATUS_SUCCESS)
    return hipErrorInvalidValue;
  if (!e->timed) pick_fastest(c, e, X, W, D, ws, s);
  return matmul(c, e, e->best, X, W, D, ws, s) == HIPBLAS_STATUS_SUCCESS ? hipSuccess
                                                                           : hipErrorLaunchFailure;
}

}  // namespace aa
