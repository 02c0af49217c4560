// Fake-quant QuantLinear forward ("NVFP4 量化流程说明" §2.2, §2.4): during
// calibration every Linear runs x -> input quantizer (NVFP4 block fake QDQ)
// -> matmul with the fake-quantized weight, still a floating-point bf16 GEMM:
//
//   y[t][o] = RN_bf16( sum_k xh[t][k] * wh[o][k] ),  fp32 accumulation,
//   xh = fake QDQ of x at its tensor scale (the fused quantize + two-DQ kernel),
//   wh = the swept weight after the two-DQ chain (static per layer: the caller
//        dequantizes it once with nvfp4_dequant).
//
// The fake QDQ is a separate HBM pass into the workspace: fused into the GEMM
// it would be recomputed for every output tile (out_features / tile times).
// The product is a plain bf16 GEMM, so it goes to hipBLASLt (TN layout:
// y^T [O, T] = wh [O, K] * xh^T [K, T] in column-major terms), fp32 compute.
// The first call for a shape on a device takes up to kTuneAlgos of
// hipBLASLt's heuristic candidates, times each on the caller's stream (so
// that call synchronises it) and keeps the fastest; a stream under graph
// capture takes the first candidate untimed instead.
#include <map>
#include <mutex>
#include <tuple>

#include <hipblaslt/hipblaslt.h>

#include "common.hpp"

namespace nvfp4 {

namespace {

constexpr size_t kGemmWorkspace = 32u << 20;       // hipBLASLt workspace, carved from the caller's buffer
constexpr size_t kAlign = 256;
constexpr int kTuneAlgos = 16;                       // heuristic candidates timed at the first call of a shape
constexpr int kTuneReps = 2;                         // timed runs per candidate (after one warm run)
constexpr int kTuneFinal = 4;                        // best candidates timed again before the pick

size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

struct Gemm {
  hipblasLtHandle_t handle = nullptr;
  std::map<std::tuple<int64_t, int64_t, int64_t, int64_t, int64_t, int64_t>, hipblasLtMatmulAlgo_t> algos;
};

std::mutex g_mu;
Gemm g_gemm[64];                                     // per device; handles live until the process ends

int blas_status(hipblasStatus_t st, const char* where) {
  if (st == HIPBLAS_STATUS_SUCCESS) return NVFP4_OK;
  set_error_text("hipBLASLt error %d in %s", (int)st, where);
  return NVFP4_ERR_HIP;
}

struct Layouts {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
  ~Layouts() {
    if (c) hipblasLtMatrixLayoutDestroy(c);
    if (b) hipblasLtMatrixLayoutDestroy(b);
    if (a) hipblasLtMatrixLayoutDestroy(a);
    if (desc) hipblasLtMatmulDescDestroy(desc);
  }
};

// Time each candidate: one warm run, then kTuneReps runs, each between its
// own pair of events, scored by its fastest run; then the kTuneFinal best
// are timed again in interleaved rounds (a candidate that drew a disturbed
// first measurement still competes on its best), and the index of the
// fastest is returned.  Candidates that fail to run are skipped.  Writes y
// (with correct results) along the way.
int tune(hipblasLtHandle_t handle, const Layouts& L, const hipblasLtMatmulHeuristicResult_t* heur, int n,
         const void* w, const void* xh, void* y, void* ws, hipStream_t s, int* pick) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t he = hipEventCreate(&e0);
  if (he == hipSuccess) he = hipEventCreate(&e1);
  if (he != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    set_hip_error(he, "hipEventCreate");
    return NVFP4_ERR_HIP;
  }
  const float alpha = 1.0f, beta = 0.0f;
  float score[kTuneAlgos];
  bool usable[kTuneAlgos];
  int st = NVFP4_OK;
  auto run = [&](int i) {
    return hipblasLtMatmul(handle, L.desc, &alpha, w, L.a, xh, L.b, &beta, y, L.c, y, L.c, &heur[i].algo, ws,
                           kGemmWorkspace, s) == HIPBLAS_STATUS_SUCCESS;
  };
  // one timed run of candidate i; false if it did not run (st set on a HIP error)
  auto time_one = [&](int i) {
    bool ok = hipEventRecord(e0, s) == hipSuccess && run(i);
    he = hipEventRecord(e1, s);
    if (he == hipSuccess) he = hipEventSynchronize(e1);
    if (he != hipSuccess) {
      set_hip_error(he, "tuning the GEMM");
      st = NVFP4_ERR_HIP;
      return false;
    }
    float ms = 0.0f;
    ok = ok && hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
    if (ok && ms < score[i]) score[i] = ms;
    return ok;
  };
  for (int i = 0; i < n; ++i) {
    score[i] = __builtin_inff();
    usable[i] = heur[i].state == HIPBLAS_STATUS_SUCCESS && heur[i].workspaceSize <= kGemmWorkspace;
  }
  for (int i = 0; i < n && st == NVFP4_OK; ++i) {
    if (!usable[i] || !run(i)) { usable[i] = false; continue; }
    for (int r = 0; r < kTuneReps && usable[i] && st == NVFP4_OK; ++r) usable[i] = time_one(i);
  }
  // the kTuneFinal best so far, timed again round-robin
  int top[kTuneFinal];
  int ntop = 0;
  for (int k = 0; k < kTuneFinal; ++k) {
    int b = -1;
    for (int i = 0; i < n; ++i) {
      bool taken = false;
      for (int j = 0; j < ntop; ++j) taken = taken || top[j] == i;
      if (usable[i] && !taken && score[i] < __builtin_inff() && (b < 0 || score[i] < score[b])) b = i;
    }
    if (b >= 0) top[ntop++] = b;
  }
  for (int r = 0; r < kTuneReps && st == NVFP4_OK; ++r)
    for (int j = 0; j < ntop && st == NVFP4_OK; ++j) (void)time_one(top[j]);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st) return st;
  int found = -1;
  for (int i = 0; i < n; ++i)
    if (usable[i] && score[i] < __builtin_inff() && (found < 0 || score[i] < score[found])) found = i;
  *pick = found < 0 ? 0 : found;
  return NVFP4_OK;
}

}  // namespace

size_t quantlinear_workspace_bytes(int64_t tokens, int64_t k) {
  return align_up((size_t)tokens * (size_t)k * 2u) + kGemmWorkspace;
}

int launch_quantlinear(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx, const float* x_scale2,
                       const uint16_t* w, int64_t out_features, int64_t ldw, uint16_t* y, int64_t ldy,
                       void* workspace, hipStream_t s) {
  uint16_t* xh = static_cast<uint16_t*>(workspace);
  void* gemm_ws = static_cast<char*>(workspace) + align_up((size_t)tokens * (size_t)k * 2u);
  int st = launch_fakequant(x, tokens, k, ldx, x_scale2, xh, k, s);
  if (st) return st;

  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) { set_hip_error(he, "hipGetDevice"); return NVFP4_ERR_HIP; }
  if (dev < 0 || dev >= 64) return NVFP4_ERR_BAD_INPUT;

  Layouts L;
  const int64_t O = out_features, T = tokens;
  if ((st = blas_status(hipblasLtMatmulDescCreate(&L.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F), "MatmulDescCreate")))
    return st;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  if ((st = blas_status(hipblasLtMatmulDescSetAttribute(L.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof ta),
                        "set TRANSA")) ||
      (st = blas_status(hipblasLtMatmulDescSetAttribute(L.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof tb),
                        "set TRANSB")))
    return st;
  // A = wh stored column-major [K, O] (ld ldw), op T; B = xh column-major [K, T] (ld k); C = D = y^T [O, T] (ld ldy)
  if ((st = blas_status(hipblasLtMatrixLayoutCreate(&L.a, HIP_R_16BF, k, O, ldw), "layout A")) ||
      (st = blas_status(hipblasLtMatrixLayoutCreate(&L.b, HIP_R_16BF, k, T, k), "layout B")) ||
      (st = blas_status(hipblasLtMatrixLayoutCreate(&L.c, HIP_R_16BF, O, T, ldy), "layout C")))
    return st;

  hipblasLtMatmulAlgo_t algo;
  hipblasLtHandle_t handle;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    Gemm& G = g_gemm[dev];
    if (!G.handle && (st = blas_status(hipblasLtCreate(&G.handle), "hipblasLtCreate"))) return st;
    handle = G.handle;
    const auto key = std::make_tuple(O, T, k, ldw, ldy, (int64_t)0);
    auto it = G.algos.find(key);
    if (it == G.algos.end()) {
      hipblasLtMatmulPreference_t pref = nullptr;
      if ((st = blas_status(hipblasLtMatmulPreferenceCreate(&pref), "PreferenceCreate"))) return st;
      const uint64_t wsb = kGemmWorkspace;
      hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof wsb);
      hipblasLtMatmulHeuristicResult_t heur[kTuneAlgos];
      int n = 0;
      hipblasStatus_t hs =
          hipblasLtMatmulAlgoGetHeuristic(handle, L.desc, L.a, L.b, L.c, L.c, pref, kTuneAlgos, heur, &n);
      hipblasLtMatmulPreferenceDestroy(pref);
      if ((st = blas_status(hs, "AlgoGetHeuristic"))) return st;
      if (n < 1) { set_error_text("hipBLASLt: no algorithm for this GEMM"); return NVFP4_ERR_HIP; }
      int pick = 0;
      hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
      if (n > 1 && hipStreamIsCapturing(s, &cap) == hipSuccess && cap == hipStreamCaptureStatusNone) {
        if ((st = tune(handle, L, heur, n, w, xh, y, gemm_ws, s, &pick))) return st;
      }
      it = G.algos.emplace(key, heur[pick].algo).first;
    }
    algo = it->second;
  }
  const float alpha = 1.0f, beta = 0.0f;
  return blas_status(hipblasLtMatmul(handle, L.desc, &alpha, w, L.a, xh, L.b, &beta, y, L.c, y, L.c, &algo, gemm_ws,
                                     kGemmWorkspace, s),
                     "hipblasLtMatmul");
}

}  // namespace nvfp4
