// C ABI entry points (include/nvfp4mi.h): argument validation on the host,
// then the launches.  No HIP call happens before validation succeeds, so
// every error code except NVFP4_ERR_HIP can be produced without a GPU.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "common.hpp"
#include "../../include/nvfp4mi_probe.h"

namespace nvfp4 {

static thread_local char g_hip_error[256] = "no HIP error recorded";

void set_hip_error(hipError_t e, const char* where) {
  snprintf(g_hip_error, sizeof g_hip_error, "HIP error in %s: %s (%d)", where, hipGetErrorString(e), (int)e);
}

void set_error_text(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_hip_error, sizeof g_hip_error, fmt, ap);
  va_end(ap);
}

int force_exact_flag() {
  const char* v = getenv("NVFP4MI_FORCE_EXACT");
  if (!v || !v[0] || v[0] == '0') return 0;
  return (v[0] == '2' || v[0] == '3') ? v[0] - '0' : 1;
}

// a * b <= INT64_MAX for non-negative a, b
static bool mul_fits(int64_t a, int64_t b) { return a == 0 || b <= INT64_MAX / a; }

// [rows][ld] matrix of `elem` bytes with `cols` used columns.
static int check_matrix(int64_t rows, int64_t cols, int64_t ld, int64_t elem) {
  if (rows < 0 || cols <= 0 || ld < cols) return NVFP4_ERR_BAD_SHAPE;
  if (!mul_fits(rows, ld) || !mul_fits(rows * ld, elem)) return NVFP4_ERR_BAD_SHAPE;
  return NVFP4_OK;
}

static int check_bf16_rows(const void* p, int64_t ld) {
  if (!aligned16(p) || (ld % 8) != 0) return NVFP4_ERR_MISALIGNED;
  return NVFP4_OK;
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL_ARG: return "a required pointer argument is NULL";
    case NVFP4_ERR_BAD_SHAPE: return "bad shape: negative size, k not a multiple of the block, ld < k, or size overflow";
    case NVFP4_ERR_MISALIGNED: return "misaligned buffer: a pointer or row stride breaks the function's alignment rule";
    case NVFP4_ERR_WORKSPACE: return "workspace smaller than the size the matching *_bytes query returns";
    case NVFP4_ERR_BAD_INPUT: return "argument value out of range";
    case NVFP4_ERR_HIP: return g_hip_error;
    case NVFP4_ERR_SCRATCH_LIMIT:
      return "input needs more scratch than the static buffer of the no-allocation entry point holds";
    default: return "unknown status";
  }
}

int nvfp4_compute_scale2(const uint16_t* x, int64_t n, float* scale2_out, float* amax_out, void* stream) {
  if (n < 0 || !mul_fits(n, 2)) return NVFP4_ERR_BAD_SHAPE;
  if (!scale2_out || (n > 0 && !x)) return NVFP4_ERR_NULL_ARG;
  if (n > 0 && !aligned16(x)) return NVFP4_ERR_MISALIGNED;
  if (!aligned4(scale2_out) || (amax_out && !aligned4(amax_out))) return NVFP4_ERR_MISALIGNED;   // atomic targets
  return launch_compute_scale2(x, n, scale2_out, amax_out, as_stream(stream));
}

int nvfp4_compute_scale2_batch(const uint16_t* const* xs, const int64_t* ns, int count, float* scale2_out,
                               float* amax_out, void* stream) {
  if (count < 1 || count > kScaleBatch) return NVFP4_ERR_BAD_SHAPE;
  if (!xs || !ns || !scale2_out) return NVFP4_ERR_NULL_ARG;
  for (int t = 0; t < count; ++t) {
    if (ns[t] < 0 || !mul_fits(ns[t], 2)) return NVFP4_ERR_BAD_SHAPE;
    if (ns[t] > 0 && !xs[t]) return NVFP4_ERR_NULL_ARG;
    if (ns[t] > 0 && !aligned16(xs[t])) return NVFP4_ERR_MISALIGNED;
  }
  if (!aligned4(scale2_out) || (amax_out && !aligned4(amax_out))) return NVFP4_ERR_MISALIGNED;
  return launch_compute_scale2_batch(xs, ns, count, scale2_out, amax_out, as_stream(stream));
}

size_t nvfp4_hessian_workspace_bytes(int64_t tokens, int64_t k) {
  if (tokens <= 0 || k <= 0 || (k % 16) != 0) return 0;
  return hessian_workspace_bytes(tokens, k);
}

// Shared validation of the two Hessian entry points.
static int check_hessian(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx, const float* H,
                         const float* amax, const void* workspace, size_t workspace_bytes) {
  int st = check_matrix(tokens, k, ldx, 2);
  if (st) return st;
  if (k % 16) return NVFP4_ERR_BAD_SHAPE;
  if (!H || (tokens > 0 && !x)) return NVFP4_ERR_NULL_ARG;
  if (tokens == 0) return NVFP4_OK;
  if ((st = check_bf16_rows(x, ldx))) return st;
  size_t need = hessian_workspace_bytes(tokens, k);
  if (workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
  if (need && !workspace) return NVFP4_ERR_NULL_ARG;
  if (!aligned16(H) || !aligned16(workspace)) return NVFP4_ERR_MISALIGNED;
  if (amax && !aligned4(amax)) return NVFP4_ERR_MISALIGNED;                                   // atomic target
  return NVFP4_OK;
}

int nvfp4_hessian_accum(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx, float* H, float* amax_inout,
                        void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_hessian(x, tokens, k, ldx, H, amax_inout, workspace, workspace_bytes);
  if (st || tokens == 0) return st;
  return launch_hessian_accum(x, tokens, k, ldx, H, amax_inout, workspace, as_stream(stream));
}

size_t nvfp4_hessian_chunks_workspace_bytes(int64_t tokens, int64_t k, int nchunks) {
  if (tokens <= 0 || k <= 0 || (k % 16) != 0 || nchunks < 1 || nchunks > kMaxChunks) return 0;
  if (!mul_fits(tokens, k) || !mul_fits(tokens * k, 2)) return 0;
  return hessian_chunks_workspace_bytes(tokens, k, nchunks);
}

// shared by both chunk-list calls; *empty is set when there is nothing to do
static int check_chunks(const uint16_t* const* xs, int nchunks, int64_t tokens, int64_t k, int64_t ldx,
                        const float* H, const float* amax, const void* workspace, size_t workspace_bytes,
                        bool* empty) {
  *empty = false;
  if (nchunks < 1 || nchunks > kMaxChunks) return NVFP4_ERR_BAD_SHAPE;
  int st = check_matrix(tokens, k, ldx, 2);
  if (st) return st;
  if (k % 16) return NVFP4_ERR_BAD_SHAPE;
  if (!xs || !H) return NVFP4_ERR_NULL_ARG;
  if (tokens == 0) {
    *empty = true;
    return NVFP4_OK;
  }
  for (int c = 0; c < nchunks; ++c) {
    if (!xs[c]) return NVFP4_ERR_NULL_ARG;
    if ((st = check_bf16_rows(xs[c], ldx))) return st;
  }
  const size_t need = hessian_chunks_workspace_bytes(tokens, k, nchunks);
  if (workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
  if (!workspace) return NVFP4_ERR_NULL_ARG;
  if (!aligned16(H) || !aligned16(workspace)) return NVFP4_ERR_MISALIGNED;
  if (amax && !aligned4(amax)) return NVFP4_ERR_MISALIGNED;                                   // atomic target
  return NVFP4_OK;
}

int nvfp4_hessian_accum_chunks(const uint16_t* const* xs, int nchunks, int64_t tokens, int64_t k, int64_t ldx,
                               float* H, float* amax_inout, void* workspace, size_t workspace_bytes,
                               void* stream) {
  bool empty = false;
  const int st = check_chunks(xs, nchunks, tokens, k, ldx, H, amax_inout, workspace, workspace_bytes, &empty);
  if (st || empty) return st;
  return launch_hessian_accum_chunks(xs, nchunks, tokens, k, ldx, H, amax_inout, workspace, as_stream(stream));
}

int nvfp4_hessian_accum_fq_chunks(const uint16_t* const* xs, int nchunks, int64_t tokens, int64_t k, int64_t ldx,
                                  const float* scale2, float* H, float* amax_inout, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  bool empty = false;
  const int st = check_chunks(xs, nchunks, tokens, k, ldx, H, amax_inout, workspace, workspace_bytes, &empty);
  if (st) return st;
  if (!scale2) return NVFP4_ERR_NULL_ARG;
  if (empty) return NVFP4_OK;
  return launch_hessian_accum_fq_chunks(xs, nchunks, tokens, k, ldx, scale2, H, amax_inout, workspace,
                                        as_stream(stream));
}

int nvfp4_hessian_accum_noalloc(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx, float* H,
                                float* amax_inout, void* stream) {
  int st = check_matrix(tokens, k, ldx, 2);
  if (st) return st;
  if (k % 16) return NVFP4_ERR_BAD_SHAPE;
  if (!H || (tokens > 0 && !x)) return NVFP4_ERR_NULL_ARG;
  if (tokens == 0) return NVFP4_OK;
  if ((st = check_bf16_rows(x, ldx))) return st;
  if (!aligned16(H) || (amax_inout && !aligned4(amax_inout))) return NVFP4_ERR_MISALIGNED;
  if (hessian_plain_workspace_bytes(tokens, k) > kHessianScratchBytes) return NVFP4_ERR_SCRATCH_LIMIT;
  return launch_hessian_accum_noalloc(x, tokens, k, ldx, H, amax_inout, as_stream(stream));
}

int nvfp4_hessian_accum_fq(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx, const float* scale2, float* H,
                           float* amax_inout, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_hessian(x, tokens, k, ldx, H, amax_inout, workspace, workspace_bytes);
  if (st) return st;
  if (!scale2) return NVFP4_ERR_NULL_ARG;
  if (tokens == 0) return NVFP4_OK;
  return launch_hessian_accum_fq(x, tokens, k, ldx, scale2, H, amax_inout, workspace, as_stream(stream));
}

static int scale_sweep(const uint16_t* w, int64_t rows, int64_t k, int64_t ldw, const float* H, const float* scale2,
                       uint8_t* packed, uint8_t* codes, float* cost, int wgs_per_cu, void* stream,
                       uint64_t* stats = nullptr) {
  int st = check_matrix(rows, k, ldw, 2);
  if (st) return st;
  if (k % 16) return NVFP4_ERR_BAD_SHAPE;
  if (wgs_per_cu < 0 || wgs_per_cu > 1) return NVFP4_ERR_BAD_INPUT;
  if (!H || !scale2 || ((!w || !packed || !codes) && rows > 0)) return NVFP4_ERR_NULL_ARG;
  if (rows == 0) return NVFP4_OK;
  if ((st = check_bf16_rows(w, ldw))) return st;
  if (!aligned8(packed) || !aligned4(cost) || !aligned8(stats)) return NVFP4_ERR_MISALIGNED;
  if (stats) return launch_scale_sweep_stats(w, rows, k, ldw, H, scale2, packed, codes, stats, as_stream(stream));
  return launch_scale_sweep(w, rows, k, ldw, H, scale2, packed, codes, cost, wgs_per_cu, as_stream(stream));
}

int nvfp4_scale_sweep(const uint16_t* w, int64_t rows, int64_t k, int64_t ldw, const float* H, const float* scale2,
                      uint8_t* packed, uint8_t* codes, float* cost, void* stream) {
  return scale_sweep(w, rows, k, ldw, H, scale2, packed, codes, cost, 0, stream);
}

int nvfp4_scale_sweep_ex(const uint16_t* w, int64_t rows, int64_t k, int64_t ldw, const float* H, const float* scale2,
                         uint8_t* packed, uint8_t* codes, float* cost, int wgs_per_cu, void* stream) {
  return scale_sweep(w, rows, k, ldw, H, scale2, packed, codes, cost, wgs_per_cu, stream);
}

int nvfp4_scale_sweep_stats(const uint16_t* w, int64_t rows, int64_t k, int64_t ldw, const float* H,
                            const float* scale2, uint8_t* packed, uint8_t* codes, uint64_t* stats, void* stream) {
  if (!stats) return NVFP4_ERR_NULL_ARG;
  return scale_sweep(w, rows, k, ldw, H, scale2, packed, codes, nullptr, 0, stream, stats);
}

static int check_probe(const void* p, size_t bytes, int wgs) {
  if (bytes % 16) return NVFP4_ERR_BAD_SHAPE;
  if (wgs < 0 || wgs > 65535) return NVFP4_ERR_BAD_INPUT;
  if (!p) return NVFP4_ERR_NULL_ARG;
  if (!aligned16(p)) return NVFP4_ERR_MISALIGNED;
  return NVFP4_OK;
}

int nvfp4_probe_read(const void* buf, size_t bytes, void* sink, int workgroups, void* stream) {
  int st = check_probe(buf, bytes, workgroups);
  if (st) return st;
  if (!sink) return NVFP4_ERR_NULL_ARG;
  if (!aligned4(sink)) return NVFP4_ERR_MISALIGNED;
  return bytes ? launch_probe_read(buf, bytes, sink, workgroups, as_stream(stream)) : NVFP4_OK;
}

int nvfp4_probe_write(void* buf, size_t bytes, uint32_t value, int workgroups, void* stream) {
  const int st = check_probe(buf, bytes, workgroups);
  if (st) return st;
  return bytes ? launch_probe_write(buf, bytes, value, workgroups, as_stream(stream)) : NVFP4_OK;
}

int nvfp4_probe_copy(const void* src, void* dst, size_t bytes, int workgroups, void* stream) {
  int st = check_probe(src, bytes, workgroups);
  if (st || (st = check_probe(dst, bytes, workgroups))) return st;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) return NVFP4_ERR_BAD_INPUT;       // overlap
  return bytes ? launch_probe_copy(src, dst, bytes, workgroups, as_stream(stream)) : NVFP4_OK;
}

int nvfp4_quantize_dynamic(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, const float* scale2,
                           uint8_t* packed, uint8_t* codes, void* stream) {
  int st = check_matrix(rows, k, ldx, 2);
  if (st) return st;
  if (k % 16) return NVFP4_ERR_BAD_SHAPE;
  if (!scale2 || ((!x || !packed || !codes) && rows > 0)) return NVFP4_ERR_NULL_ARG;
  if (rows == 0) return NVFP4_OK;
  if ((st = check_bf16_rows(x, ldx))) return st;
  if (!aligned16(packed)) return NVFP4_ERR_MISALIGNED;
  return launch_quantize_dynamic(x, rows, k, ldx, scale2, packed, codes, as_stream(stream));
}

int nvfp4_dequant(const uint8_t* packed, const uint8_t* codes, const float* scale2, int64_t rows, int64_t k,
                  uint16_t* out, void* stream) {
  int st = check_matrix(rows, k, k, 2);
  if (st) return st;
  if (k % 16) return NVFP4_ERR_BAD_SHAPE;
  if (!scale2 || ((!packed || !codes || !out) && rows > 0)) return NVFP4_ERR_NULL_ARG;
  if (rows == 0) return NVFP4_OK;
  if (!aligned16(packed) || !aligned16(out)) return NVFP4_ERR_MISALIGNED;
  return launch_dequant(packed, codes, scale2, rows, k, out, as_stream(stream));
}

int mxfp4_to_nvfp4_cast(uint8_t* packed, const uint8_t* e8m0, int64_t groups, int64_t mats_per_group,
                        int64_t rows, int64_t k, uint8_t* codes_out, float* scale2_out,
                        int64_t* fallback_blocks_out, void* stream) {
  if (groups < 0 || rows < 0 || k <= 0 || (k % 32) != 0) return NVFP4_ERR_BAD_SHAPE;
  if (mats_per_group <= 0) return NVFP4_ERR_BAD_INPUT;
  if (!mul_fits(groups, mats_per_group) || !mul_fits(groups * mats_per_group, rows) ||
      !mul_fits(groups * mats_per_group * rows, k))
    return NVFP4_ERR_BAD_SHAPE;
  if (groups == 0) return NVFP4_OK;
  if (!scale2_out) return NVFP4_ERR_NULL_ARG;
  if (rows > 0 && (!packed || !e8m0 || !codes_out)) return NVFP4_ERR_NULL_ARG;
  if (rows > 0 && (!aligned16(packed) || !aligned16(e8m0) || !aligned16(codes_out))) return NVFP4_ERR_MISALIGNED;
  if (!aligned4(scale2_out) || (fallback_blocks_out && !aligned8(fallback_blocks_out)))          // atomic targets
    return NVFP4_ERR_MISALIGNED;
  return launch_mx_cast(packed, e8m0, groups, mats_per_group, rows, k, codes_out, scale2_out,
                        fallback_blocks_out, as_stream(stream));
}

int fp8e4m3_compute_scale(const uint16_t* x, int64_t n, float* scale_out, float* amax_out, void* stream) {
  if (n < 0 || !mul_fits(n, 2)) return NVFP4_ERR_BAD_SHAPE;
  if (!scale_out || (n > 0 && !x)) return NVFP4_ERR_NULL_ARG;
  if (n > 0 && !aligned16(x)) return NVFP4_ERR_MISALIGNED;
  if (!aligned4(scale_out) || (amax_out && !aligned4(amax_out))) return NVFP4_ERR_MISALIGNED;    // atomic targets
  return launch_fp8_scale(x, n, scale_out, amax_out, as_stream(stream));
}

int fp8e4m3_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, const float* scale, uint8_t* q,
                     void* stream) {
  int st = check_matrix(rows, k, ldx, 2);
  if (st) return st;
  if (k % 8) return NVFP4_ERR_BAD_SHAPE;
  if (!scale || ((!x || !q) && rows > 0)) return NVFP4_ERR_NULL_ARG;
  if (rows == 0) return NVFP4_OK;
  if ((st = check_bf16_rows(x, ldx))) return st;
  if (reinterpret_cast<uintptr_t>(q) % 8) return NVFP4_ERR_MISALIGNED;
  return launch_fp8_quantize(x, rows, k, ldx, scale, q, as_stream(stream));
}

int fp8e4m3_dequant(const uint8_t* q, const float* scale, int64_t rows, int64_t k, uint16_t* out, void* stream) {
  int st = check_matrix(rows, k, k, 2);
  if (st) return st;
  if (k % 8) return NVFP4_ERR_BAD_SHAPE;
  if (!scale || ((!q || !out) && rows > 0)) return NVFP4_ERR_NULL_ARG;
  if (rows == 0) return NVFP4_OK;
  if (reinterpret_cast<uintptr_t>(q) % 8 || !aligned16(out)) return NVFP4_ERR_MISALIGNED;
  return launch_fp8_dequant(q, scale, rows, k, out, as_stream(stream));
}

int nvfp4_block_hadamard(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, uint16_t* out, int64_t ldo,
                         void* stream) {
  int st = check_matrix(rows, k, ldx, 2);
  if (st) return st;
  if ((st = check_matrix(rows, k, ldo, 2))) return st;
  if (k % 16) return NVFP4_ERR_BAD_SHAPE;
  if ((!x || !out) && rows > 0) return NVFP4_ERR_NULL_ARG;
  if (rows == 0) return NVFP4_OK;
  if ((st = check_bf16_rows(x, ldx)) || (st = check_bf16_rows(out, ldo))) return st;
  return launch_block_hadamard(x, rows, k, ldx, out, ldo, as_stream(stream));
}

int nvfp4_hessian_hadamard(const float* H, int64_t groups, float* H_out, void* stream) {
  if (groups < 0 || !mul_fits(groups, 1024)) return NVFP4_ERR_BAD_SHAPE;
  if (groups == 0) return NVFP4_OK;
  if (!H || !H_out) return NVFP4_ERR_NULL_ARG;
  if (!aligned4(H) || !aligned4(H_out)) return NVFP4_ERR_MISALIGNED;
  return launch_hessian_hadamard(H, groups, H_out, as_stream(stream));
}

int nvfp4_fakequant(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, const float* scale2, uint16_t* out,
                    int64_t ldo, void* stream) {
  int st = check_matrix(rows, k, ldx, 2);
  if (st) return st;
  if ((st = check_matrix(rows, k, ldo, 2))) return st;
  if (k % 16) return NVFP4_ERR_BAD_SHAPE;
  if (!scale2 || ((!x || !out) && rows > 0)) return NVFP4_ERR_NULL_ARG;
  if (rows == 0) return NVFP4_OK;
  if ((st = check_bf16_rows(x, ldx)) || (st = check_bf16_rows(out, ldo))) return st;
  return launch_fakequant(x, rows, k, ldx, scale2, out, ldo, as_stream(stream));
}

size_t nvfp4_quantlinear_workspace_bytes(int64_t tokens, int64_t k) {
  if (tokens < 0 || k <= 0 || (k % 16) != 0 || !mul_fits(tokens, k) || !mul_fits(tokens * k, 2)) return 0;
  return quantlinear_workspace_bytes(tokens, k);
}

int nvfp4_quantlinear_forward(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx, const float* x_scale2,
                              const uint16_t* w, int64_t out_features, int64_t ldw, uint16_t* y, int64_t ldy,
                              void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_matrix(tokens, k, ldx, 2);
  if (st) return st;
  if ((st = check_matrix(out_features, k, ldw, 2))) return st;
  if (out_features <= 0) return NVFP4_ERR_BAD_SHAPE;
  if ((st = check_matrix(tokens, out_features, ldy, 2))) return st;
  if (k % 16) return NVFP4_ERR_BAD_SHAPE;
  if (!x_scale2 || !w || ((!x || !y) && tokens > 0)) return NVFP4_ERR_NULL_ARG;
  if (tokens == 0) return NVFP4_OK;
  if ((st = check_bf16_rows(x, ldx)) || (st = check_bf16_rows(w, ldw)) || (st = check_bf16_rows(y, ldy))) return st;
  const size_t need = quantlinear_workspace_bytes(tokens, k);
  if (workspace_bytes < need) return NVFP4_ERR_WORKSPACE;
  if (!workspace) return NVFP4_ERR_NULL_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) % 256) return NVFP4_ERR_MISALIGNED;
  return launch_quantlinear(x, tokens, k, ldx, x_scale2, w, out_features, ldw, y, ldy, workspace,
                            as_stream(stream));
}

}  // extern "C"
