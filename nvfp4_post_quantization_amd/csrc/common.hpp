// Host-side helpers shared by the launchers: status codes, HIP error capture.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/nvfp4mi.h"

namespace nvfp4 {

// Remembers the text of the last failing HIP call on this thread.
void set_hip_error(hipError_t e, const char* where);

inline int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return NVFP4_OK;
  set_hip_error(e, where);
  return NVFP4_ERR_HIP;
}

inline int launch_status(const char* where) { return hip_status(hipGetLastError(), where); }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Test hook read from the environment: NVFP4MI_FORCE_EXACT=1 disables the
// certified FP4-convert fast paths (exact thresholds everywhere); =2 skips the
// one-float reciprocal (level 0); =3 skips level 0 and the uncorrected
// two-float quotient (level 1), leaving the corrected one where certified.
int force_exact_flag();


// Launchers (one per kernel family); arguments are validated by the caller.
int launch_compute_scale2(const uint16_t* x, int64_t n, float* scale2_out, float* amax_out, hipStream_t s);
constexpr int kScaleBatch = 16;          // tensors per nvfp4_compute_scale2_batch call
int launch_compute_scale2_batch(const uint16_t* const* xs, const int64_t* ns, int count, float* scale2_out,
                                float* amax_out, hipStream_t s);
int launch_quantize_dynamic(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, const float* scale2,
                            uint8_t* packed, uint8_t* codes, hipStream_t s);
int launch_dequant(const uint8_t* packed, const uint8_t* codes, const float* scale2, int64_t rows, int64_t k,
                   uint16_t* out, hipStream_t s);
size_t hessian_workspace_bytes(int64_t tokens, int64_t k);
// partial slots of the plain accumulate alone, and the static buffer that
// holds them for nvfp4_hessian_accum_noalloc
size_t hessian_plain_workspace_bytes(int64_t tokens, int64_t k);
constexpr size_t kHessianScratchBytes = size_t(16) << 20;
int launch_hessian_accum_noalloc(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx, float* H, float* amax,
                                 hipStream_t s);
int launch_hessian_accum(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx, float* H, float* amax,
                         void* workspace, hipStream_t s);
constexpr int kMaxChunks = 64;           // chunks per nvfp4_hessian_accum_chunks call
int launch_hessian_accum_chunks(const uint16_t* const* xs, int nchunks, int64_t tokens, int64_t k, int64_t ldx,
                                float* H, float* amax, void* workspace, hipStream_t s);
size_t hessian_chunks_workspace_bytes(int64_t tokens, int64_t k, int nchunks);
int launch_hessian_accum_fq_chunks(const uint16_t* const* xs, int nchunks, int64_t tokens, int64_t k, int64_t ldx,
                                   const float* scale2, float* H, float* amax, void* workspace, hipStream_t s);
int launch_hessian_accum_fq(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx, const float* scale2, float* H,
                            float* amax, void* workspace, hipStream_t s);
int launch_fp8_scale(const uint16_t* x, int64_t n, float* scale_out, float* amax_out, hipStream_t s);
int launch_fp8_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, const float* scale, uint8_t* q,
                        hipStream_t s);
int launch_fp8_dequant(const uint8_t* q, const float* scale, int64_t rows, int64_t k, uint16_t* out, hipStream_t s);
int launch_block_hadamard(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, uint16_t* out, int64_t ldo,
                          hipStream_t s);
int launch_hessian_hadamard(const float* H, int64_t groups, float* Hout, hipStream_t s);
int launch_fakequant(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, const float* scale2, uint16_t* out,
                     int64_t ldo, hipStream_t s);
size_t quantlinear_workspace_bytes(int64_t tokens, int64_t k);
int launch_quantlinear(const uint16_t* x, int64_t tokens, int64_t k, int64_t ldx, const float* x_scale2,
                       const uint16_t* w, int64_t out_features, int64_t ldw, uint16_t* y, int64_t ldy,
                       void* workspace, hipStream_t s);
// printf-style text for the next nvfp4_status_string(NVFP4_ERR_HIP) on this thread
void set_error_text(const char* fmt, ...);
int launch_scale_sweep(const uint16_t* w, int64_t rows, int64_t k, int64_t ldw, const float* H,
                       const float* scale2, uint8_t* packed, uint8_t* codes, float* cost, int wgs_per_cu,
                       hipStream_t s);
// the counting build (nvfp4_scale_sweep_stats), uncapped
int launch_scale_sweep_stats(const uint16_t* w, int64_t rows, int64_t k, int64_t ldw, const float* H,
                             const float* scale2, uint8_t* packed, uint8_t* codes, uint64_t* stats,
                             hipStream_t s);
// measurement support (include/nvfp4mi_probe.h)
int launch_probe_read(const void* buf, size_t bytes, void* sink, int wgs, hipStream_t s);
int launch_probe_write(void* buf, size_t bytes, uint32_t value, int wgs, hipStream_t s);
int launch_probe_copy(const void* src, void* dst, size_t bytes, int wgs, hipStream_t s);
int launch_mx_cast(uint8_t* packed, const uint8_t* e8m0, int64_t groups, int64_t mats, int64_t rows, int64_t k,
                   uint8_t* codes, float* scale2, int64_t* fallback, hipStream_t s);

}  // namespace nvfp4
