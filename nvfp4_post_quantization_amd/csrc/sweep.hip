// Hessian-weighted E4M3 block-scale sweep (fp8_scale_sweep, "Coder390 NVFP4
// 校正（校准）方式" §2 step 3): the launcher of nvfp4_scale_sweep and
// nvfp4_scale_sweep_ex.  The search itself, its exact pruning and its
// mapping on gfx950 are in sweep_kernel.hpp; this unit instantiates the plain
// kernel only.
#include <mutex>

#include "sweep_kernel.hpp"

namespace nvfp4 {

// The capped launch reserves, per workgroup, half the CU's LDS plus 1 KiB
// less what the kernel declares, so that at most one sweep workgroup fits on
// a CU; the rest of the CU (just under half its LDS, and about 260 of 512
// VGPRs per SIMD beside the sweep's one wave) stays free for a kernel on
// another stream.  The size is found and the kernel's limit raised once per
// device, at that device's first capped launch (0 = not done yet).
static std::mutex g_lds_mu;
static int g_lds_want[64] = {};

static int one_per_cu_lds(unsigned* dyn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) { set_hip_error(e, "hipGetDevice"); return NVFP4_ERR_HIP; }
  if (dev < 0 || dev >= 64) return NVFP4_ERR_BAD_INPUT;
  std::lock_guard<std::mutex> lock(g_lds_mu);
  if (g_lds_want[dev] == 0) {
    int lds_cu = 0;
    hipFuncAttributes fa;
    e = hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e == hipSuccess) e = hipFuncGetAttributes(&fa, (const void*)sweep_kernel<false>);
    if (e == hipSuccess) {
      const int want = lds_cu / 2 + 1024 - (int)fa.sharedSizeBytes;
      e = hipFuncSetAttribute((const void*)sweep_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize, want);
      if (e == hipSuccess) g_lds_want[dev] = want;
    }
    if (e != hipSuccess) { set_hip_error(e, "sweep LDS reservation"); return NVFP4_ERR_HIP; }
  }
  *dyn = (unsigned)g_lds_want[dev];
  return NVFP4_OK;
}

int launch_scale_sweep(const uint16_t* w, int64_t rows, int64_t k, int64_t ldw, const float* H,
                       const float* scale2, uint8_t* packed, uint8_t* codes, float* cost, int wgs_per_cu,
                       hipStream_t s) {
  int64_t rpw = 0;
  const dim3 grid = sweep_grid(rows, k, &rpw);
  unsigned dyn = 0;
  if (wgs_per_cu == 1) {
    const int st = one_per_cu_lds(&dyn);
    if (st) return st;
  }
  sweep_kernel<false><<<grid, kThreads, dyn, s>>>(w, rows, k, ldw, H, scale2, rpw, packed, codes, cost,
                                                  force_exact_flag());
  return launch_status("sweep_kernel");
}

}  // namespace nvfp4
