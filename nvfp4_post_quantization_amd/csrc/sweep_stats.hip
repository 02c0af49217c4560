// Measurement support: the counting build of the block-scale sweep
// (nvfp4_scale_sweep_stats).  Same search as nvfp4_scale_sweep, from the same
// device code (sweep_kernel.hpp), instantiated in this unit of its own so
// that the plain kernel's compilation is unchanged; uncapped launch.
#include "sweep_kernel.hpp"

namespace nvfp4 {

int launch_scale_sweep_stats(const uint16_t* w, int64_t rows, int64_t k, int64_t ldw, const float* H,
                             const float* scale2, uint8_t* packed, uint8_t* codes, uint64_t* stats,
                             hipStream_t s) {
  int64_t rpw = 0;
  const dim3 grid = sweep_grid(rows, k, &rpw);
  sweep_kernel<true><<<grid, kThreads, 0, s>>>(w, rows, k, ldw, H, scale2, rpw, packed, codes,
                                               reinterpret_cast<float*>(stats), force_exact_flag());
  return launch_status("sweep_kernel<stats>");
}

}  // namespace nvfp4
