// Closed-form MXFP4 -> NVFP4 cast ("从MXFP4到NVFP4：Model Optimizer混合精度格式
// 转换完全攻略" §2-§3; nibbles move unchanged and scale bytes double per the
// DeepSeek-V4 NVFP4 pipeline article's export stage).
//
// Per group (matrices sharing one scale_2, e.g. an expert's w1/w3):
//   k_max = max_j (e8m0_j - 127), scale_2 = 2^(k_max - 8);
//   MX block j with delta = k_max - k_j <= 17: both 16-element halves get the
//     E4M3 code of 2^(8 - delta) (exact), nibbles untouched;
//   otherwise the half is requantized from its data: its block amax over
//     6*scale_2 is at most 2^-10, which rounds to code 0x00 and is raised to
//     0x01 for a nonzero half, so d = 2^(k_max - 17) and each nibble becomes
//     RNE(e2m1 * 2^(17 - delta)) with its sign (an exact power-of-two rescale,
//     so the FP4 convert is exact); an all-zero half keeps code 0x00.
// E8M0 255 (NaN) is left out of k_max and gives E4M3 NaN codes.
//
// Three launches: per-group max of the E8M0 bytes (atomicMax into scale2_out,
// used as int scratch), the code/fallback pass, and scale_2.
#include "common.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kThreads = 256;

__global__ void cast_init_kernel(int32_t* kmax, int64_t* fallback, int64_t groups) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < groups) {
    kmax[i] = -1;
    if (fallback) fallback[i] = 0;
  }
}

// Largest E8M0 code != 255 in [lo, hi) of the flat byte array.
__global__ __launch_bounds__(kThreads) void cast_kmax_kernel(const uint8_t* __restrict__ e8m0, int64_t per_group,
                                                             int64_t chunk, int32_t* kmax) {
  const int64_t g = blockIdx.y;
  const int64_t lo = g * per_group + (int64_t)blockIdx.x * chunk;
  int64_t hi = lo + chunk;
  if (hi > (g + 1) * per_group) hi = (g + 1) * per_group;
  uint32_t m = 0;
  bool any = false;
  // 16-byte chunks fully inside [lo, hi), then the ragged edges byte by byte
  const int64_t a0 = (lo + 15) & ~(int64_t)15;
  const int64_t a1 = hi & ~(int64_t)15;
  for (int64_t p = a0 + 16 * (int64_t)threadIdx.x; p < a1; p += 16 * kThreads) {
    const uint4 v = *reinterpret_cast<const uint4*>(e8m0 + p);
    const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
    uint32_t mm = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mm = max(mm, max(max(wds[i] & 0xFFu, (wds[i] >> 8) & 0xFFu), max((wds[i] >> 16) & 0xFFu, wds[i] >> 24)));
    }
    if (mm == 0xFFu) {                       // a NaN exponent: redo without it
      mm = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint32_t b = (wds[i >> 2] >> (8 * (i & 3))) & 0xFFu;
        if (b != 0xFFu) { mm = max(mm, b); any = true; }
      }
    } else {
      any = true;
    }
    m = max(m, mm);
  }
  for (int64_t p = lo + threadIdx.x; p < hi; p += kThreads) {
    if ((p >= a0 && p < a1)) continue;
    uint32_t b = e8m0[p];
    if (b != 0xFFu) { m = max(m, b); any = true; }
  }
  // workgroup max; only workgroups that saw a valid code publish
  __shared__ int32_t part[kThreads / 64];
  int32_t v = any ? (int32_t)m : -1;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t r = -1;
    for (int i = 0; i < kThreads / 64; ++i) r = max(r, part[i]);
    if (r >= 0) atomicMax(&kmax[g], r);
  }
}

// E4M3 code of 2^e for e in [-9, 8].
__device__ __forceinline__ uint32_t pow2_code(int e) {
  return e >= -6 ? (uint32_t)((e + 7) << 3) : (uint32_t)(1 << (e + 9));
}

// Requantize one fallback MX block (16 bytes of nibbles) in place; returns
// the two E4M3 codes (low byte = first half).
__device__ __forceinline__ uint32_t fallback_block(uint8_t* nib16, int delta) {
  uint4 v = *reinterpret_cast<const uint4*>(nib16);
  uint32_t wds[4] = {v.x, v.y, v.z, v.w};
  uint32_t codes = 0;
  const int sh = 17 - delta;                          // <= -1
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t mag = (wds[2 * h] | wds[2 * h + 1]) & 0x77777777u;
    if (mag == 0u) continue;                          // all-zero half: code 0, nibbles kept
    codes |= 1u << (8 * h);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t wsrc = wds[2 * h + i];
      float a0, b0, a1, b1, a2, b2, a3, b3;
      fp4x2_to_f32<0>(wsrc, a0, b0);
      fp4x2_to_f32<1>(wsrc, a1, b1);
      fp4x2_to_f32<2>(wsrc, a2, b2);
      fp4x2_to_f32<3>(wsrc, a3, b3);
      uint32_t o = 0;
      o = cvt_fp4x2<0>(o, ldexpf(a0, sh), ldexpf(b0, sh));
      o = cvt_fp4x2<1>(o, ldexpf(a1, sh), ldexpf(b1, sh));
      o = cvt_fp4x2<2>(o, ldexpf(a2, sh), ldexpf(b2, sh));
      o = cvt_fp4x2<3>(o, ldexpf(a3, sh), ldexpf(b3, sh));
      wds[2 * h + i] = o;
    }
  }
  if (codes) *reinterpret_cast<uint4*>(nib16) = make_uint4(wds[0], wds[1], wds[2], wds[3]);
  return codes;
}

// Codes for one MX block with E8M0 byte b; may rewrite its nibbles.
__device__ __forceinline__ uint32_t mx_block_codes(uint32_t b, int32_t kmax_code, uint8_t* nib16, int& nfb) {
  if (b == 0xFFu) return 0x7F7Fu;
  const int delta = kmax_code - (int)b;
  if (delta <= 17) {
    const uint32_t c = pow2_code(8 - delta);
    return c | (c << 8);
  }
  ++nfb;
  return fallback_block(nib16, delta);
}

// One thread: 4 consecutive MX blocks of a group (vector path) or 1 (generic).
__global__ __launch_bounds__(kThreads) void cast_codes_kernel(uint8_t* __restrict__ packed,
                                                              const uint8_t* __restrict__ e8m0,
                                                              int64_t per_group, const int32_t* __restrict__ kmax,
                                                              uint8_t* __restrict__ codes,
                                                              unsigned long long* fallback, int vec4) {
  const int64_t g = blockIdx.y;
  int32_t km = kmax[g];
  if (km < 0) km = 127;                                 // no valid exponent at all
  const int64_t base = g * per_group;
  int nfb = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  if (vec4) {
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; 4 * u < per_group; u += stride) {
      const int64_t j = base + 4 * u;
      const uint32_t bytes = *reinterpret_cast<const uint32_t*>(e8m0 + j);
      uint32_t c[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = mx_block_codes((bytes >> (8 * i)) & 0xFFu, km, packed + (j + i) * 16, nfb);
      *reinterpret_cast<uint2*>(codes + 2 * j) = make_uint2(c[0] | (c[1] << 16), c[2] | (c[3] << 16));
    }
  } else {
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < per_group; u += stride) {
      const int64_t j = base + u;
      const uint32_t c = mx_block_codes(e8m0[j], km, packed + j * 16, nfb);
      codes[2 * j] = (uint8_t)(c & 0xFFu);
      codes[2 * j + 1] = (uint8_t)(c >> 8);
    }
  }
  if (fallback) {
    __shared__ int part[kThreads / 64];
    int v = nfb;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
      int r = 0;
      for (int i = 0; i < kThreads / 64; ++i) r += part[i];
      if (r) atomicAdd(&fallback[g], (unsigned long long)r);
    }
  }
}

__global__ void cast_scale_kernel(float* scale2, int64_t groups) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < groups) {
    int32_t km = reinterpret_cast<const int32_t*>(scale2)[i];
    if (km < 0) km = 127;
    scale2[i] = ldexpf(1.0f, km - 127 - 8);
  }
}

}  // namespace

int launch_mx_cast(uint8_t* packed, const uint8_t* e8m0, int64_t groups, int64_t mats, int64_t rows, int64_t k,
                   uint8_t* codes, float* scale2, int64_t* fallback, hipStream_t s) {
  int32_t* kmax = reinterpret_cast<int32_t*>(scale2);
  const unsigned gi = (unsigned)((groups + 255) / 256);
  cast_init_kernel<<<gi, 256, 0, s>>>(kmax, fallback, groups);
  int st = launch_status("cast_init_kernel");
  if (st) return st;
  const int64_t per_group = mats * rows * (k / 32);   // MX blocks (= E8M0 bytes) per group
  if (per_group > 0) {
    const int vec4 = (per_group % 4) == 0;
    const int64_t units = vec4 ? per_group / 4 : per_group;
    const int64_t chunk = 16384;                      // phase 1: ~16 KiB of exponents per workgroup
    const int64_t nx = (per_group + chunk - 1) / chunk;
    // grid.y is limited to 65535: run the groups in batches
    for (int64_t g0 = 0; g0 < groups; g0 += 65535) {
      const int64_t ng = (groups - g0 < 65535) ? groups - g0 : 65535;
      cast_kmax_kernel<<<dim3((unsigned)nx, (unsigned)ng, 1), kThreads, 0, s>>>(e8m0 + g0 * per_group, per_group,
                                                                                chunk, kmax + g0);
      if ((st = launch_status("cast_kmax_kernel"))) return st;
      int64_t wx = (units + kThreads - 1) / kThreads;
      int64_t cap = (kStreamGrid + ng - 1) / ng;
      if (wx > cap * 4) wx = cap * 4;
      if (wx < 1) wx = 1;
      cast_codes_kernel<<<dim3((unsigned)wx, (unsigned)ng, 1), kThreads, 0, s>>>(
          packed + g0 * per_group * 16, e8m0 + g0 * per_group, per_group, kmax + g0, codes + g0 * per_group * 2,
          fallback ? reinterpret_cast<unsigned long long*>(fallback + g0) : nullptr, vec4);
      if ((st = launch_status("cast_codes_kernel"))) return st;
    }
  }
  cast_scale_kernel<<<gi, 256, 0, s>>>(scale2, groups);
  return launch_status("cast_scale_kernel");
}

}  // namespace nvfp4
